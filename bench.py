#!/usr/bin/env python3
"""Throughput of one MoE layer (route -> capacity dispatch -> expert FFN ->
combine, plus the ledger) on one MI355X, through the C ABI of libmoe.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--mode graph]

A step is one pass of the whole path over one batch of tokens: moe_route,
moe_dispatch (routing metadata), moe_expert_ffn_rows (the expert FFN, whose
first GEMM gathers each dispatched row x[row_token[r]] in its own loads),
then the combine and the ledger (its counting kernels, whose counters land
in a page-locked host stage) in one moe_combine_ledger call, all on one
stream.  --gather dispatch has moe_dispatch copy the rows into x_disp for
moe_expert_ffn_packed instead.  --ledger-stream main issues
moe_combine and moe_ledger_launch as two calls instead; side moves the
ledger to a second stream that starts after the dispatch and joins before
the step ends.  The host decodes every step's ledger (moe_ledger_finalize,
into buffers allocated once) a few steps behind the device, while later
steps run.  Inputs are resident in HBM.
So that the 256 MB last-level cache cannot serve the weights, successive steps
rotate over several copies of x and of all weights (>= 1 GiB in total).

Modes: "eager" (default) issues the pre-marshalled C calls every step;
"graph" captures each rotation's step once into a HIP graph and replays it
(measured slower than eager on this stack, so not the default).  Either
way a second, eager timed pass records HIP events around each call on the
stream it runs on; the expert-FFN interval (its two grouped-GEMM launches)
gives the roofline of the dominant kernel.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BASELINE_METRIC = ("routed tokens/s through route→dispatch→FFN→combine; "
                   "% of HBM/MFMA peak")
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2,
                   help="workload id (2 = the Switch-Base-shaped layer, the headline)")
    p.add_argument("--mode", choices=["graph", "eager"], default="eager")
    p.add_argument("--weights", choices=["packed", "rowmajor"], default="packed",
                   help="expert weights in the packed fragment layout (packed once at setup, "
                        "as a server does at load time) or row-major")
    p.add_argument("--rotate-bytes", type=float, default=float(1 << 30),
                   help="total bytes of rotated input copies (defeats the 256 MB cache)")
    p.add_argument("--ledger-stream", choices=["fused", "main", "side"], default="fused",
                   help="fused: combine and ledger in one moe_combine_ledger call; main: "
                        "moe_combine then moe_ledger_launch; side: the ledger on a second "
                        "stream beside the FFN")
    p.add_argument("--gather", choices=["ffn", "dispatch"], default="ffn",
                   help="ffn: the first GEMM's loads gather the dispatched rows "
                        "(moe_expert_ffn_rows); dispatch: moe_dispatch copies them into x_disp")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-next-rows", action="store_true",
                   help="skip the timings of the entry points beyond the layer step (bias "
                        "update, FP8 payload, routing scenarios), e.g. under a profiler")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="rough budget of the CPU-oracle baseline")
    return p.parse_args()


def algorithmic(wl, R, E_nz):
    """Bytes / flops the method must move / do (not padded rows, not dense T*E)."""
    T, h, E, K, F, b = wl.T, wl.h, wl.E, wl.K, wl.F, wl.bytes_per_elem
    return {
        "ffn_bytes": E_nz * 2 * h * F * b + R * h * b + 2 * R * F * b + R * h * 4,
        "ffn_flops": 4 * h * F * R,
        "route_bytes": T * h * b + E * h * b + T * E * 4 + T * K * 8,
        "route_flops": 2 * T * h * E,
        "dispatch_bytes": 2 * R * h * b + T * K * 4 * 4,
        "combine_bytes": R * h * 4 + T * h * 4 + T * K * 8,
    }


def next_rows(M, bufs, torch, stream, x, reps=200):
    """Per-call time (HIP events on `stream`, one pair per call, averaged; an
    upper bound that includes the launch) of the entry points beyond the
    layer step, on the step's own buffers: moe_bias_update (aux-loss-free
    balancing) and the FP8 payload (moe_fp8_scale, moe_dispatch_fp8,
    moe_fp8_dequantize), with the dispatch payload bytes of both formats."""
    cfg, b = bufs.cfg, bufs
    bias = torch.zeros((cfg.E,), dtype=torch.float32, device="cuda")
    calls = {"bias_update_us": lambda: M.moe_bias_update(cfg, b.topk_idx, bias, 1e-3, None,
                                                         stream)}
    out = {}
    if cfg.dtype == M.MOE_BF16:
        scale = torch.zeros((1,), dtype=torch.float32, device="cuda")
        xq = torch.empty((max(b.r_max, 1), cfg.h), dtype=torch.uint8, device="cuda")
        xd = torch.empty_like(b.x_disp)
        calls["fp8_scale_us"] = lambda: M.moe_fp8_scale(cfg, x, scale, b.ws, stream)
        calls["fp8_dispatch_us"] = lambda: M.moe_dispatch_fp8(
            cfg, x, scale, b.topk_idx, b.capacity, b.expert_offsets, b.route_rank, b.route_row,
            b.row_token, xq, None, b.ws, stream)
        calls["fp8_dequantize_us"] = lambda: M.moe_fp8_dequantize(
            cfg, b.capacity, xq, scale, b.expert_offsets, xd, stream)
        R = int(b.expert_offsets[-1].item())
        out["fp8_payload_bytes"] = R * cfg.h
        out["bf16_payload_bytes"] = R * cfg.h * 2
    for name, fn in calls.items():
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        with torch.cuda.stream(stream):
            for a, e in evs:
                a.record(stream)
                fn()
                e.record(stream)
        torch.cuda.synchronize()
        out[name] = statistics.fmean(a.elapsed_time(e) for a, e in evs) * 1e3
    return out


def routing_scenarios(M, W, torch, stream, reps=200):
    """The expert-parallel mechanism workload of the pages (2 ranks x 256
    tokens, h 1024, 4 experts, top-2, cf 1.25, bf16) under its three routing
    scenarios: the whole step (logits-in route, dispatch, FFN, combine,
    ledger) per scenario, its average time, the ledger's locality / overflow /
    balance and the plan decision."""
    from expert_dispatch_combine_amd.runner import (LayerBuffers, LayerPlan, capacity_of,
                                                    cfg_from, pack_weights)
    cfg = W.SCENARIO_CONFIG
    inp = W.make_inputs(cfg, "cuda")
    mc = cfg_from(cfg)
    b = LayerBuffers(mc, capacity_of(mc), "cuda")
    w1, w2 = pack_weights(mc, inp.w1, inp.w2)
    out = {"workload": f"{cfg.name}: T={cfg.T} h={cfg.h} E={cfg.E} K={cfg.K} F={cfg.F} "
                       f"cf={cfg.cf} n_ep={cfg.n_ep}"}
    for name in W.ROUTING_SCENARIOS:
        b.logits.copy_(torch.from_numpy(W.scenario_logits(name)))
        plan = LayerPlan(b, inp.x, inp.w_gate, None, w1, inp.b1, w2, inp.b2, inp.src_rank,
                         inp.owner_rank, cfg.n_ep, main=stream, logits_in=True, packed=True)
        with torch.cuda.stream(stream):
            for _ in range(10):
                plan.launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                plan.launch()
            e1.record(stream)
        torch.cuda.synchronize()
        led = plan.ledger()
        out[name] = {"step_us": e0.elapsed_time(e1) * 1e3 / reps,
                     "local_hit_ratio": led["local_hit_ratio"],
                     "cross_rank_dispatch_bytes": led["cross_rank_dispatch_bytes"],
                     "overflow": led["overflow"], "balance_ratio": led["balance_ratio"],
                     "plan": M.moe_recommend_plan(led)}
    return out


def committed_traffic(kernel, workload):
    """HBM bytes per call of `kernel` on `workload` from the rocprofv3 counter
    summary committed under profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled
    by a plain copy's reading), or None when there is none or the kernel's
    sources have changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path, encoding="utf-8") as fh:
            for line in fh:
                if not line.startswith("traffic-json: "):
                    continue
                rec = json.loads(line[len("traffic-json: "):])
                if rec.get("kernel") != kernel or rec.get("workload") != workload:
                    continue
                h = hashlib.sha256()
                for src in rec["sources"]:
                    with open(os.path.join(ROOT, src), "rb") as sf:
                        h.update(sf.read())
                if h.hexdigest() == rec["sources_sha256"]:
                    return int(rec["bytes_per_call"])
    return None


def cpu_baseline(wl, inp, budget_s):
    """The oracle as it stands, on the host cores: the whole layer of the same
    workload (route -> dispatch -> FFN -> combine, float64), timed per pass."""
    import oracle as O
    import moe_workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    x, wg = W.host_f64(inp.x), W.host_f64(inp.w_gate)
    w1, b1, w2, b2 = (W.host_f64(t) for t in (inp.w1, inp.b1, inp.w2, inp.b2))
    bias = None if inp.logit_bias is None else inp.logit_bias.cpu().numpy()
    h_round = "bf16" if wl.dtype == "bf16" else "f32"
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        O.moe_layer(x, wg, w1, b1, w2, b2, wl.K, wl.cf, logit_bias=bias, h_round=h_round)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 5:
            break
    med = statistics.median(times)
    return {"value": wl.T / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} full passes of the {wl.name} layer ({wl.T} tokens; "
                      f"route, dispatch, FFN, combine), float64 oracle, median {med:.3f} s "
                      f"per pass"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this MoE layer path has no multi-GPU mode "
              "(expert parallelism over several GPUs is described, not built). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_workloads as W
    import expert_dispatch_combine_amd as M
    from expert_dispatch_combine_amd.runner import (LayerBuffers, LayerPlan, capacity_of,
                                                    cfg_from, pack_weights)

    M.load_library()
    wl = W.CONFIGS[args.config]
    torch.cuda.set_device(0)
    inp = W.make_inputs(wl, "cuda")
    mc = cfg_from(wl)
    cap = capacity_of(mc)
    bufs = LayerBuffers(mc, cap, "cuda")

    # rotation sets: distinct copies of x and all weights
    set_bytes = sum(t.numel() * t.element_size() for t in
                    (inp.x, inp.w_gate, inp.w1, inp.b1, inp.w2, inp.b2))
    n_rot = max(1, int(-(-args.rotate_bytes // set_bytes)))
    packed = args.weights == "packed" and wl.dtype == "bf16"
    sets = []
    for i in range(n_rot):
        st = [inp.x, inp.w_gate, inp.logit_bias, inp.w1, inp.b1, inp.w2, inp.b2]
        if i > 0:
            st = [None if t is None else t.clone() for t in st]
        if packed:  # one-time layout change of the static weights (not timed)
            st[3], st[5] = pack_weights(mc, st[3], st[5])
        sets.append(tuple(st))
    torch.cuda.synchronize()

    main_s = torch.cuda.Stream()
    side_s = torch.cuda.Stream() if args.ledger_stream == "side" else None
    ledger_ws = torch.empty_like(bufs.ws)
    plans = [LayerPlan(bufs, *st, inp.src_rank, inp.owner_rank, wl.n_ep, 0.01, main=main_s,
                       side=side_s, ledger_ws=ledger_ws, packed=packed,
                       fused_tail=args.ledger_stream == "fused",
                       gather_in_ffn=args.gather == "ffn") for st in sets]
    torch.cuda.synchronize()
    done = [torch.cuda.Event() for _ in range(n_rot)]

    # eager warm-up (also before any capture)
    with torch.cuda.stream(main_s):
        for i in range(max(args.warmup, n_rot)):
            plans[i % n_rot].launch()
    torch.cuda.synchronize()
    led = plans[0].ledger()

    graphs = None
    if args.mode == "graph":
        graphs = []
        for pl in plans:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=main_s):
                pl.launch()
            graphs.append(g)
        torch.cuda.synchronize()
        with torch.cuda.stream(main_s):
            for i in range(args.warmup):
                graphs[i % n_rot].replay()
        torch.cuda.synchronize()

    # The host decodes step i-lag's ledger (C moe_ledger_finalize into the
    # plan's buffers) after issuing step i, so up to `lag` later steps stay
    # queued on the device while it does.  A plan's stage is rewritten only
    # when the plan is launched again, n_rot steps later, so lag < n_rot (with
    # a single rotation set each step is decoded before the next is issued).
    lag = min(4, n_rot - 1)

    def run_steps(K, events=None):
        pending = []
        with torch.cuda.stream(main_s):
            for i in range(K):
                j = i % n_rot
                if graphs is not None and events is None:
                    graphs[j].replay()
                else:
                    plans[j].launch(events[i] if events else None)
                done[j].record(main_s)
                pending.append(j)
                if len(pending) > lag:
                    old = pending.pop(0)
                    done[old].synchronize()
                    plans[old].decode()
            for old in pending:
                done[old].synchronize()
                plans[old].decode()
        return j

    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    last = run_steps(K)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    led = plans[last].ledger()

    # eager pass with events around each call (per-call times, roofline)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run_steps(K, evs)
    torch.cuda.synchronize()
    elapsed_eager = time.perf_counter() - t1

    def mean_ms(a, b):
        return statistics.fmean(evs[i][a].elapsed_time(evs[i][b]) for i in range(K))

    t_route, t_disp, t_ffn, t_comb = mean_ms(0, 1), mean_ms(1, 2), mean_ms(2, 3), mean_ms(3, 4)
    R = int(led["accepted_routes"])
    offs = bufs.expert_offsets.cpu().tolist()
    e_nz = sum(1 for e in range(wl.E) if offs[e + 1] > offs[e])
    alg = algorithmic(wl, R, e_nz)
    ffn_s = t_ffn * 1e-3
    ai = alg["ffn_flops"] / alg["ffn_bytes"]
    peak_flops = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    ridge = peak_flops * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": alg["ffn_bytes"] / ffn_s / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": alg["ffn_flops"] / ffn_s / 1e12,
                "peak": peak_flops, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = committed_traffic("expert_ffn", wl.name) if packed else None
    roof.update({
        "kernel": "expert FFN grouped GEMM: the two launches (GEMM1, GEMM2) of one "
                  "moe_expert_ffn, timed together",
        "algorithmic_bytes": alg["ffn_bytes"], "algorithmic_flops": alg["ffn_flops"],
        "arithmetic_intensity": ai, "mfma_util": alg["ffn_flops"] / ffn_s / 1e12 / peak_flops,
        "avg_ms": t_ffn,
    })
    if roof["traffic"] is not None:
        roof["traffic_over_algorithmic"] = roof["traffic"] / alg["ffn_bytes"]

    res = {
        "metric": BASELINE_METRIC,
        "value": wl.T * K / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: T={wl.T} h={wl.h} E={wl.E} K={wl.K} F={wl.F} "
                               f"cf={wl.cf}", "T": wl.T, "h": wl.h, "E": wl.E, "K": wl.K,
                   "F": wl.F, "capacity_factor": wl.cf, "capacity": cap, "n_ep": wl.n_ep,
                   "mode": args.mode, "weights": "packed" if packed else "row-major",
                   "ledger_stream": args.ledger_stream, "gather": args.gather,
                   "rotated_copies": n_rot, "parallelism": "single GPU"},
        "routes_per_s": wl.A * K / elapsed,
        "accepted_routes_per_s": R * K / elapsed,
        "eager_tokens_per_s": wl.T * K / elapsed_eager,
        "per_call_ms": {"route": t_route, "dispatch": t_disp, "expert_ffn": t_ffn,
                        ("combine_ledger" if args.ledger_stream == "fused" else "combine"):
                        t_comb},
        "roofline": roof,
        "ledger": {k: led[k] for k in ("accepted_routes", "overflow", "balance_ratio",
                                        "local_hit_ratio", "l_aux")},
    }
    if not args.no_next_rows:
        res["next_rows"] = next_rows(M, bufs, torch, main_s, inp.x)
        res["next_rows"]["routing_scenarios"] = routing_scenarios(M, W, torch, main_s)
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wl, inp,
                                                                         args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

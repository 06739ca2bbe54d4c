#!/usr/bin/env python3
"""Throughput of one MoE layer (route -> capacity dispatch -> expert FFN ->
combine, plus the ledger) on one MI355X, through the C ABI of libmoe.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the whole path over one batch: moe_route, moe_dispatch,
moe_expert_ffn, moe_combine on the main stream and moe_ledger (the counters,
read back to the host) on a side stream that waits for the dispatch, so the
host-side readback overlaps the expert FFN.  Inputs are resident in HBM.  To
keep the 256 MB last-level cache from serving the weights, successive steps
rotate over several copies of x and of all weights (>= 1 GiB in total).

Prints ONE JSON line: routed tokens/s (whole job), per-call times from HIP
events, the roofline of the dominant kernel (the expert FFN grouped GEMM,
whose two launches are timed together with events on its stream), and the CPU
oracle timed on a bounded sample of the same workload.
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
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=2,
                   help="workload id (2 = Switch-Base-shaped layer, the headline)")
    p.add_argument("--rotate-bytes", type=float, default=float(1 << 30),
                   help="total bytes of rotated input copies (defeats the 256 MB cache)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="rough budget of the CPU-oracle baseline")
    return p.parse_args()


def algorithmic(cfg, R, E_nz, b):
    """Bytes / flops the method must move / do (not padded rows, not dense T*E)."""
    T, h, E, K, F = cfg.T, cfg.h, cfg.E, cfg.K, cfg.F
    return {
        "ffn_bytes": E_nz * 2 * h * F * b + R * h * b + 2 * R * F * b + R * h * 4,
        "ffn_flops": 4 * h * F * R,
        "route_bytes": T * h * b + E * h * b + T * E * 4 + T * K * 8,
        "route_flops": 2 * T * h * E,
        "dispatch_bytes": 2 * R * h * b + T * K * 4 * 4,
        "combine_bytes": R * h * 4 + T * h * 4 + T * K * 8,
    }


def cpu_baseline(wl, inp, budget_s):
    """The oracle as it stands, on the host cores: the whole layer of the same
    workload (route -> dispatch -> FFN -> combine, float64), timed per pass."""
    import numpy as np
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
            "sample": f"{len(times)} full passes of the {wl.name} layer ({wl.T} tokens), "
                      f"float64 oracle, median {med:.2f} s per pass"}


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
    from expert_dispatch_combine_amd.runner import (LayerBuffers, capacity_of, cfg_from,
                                                    run_combine, run_dispatch, run_ffn,
                                                    run_route)

    M.load_library()
    wl = W.CONFIGS[args.config]
    torch.cuda.set_device(0)
    dev = "cuda"
    inp = W.make_inputs(wl, dev)
    mc = cfg_from(wl)
    cap = capacity_of(mc)
    bufs = LayerBuffers(mc, cap, dev)

    # rotation sets: distinct copies of x and all weights
    set_bytes = sum(t.numel() * t.element_size() for t in
                    (inp.x, inp.w_gate, inp.w1, inp.b1, inp.w2, inp.b2))
    n_rot = max(1, int(-(-args.rotate_bytes // set_bytes)))
    sets = [(inp.x, inp.w_gate, inp.logit_bias, inp.w1, inp.b1, inp.w2, inp.b2)]
    for _ in range(n_rot - 1):
        sets.append(tuple(None if t is None else t.clone() for t in sets[0]))
    src, owner = inp.src_rank, inp.owner_rank

    main_s = torch.cuda.current_stream()
    side_s = torch.cuda.Stream()
    ledger_ws = torch.empty_like(bufs.ws)  # the ledger runs beside the FFN: own workspace
    ev_disp_done = torch.cuda.Event()

    def step(i, ev=None):
        x, wg, lb, w1, b1, w2, b2 = sets[i % n_rot]
        if ev:
            ev[0].record(main_s)
        run_route(bufs, x, wg, lb, expert_load=False)
        if ev:
            ev[1].record(main_s)
        run_dispatch(bufs, x, expert_load=True)
        ev_disp_done.record(main_s)
        if ev:
            ev[2].record(main_s)
        run_ffn(bufs, w1, b1, w2, b2)
        if ev:
            ev[3].record(main_s)
        run_combine(bufs)
        if ev:
            ev[4].record(main_s)
        # ledger of this batch on the side stream (reads topk/route_row only)
        side_s.wait_event(ev_disp_done)
        with torch.cuda.stream(side_s):
            led = M.moe_ledger(mc, bufs.topk_idx, bufs.topk_gate, bufs.route_row, cap, src,
                               owner, wl.n_ep, 0.01, ledger_ws, side_s)
        main_s.wait_stream(side_s)  # next step's route overwrites what the ledger read
        return led

    for i in range(args.warmup):
        led = step(i)
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        led = step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def mean_ms(a, b):
        return statistics.fmean(evs[i][a].elapsed_time(evs[i][b]) for i in range(K))

    t_route, t_disp, t_ffn, t_comb = mean_ms(0, 1), mean_ms(1, 2), mean_ms(2, 3), mean_ms(3, 4)
    R = int(led["accepted_routes"])
    offs = bufs.expert_offsets.cpu().tolist()
    e_nz = sum(1 for e in range(wl.E) if offs[e + 1] > offs[e])
    alg = algorithmic(wl, R, e_nz, wl.bytes_per_elem)
    ms_per_step = elapsed * 1e3 / K
    tokens_per_s = wl.T * K / elapsed
    ffn_s = t_ffn * 1e-3
    ai = alg["ffn_flops"] / alg["ffn_bytes"]
    peak_flops = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    ridge = peak_flops * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": alg["ffn_bytes"] / ffn_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": alg["ffn_flops"] / ffn_s / 1e12,
                "peak": peak_flops, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "expert FFN grouped GEMM (GEMM1 + GEMM2 launches of one moe_expert_ffn)"
    roof["algorithmic_bytes"] = alg["ffn_bytes"]
    roof["algorithmic_flops"] = alg["ffn_flops"]
    roof["mfma_util"] = alg["ffn_flops"] / ffn_s / 1e12 / peak_flops
    roof["avg_ms"] = t_ffn

    res = {
        "metric": BASELINE_METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: T={wl.T} h={wl.h} E={wl.E} K={wl.K} F={wl.F} "
                               f"cf={wl.cf}", "T": wl.T, "h": wl.h, "E": wl.E, "K": wl.K,
                   "F": wl.F, "capacity_factor": wl.cf, "capacity": cap, "n_ep": wl.n_ep,
                   "rotated_copies": n_rot, "parallelism": "single GPU"},
        "routes_per_s": wl.A * K / elapsed,
        "accepted_routes_per_s": R * K / elapsed,
        "per_call_ms": {"route": t_route, "dispatch": t_disp, "expert_ffn": t_ffn,
                        "combine": t_comb},
        "roofline": roof,
        "ledger": {k: led[k] for k in ("accepted_routes", "overflow", "balance_ratio",
                                        "local_hit_ratio", "l_aux")},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

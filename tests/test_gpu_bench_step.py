"""The benchmarked step itself, against the oracle, on every workload at full
size: every accepted row of both GEMMs and every token.

The step is built by bench.py's own `step_plan` with its defaults: packed
expert weights (bf16 workloads), moe_dispatch moving no row and the first GEMM
gathering x[row_token[r]] in its loads (moe_expert_ffn_rows), and the combine
with the ledger in one moe_combine_ledger call whose stage is decoded on the
host.  One launch() of that plan, then:

  router   GPU logits within the rigorous fp32-accumulation bound of the
           oracle's float64 logits;
  routing  the oracle's top-k + softmax fed the GPU's own fp32 logits: ids
           bit-exact, gates within 1e-5 relative;
  slots    the oracle's capacity slotting of the GPU's ids: ranks, rows,
           row_token and offsets bit-exact;
  FFN      every accepted row's H and Y against O.expert_ffn_segment on
           x[row_token] (one expert's weights on the host at a time), within
           the derived bounds of gpu_util.check_ffn_segment;
  combine  out against O.combine of the GPU's own Y and gates within the fp32
           bound (K + 1) u sum_k |g_k Y_k|; and against O.combine of the
           oracle's Y within 2e-2 RMS, every token (pinned routing);
  layer    the oracle's own routing (from its float64 logits): tokens whose
           ids differ must be near ties (adjacent logits among the top K + 1
           within 1e-4), tokens whose accepted expert set differs only through
           such flips (at most twice their number); every other token's
           output, sum_k g_k FFN_e(x_t) over the oracle's accepted routes,
           within 2e-2 RMS;
  ledger   the decoded stage against O.ledger of the GPU's routing (integer
           fields bit-exact, P within its fixed-point bound).
"""
import importlib.util
import os

import numpy as np
import pytest
import torch

import oracle as O
from conftest import ROOT
from expert_dispatch_combine_amd.runner import pack_weights
from gpu_util import (U32, banner, bias_np, buffers_for, check_ffn_segment, compare_ledger,
                      device_inputs, host, host_expert, logit_bound, near_tie_tokens, rms)

pytestmark = pytest.mark.gpu


def _bench():
    spec = importlib.util.spec_from_file_location("bench_step", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_benchmarked_step_matches_the_oracle(cid):
    banner(f"benchmarked step config {cid}")
    bench = _bench()
    inp = device_inputs(cid)
    wl = inp.cfg
    b = buffers_for(wl)
    packed = wl.dtype == "bf16"
    w1, w2 = pack_weights(b.cfg, inp.w1, inp.w2) if packed else (inp.w1, inp.w2)
    main = torch.cuda.Stream()
    plan = bench.step_plan(b, (inp.x, inp.w_gate, inp.logit_bias, w1, inp.b1, w2, inp.b2),
                           inp, wl, main, packed)
    b.out.fill_(float("nan"))
    b.h_buf.zero_()
    b.y.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(main):
        plan.launch()
    torch.cuda.synchronize()
    led = plan.ledger()
    del w1, w2

    T, K, E = wl.T, wl.K, wl.E
    bias = bias_np(inp)
    x64 = host(inp.x)
    logits_g = b.logits.cpu().numpy()
    idx_g = b.topk_idx.cpu().numpy()
    gate_g = b.topk_gate.cpu().numpy()
    rank_g = b.route_rank.cpu().numpy()
    row_g = b.route_row.cpu().numpy()
    offs_g = b.expert_offsets.cpu().numpy()
    R = int(offs_g[-1])
    tok_g = b.row_token[:R].cpu().numpy()
    out_g = b.out.cpu().numpy().astype(np.float64)

    # router: float64 logits rounded once vs the fp32-accumulated product
    wg64 = host(inp.w_gate)
    logits_o = O.router_logits(x64, wg64)
    assert np.all(np.abs(logits_g.astype(np.float64) - logits_o)
                  <= logit_bound(x64, wg64) + 2 * U32 * np.abs(logits_o))

    # routing and slots on the GPU's own logits
    idx_p, gate_p = O.topk_softmax(logits_g, K, bias)
    assert np.array_equal(idx_g, idx_p)
    assert np.all(np.abs(gate_g - gate_p) <= 1e-5 * np.abs(gate_p))
    cap = O.capacity(T * K, E, wl.cf)
    assert cap == b.capacity
    sl = O.slot_routes(idx_g, E, cap)
    assert np.array_equal(rank_g, sl["route_rank"])
    assert np.array_equal(row_g, sl["route_row"])
    assert np.array_equal(offs_g, sl["expert_offsets"])
    assert R == sl["R"] and np.array_equal(tok_g, sl["row_token"])

    # expert FFN: every accepted row, one expert's weights at a time
    h_round = "bf16" if wl.dtype == "bf16" else "f32"
    Y_o = np.zeros((R, wl.h))
    H_g = b.h_buf[:R].float().cpu().numpy() if R else np.zeros((0, wl.F))
    Y_g = b.y[:R].cpu().numpy() if R else np.zeros((0, wl.h))
    experts = 0
    for e in range(E):
        lo, hi = int(offs_g[e]), int(offs_g[e + 1])
        if hi == lo:
            continue
        experts += 1
        Y_o[lo:hi] = check_ffn_segment(h_round, x64[tok_g[lo:hi]], host_expert(inp.w1, e),
                                       host_expert(inp.b1, e), host_expert(inp.w2, e),
                                       host_expert(inp.b2, e), H_g[lo:hi].astype(np.float64),
                                       Y_g[lo:hi].astype(np.float64))
    del H_g

    # combine: the kernel on its own inputs, then the oracle's Y (every token)
    want = O.combine(Y_g, row_g, gate_g)
    mag = np.zeros((T, wl.h))
    for k in range(K):
        m = row_g[:, k] >= 0
        mag[m] += np.abs(gate_g[m, k][:, None].astype(np.float64) * Y_g[row_g[m, k]])
    assert np.all(np.abs(out_g - want) <= (K + 1) * U32 * mag + 1e-30)
    pinned = O.combine(Y_o, row_g, gate_g)
    assert np.max(np.abs(out_g - pinned)) <= 2e-2 * rms(pinned)
    del Y_g, mag, want

    # the layer against the oracle's own routing
    idx_o, gate_o = O.topk_softmax(logits_o, K, bias)
    sl_o = O.slot_routes(idx_o, E, cap)
    tie = near_tie_tokens(logits_o, bias, K)
    flipped = ~np.all(idx_g == idx_o, axis=1)
    assert not np.any(flipped & ~tie), np.nonzero(flipped & ~tie)[0][:8]
    acc_o = sl_o["route_row"] >= 0
    acc_g = row_g >= 0
    set_differs = np.array([sorted(idx_o[t][acc_o[t]]) != sorted(idx_g[t][acc_g[t]])
                            for t in range(T)], bool)
    cascade = set_differs & ~flipped
    assert cascade.sum() <= 2 * flipped.sum(), (int(cascade.sum()), int(flipped.sum()))
    keep = ~(flipped | set_differs)
    # kept tokens have the same ids in the same slots and the same accepted
    # routes, so the oracle's FFN output of route (t, k) is Y_o[row_g[t, k]]
    out_o = np.zeros((T, wl.h))
    for k in range(K):
        m = keep & acc_o[:, k]
        out_o[m] += gate_o[m, k][:, None].astype(np.float64) * Y_o[row_g[m, k]]
    out_o = O.round_f32(out_o)
    err = float(np.abs(out_g[keep] - out_o[keep]).max()) if keep.any() else 0.0
    scale = rms(out_o[keep])
    covered = {int(e) for t in np.nonzero(keep)[0] for e in idx_o[t][acc_o[t]]}
    print(f"[step] config {cid}: rows={R} experts={experts} tokens={int(keep.sum())}/{T} "
          f"flips={int(flipped.sum())} cascade={int(cascade.sum())} "
          f"max_err/rms={err / max(scale, 1e-30):.3e}", flush=True)
    assert err <= 2e-2 * scale
    # every expert that received a row is exercised by some compared token,
    # unless each of its rows belongs to an excluded (near-tie) token
    for e in {e for e in range(E) if offs_g[e + 1] > offs_g[e]} - covered:
        assert not keep[tok_g[offs_g[e]:offs_g[e + 1]]].any(), e

    # ledger: the decoded stage of the fused tail
    src, owner = inp.src_rank.cpu().numpy(), inp.owner_rank.cpu().numpy()
    o = O.ledger(idx_g, gate_g, row_g, cap, src, owner, wl.n_ep, wl.h, wl.bytes_per_elem)
    compare_ledger(led, o)
    assert led["status"] == 0

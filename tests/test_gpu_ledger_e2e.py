"""moe_ledger and the whole layer (route -> dispatch -> FFN -> combine) on the
GPU vs the oracle.

Ledger: fed the oracle's routing; integer counters bit-exact, float64 values
from the same formulas equal.  The device adds gates in fixed point (each fp32
gate rounded to a multiple of 2^-32, then summed exactly), so each P_e may
differ from the float64 sum by at most load_e * 2^-33 / T (plus the oracle's
own float64 rounding), and L_aux by alpha * sum_e f_e * that bound.

Layer: GPU logits come from bf16 MFMA, the oracle's from float64, so tokens
whose K-th and (K+1)-th oracle logits lie within 1e-4 may route differently
and are excluded; under capacity overflow each such flip can move the
acceptance boundary of its two experts, so tokens whose accepted expert set
differs are excluded too, and their number must stay within twice the flips.
Every remaining token must satisfy max |out - out_oracle| <= 2e-2 RMS(out_oracle).
"""
import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
import moe_workloads as W
import oracle as O
from expert_dispatch_combine_amd.runner import LayerBuffers, run_layer
from gpu_util import (banner, bias_np, buffers_for, compare_ledger, custom_inputs,
                      device_inputs, host, near_tie_tokens, rms, to_dev)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ ledger
def _oracle_routing(inp):
    cfg = inp.cfg
    logits = O.router_logits(host(inp.x), host(inp.w_gate))
    idx, gate = O.topk_softmax(logits, cfg.K, bias_np(inp))
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    sl = O.slot_routes(idx, cfg.E, cap)
    return idx, gate, cap, sl


def _gpu_ledger(cfg, idx, gate, route_row, cap, src, owner, n_ep, alpha=0.01, **kw):
    mc = M.MoeCfg.make(cfg.T, cfg.h, cfg.E, cfg.K, cfg.F, cfg.dtype, cfg.cf)
    ws = torch.empty(M.moe_workspace_bytes(mc), dtype=torch.uint8, device="cuda")
    return M.moe_ledger(mc, to_dev(idx, torch.int32), to_dev(gate, torch.float32),
                        to_dev(route_row, torch.int32), cap, to_dev(src, torch.int32),
                        to_dev(owner, torch.int32), n_ep, alpha, ws, **kw)


_compare_ledger = compare_ledger


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_ledger_on_workloads(cid):
    banner(f"ledger config {cid}")
    inp = device_inputs(cid, with_experts=cid in (3, 4))
    cfg = inp.cfg
    idx, gate, cap, sl = _oracle_routing(inp)
    src, owner = inp.src_rank.cpu().numpy(), inp.owner_rank.cpu().numpy()
    g = _gpu_ledger(cfg, idx, gate, sl["route_row"], cap, src, owner, cfg.n_ep)
    o = O.ledger(idx, gate, sl["route_row"], cap, src, owner, cfg.n_ep, cfg.h,
                 cfg.bytes_per_elem)
    _compare_ledger(g, o)
    assert g["status"] == 0 and g["invalid_routes"] == 0
    if cid == 5:
        assert g["imbalanced"] == 1 and g["balance_ratio"] > 2.0
    if cid == 4:  # the per-pair all-to-all volume of the page's DeepSeek-V3 row
        assert g["pair_bytes_uniform"] == 58720256.0
    if cid == 2:
        assert g["pair_bytes_uniform"] == 196608.0


@pytest.mark.parametrize("T,E,K,n_ep,cf", [(1, 1, 1, 1, 1.0), (300, 5, 2, 3, 0.7),
                                           (5000, 64, 6, 64, 1.0), (999, 1000, 4, 7, 1.0),
                                           (4097, 256, 8, 8, 0.5),
                                           (1500, 1024, 32, 64, 0.5)])  # E, K, n_ep at their limits
def test_ledger_random(T, E, K, n_ep, cf):
    banner(f"ledger random T={T} E={E} K={K} n_ep={n_ep}")
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    gate = rng.random((T, K)).astype(np.float32)
    cap = O.capacity(T * K, E, cf)
    sl = O.slot_routes(idx, E, cap)
    src = rng.integers(0, n_ep, T).astype(np.int32)
    owner = (np.arange(E) % n_ep).astype(np.int32)
    cfg = W.custom(T=T, h=192, E=E, K=K, F=64, cf=cf, dtype="bf16")
    g = _gpu_ledger(cfg, idx, gate, sl["route_row"], cap, src, owner, n_ep, alpha=0.02)
    o = O.ledger(idx, gate, sl["route_row"], cap, src, owner, n_ep, 192, 2, alpha=0.02)
    _compare_ledger(g, o)


def test_ledger_empty_and_errors():
    banner("ledger empty / errors")
    cfg = W.custom(T=0, h=64, E=4, K=2, F=64, dtype="bf16")
    mc = M.MoeCfg.make(0, 64, 4, 2, 64, "bf16", 1.0)
    ws = torch.empty(M.moe_workspace_bytes(mc), dtype=torch.uint8, device="cuda")
    owner = to_dev(np.arange(4) % 2, torch.int32)
    g = M.moe_ledger(mc, None, None, None, 0, None, owner, 2, 0.01, ws)
    assert g["total_routes"] == 0 and g["capacity"] == 0 and g["balance_ratio"] == 0.0
    assert g["local_hit_ratio"] == 0.0 and g["l_aux"] == 0.0 and g["loads"] == [0] * 4
    # an expert id outside [0, E) is reported
    idx = np.array([[0, 1], [2, 4]], np.int32)
    cfg = W.custom(T=2, h=64, E=4, K=2, F=64, dtype="bf16")
    g = _gpu_ledger(cfg, idx, np.full((2, 2), 0.5, np.float32), np.full((2, 2), -1, np.int32),
                    1, np.zeros(2, np.int32), np.arange(4) % 2, 2, raise_on_error=False)
    assert g["return_status"] == 2 and g["invalid_routes"] == 1
    # an owner rank outside [0, n_ep) is reported
    idx = np.array([[0, 1], [2, 3]], np.int32)
    g = _gpu_ledger(cfg, idx, np.full((2, 2), 0.5, np.float32), np.full((2, 2), -1, np.int32),
                    1, np.zeros(2, np.int32), np.array([0, 1, 5, 0]), 2, raise_on_error=False)
    assert g["return_status"] == 1


@pytest.mark.parametrize("T,h,E,K,n_ep,cf,dtype,pinned", [
    (2048, 768, 16, 1, 8, 1.25, "bf16", True),    # one launch
    (2048, 768, 16, 2, 8, 0.6, "bf16", True),     # 4096 routes: still one launch, drops
    (2049, 64, 16, 2, 4, 1.0, "bf16", False),     # 4098 routes: two launches, copied stage
    (100, 7168, 64, 2, 8, 1.0, "f32", True),      # one token per combine workgroup (U = 7)
    (37, 30, 3, 3, 2, 0.5, "f32", False),         # scalar rows, K = E, heavy drops
    (1, 64, 1, 1, 1, 1.0, "bf16", True)])
def test_combine_ledger_equals_the_two_calls(T, h, E, K, n_ep, cf, dtype, pinned):
    """moe_combine_ledger gives the same `out` (bit for bit) and the same
    decoded ledger as moe_combine followed by moe_ledger_launch (its stage may
    hold the counters in several integer parts), and that ledger equals the
    oracle's."""
    banner(f"combine+ledger T={T} h={h} E={E} K={K} pinned={pinned}")
    rng = np.random.default_rng(T * 31 + h)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    gate = rng.random((T, K)).astype(np.float32)
    cap = O.capacity(T * K, E, cf)
    sl = O.slot_routes(idx, E, cap)
    src = rng.integers(0, n_ep, T).astype(np.int32)
    owner = (np.arange(E) % n_ep).astype(np.int32)
    mc = M.MoeCfg.make(T, h, E, K, 64, dtype, cf)
    R = max(int(sl["R"]), 1)
    y = torch.randn(R, h, dtype=torch.float32, device="cuda")
    d = dict(idx=to_dev(idx, torch.int32), gate=to_dev(gate, torch.float32),
             row=to_dev(sl["route_row"], torch.int32), src=to_dev(src, torch.int32),
             owner=to_dev(owner, torch.int32))
    ws = torch.empty(M.moe_workspace_bytes(mc), dtype=torch.uint8, device="cuda")
    nst = M.moe_ledger_stage_bytes(mc, n_ep)
    st_two = torch.zeros((nst,), dtype=torch.uint8, pin_memory=pinned)
    st_one = torch.full((nst,), 0xAB, dtype=torch.uint8, pin_memory=pinned)
    out_two = torch.empty(T, h, dtype=torch.float32, device="cuda")
    out_one = torch.full((T, h), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_combine(mc, y, d["row"], d["gate"], out_two)
    M.moe_ledger_launch(mc, d["idx"], d["gate"], d["row"], d["src"], d["owner"], n_ep, st_two,
                        ws)
    torch.cuda.synchronize()
    M.moe_combine_ledger(mc, y, d["row"], d["gate"], out_one, d["idx"], d["src"], d["owner"],
                         n_ep, st_one, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_one, out_two)
    g = M.moe_ledger_finalize(mc, cap, n_ep, 0.01, st_one)
    assert g == M.moe_ledger_finalize(mc, cap, n_ep, 0.01, st_two)
    o = O.ledger(idx, gate, sl["route_row"], cap, src, owner, n_ep, h, 2 if dtype == "bf16" else 4)
    _compare_ledger(g, o)


def test_combine_ledger_empty_batch():
    banner("combine+ledger empty")
    mc = M.MoeCfg.make(0, 64, 4, 2, 64, "bf16", 1.0)
    ws = torch.empty(M.moe_workspace_bytes(mc), dtype=torch.uint8, device="cuda")
    owner = to_dev(np.arange(4) % 2, torch.int32)
    stage = torch.full((M.moe_ledger_stage_bytes(mc, 2),), 0xAB, dtype=torch.uint8,
                       pin_memory=True)
    M.moe_combine_ledger(mc, None, None, None, None, None, None, owner, 2, stage, ws)
    torch.cuda.synchronize()
    g = M.moe_ledger_finalize(mc, 0, 2, 0.01, stage)
    assert g["total_routes"] == 0 and g["loads"] == [0] * 4 and g["l_aux"] == 0.0


# ------------------------------------------------------------------ the layer
class _HostExperts:
    """Per-expert float64 host copies of device weights, fetched on demand."""

    def __init__(self, t):
        self.t = t
        self.key = None
        self.val = None

    def __getitem__(self, e):
        e = int(e)
        if self.key != e:
            self.key, self.val = e, host(self.t[e])
        return self.val


def _oracle_token_outputs(inp, tokens, idx, gate, accepted):
    """out[t] = sum over accepted k of g * FFN_e(x_t) for the given tokens
    ([DSV3] section 一), computed token by token (grouped by expert)."""
    cfg = inp.cfg
    h_round = "bf16" if cfg.dtype == "bf16" else "f32"
    x64 = host(inp.x)
    out = np.zeros((len(tokens), cfg.h))
    pairs = [(int(idx[t, k]), i, k) for i, t in enumerate(tokens) for k in range(cfg.K)
             if accepted[t, k]]
    pairs.sort()
    w1, w2 = _HostExperts(inp.w1), _HostExperts(inp.w2)
    b1, b2 = host(inp.b1), host(inp.b2)
    for e, i, k in pairs:
        t = tokens[i]
        _, y = O.expert_ffn_rows(x64[t:t + 1], [0], [w1[e]], [b1[e]], [w2[e]], [b2[e]], h_round)
        out[i] += float(gate[t, k]) * y[0]
    return O.round_f32(out)


def _check_layer(inp, b, max_tokens=None, seed=0):
    cfg = inp.cfg
    x64 = host(inp.x)
    logits_o = O.router_logits(x64, host(inp.w_gate))
    bias = bias_np(inp)
    idx_o, gate_o = O.topk_softmax(logits_o, cfg.K, bias)
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    sl_o = O.slot_routes(idx_o, cfg.E, cap)
    idx_g = b.topk_idx.cpu().numpy()
    row_g = b.route_row.cpu().numpy()
    tie = near_tie_tokens(logits_o, bias, cfg.K)
    flipped = ~np.all(idx_g == idx_o, axis=1)
    assert not np.any(flipped & ~tie), np.nonzero(flipped & ~tie)[0][:8]
    acc_o = sl_o["route_row"] >= 0
    acc_g = row_g >= 0
    set_differs = np.array([sorted(idx_o[t][acc_o[t]]) != sorted(idx_g[t][acc_g[t]])
                            for t in range(cfg.T)], bool)
    cascade = set_differs & ~flipped
    assert cascade.sum() <= 2 * flipped.sum(), (int(cascade.sum()), int(flipped.sum()))
    keep = np.nonzero(~(flipped | set_differs))[0]
    if max_tokens is not None and len(keep) > max_tokens:
        rng = np.random.default_rng(seed)
        keep = np.sort(rng.choice(keep, max_tokens, replace=False))
    want = _oracle_token_outputs(inp, keep, idx_o, gate_o, acc_o)
    got = b.out.cpu().numpy()[keep].astype(np.float64)
    scale = rms(want)
    err = float(np.abs(got - want).max()) if len(keep) else 0.0
    print(f"[e2e] tokens={len(keep)} flips={int(flipped.sum())} cascade={int(cascade.sum())} "
          f"max_err={err:.3e} rms={scale:.3e} ratio={err / max(scale, 1e-30):.3e}", flush=True)
    assert err <= 2e-2 * scale
    return err / max(scale, 1e-30)


@pytest.mark.parametrize("cid", [1, 2])
def test_layer_end_to_end_every_token(cid):
    banner(f"layer e2e config {cid}")
    inp = device_inputs(cid)
    b = buffers_for(inp.cfg)
    run_layer(b, inp.x, inp.w_gate, inp.logit_bias, inp.w1, inp.b1, inp.w2, inp.b2)
    torch.cuda.synchronize()
    _check_layer(inp, b)


@pytest.mark.parametrize("cid,ntok", [(3, 48), (4, 12), (5, 96)])
def test_layer_end_to_end_sampled_tokens(cid, ntok):
    banner(f"layer e2e sampled config {cid}")
    inp = device_inputs(cid)
    b = buffers_for(inp.cfg)
    run_layer(b, inp.x, inp.w_gate, inp.logit_bias, inp.w1, inp.b1, inp.w2, inp.b2)
    torch.cuda.synchronize()
    _check_layer(inp, b, max_tokens=ntok, seed=cid)


@pytest.mark.parametrize("T,h,E,K,F,cf", [(1, 64, 1, 1, 64, 1.0), (333, 128, 6, 2, 192, 0.6),
                                          (1000, 256, 16, 1, 256, 1.25),
                                          (700, 128, 100, 4, 128, 1.0)])
def test_layer_end_to_end_ragged(T, h, E, K, F, cf):
    banner(f"layer e2e ragged T={T} h={h} E={E} K={K} F={F}")
    cfg = W.custom(T=T, h=h, E=E, K=K, F=F, cf=cf, dtype="bf16", seed=T + 3 * E)
    inp = custom_inputs(cfg)
    b = buffers_for(cfg)
    run_layer(b, inp.x, inp.w_gate, None, inp.w1, inp.b1, inp.w2, inp.b2)
    torch.cuda.synchronize()
    _check_layer(inp, b)


def test_layer_is_deterministic():
    banner("layer determinism")
    inp = device_inputs(2)
    b = buffers_for(inp.cfg)
    outs = []
    for _ in range(3):
        run_layer(b, inp.x, inp.w_gate, inp.logit_bias, inp.w1, inp.b1, inp.w2, inp.b2)
        torch.cuda.synchronize()
        outs.append(b.out.clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])

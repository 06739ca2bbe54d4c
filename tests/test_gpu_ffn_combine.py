"""moe_expert_ffn and moe_combine on the GPU vs the oracle, each fed the
oracle's own inputs (its dispatched rows, its expert outputs), so each kernel
is checked on its own.

Tolerances (derived, written out in each test):
  H (bf16): the oracle rounds the exact f64 value, the GPU an fp32-accumulated
     one; both land on the bf16 grid, so they differ by at most one bf16 ulp
     (<= 2^-7 |H|) plus the pre-activation error (<= h u sum|x W1|, GELU'
     <= 1.13).
  Y (fp32): |dY_n| <= sum_f |dH_f| |W2_nf| + F u sum_f |H_f W2_nf| + u |Y|;
     and in RMS, dY must stay below 2^-8 RMS(Y), far under what any indexing
     or operand mistake produces.
  out: fp32 fma of K terms: |d| <= (K+1) u sum_k |g_k Y_k|.
"""
import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
import moe_workloads as W
import oracle as O
from expert_dispatch_combine_amd.runner import LayerBuffers, pack_weights
from gpu_util import (U32, banner, bias_np, check_ffn_segment, custom_inputs, device_inputs,
                      host, host_expert, to_dev)

pytestmark = pytest.mark.gpu


def _oracle_dispatch(inp: W.Inputs):
    cfg = inp.cfg
    x64 = host(inp.x)
    logits = O.router_logits(x64, host(inp.w_gate))
    idx, gate = O.topk_softmax(logits, cfg.K, bias_np(inp))
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    sl = O.slot_routes(idx, cfg.E, cap)
    return idx, gate, cap, sl


def _run_ffn(inp: W.Inputs, cap, sl, packed=False):
    cfg = inp.cfg
    mc = M.MoeCfg.make(cfg.T, cfg.h, cfg.E, cfg.K, cfg.F, cfg.dtype, cfg.cf)
    b = LayerBuffers(mc, cap)
    R = sl["R"]
    if R:
        b.x_disp[:R].copy_(inp.x[torch.from_numpy(sl["row_token"].astype(np.int64)).cuda()])
    b.expert_offsets.copy_(torch.from_numpy(sl["expert_offsets"]))
    if packed:
        w1p, w2p = pack_weights(mc, inp.w1, inp.w2)
        M.moe_expert_ffn_packed(mc, cap, b.x_disp, b.expert_offsets, w1p, inp.b1, w2p, inp.b2,
                                b.h_buf, b.y)
        torch.cuda.synchronize()
        del w1p, w2p
    else:
        M.moe_expert_ffn(mc, cap, b.x_disp, b.expert_offsets, inp.w1, inp.b1, inp.w2, inp.b2,
                         b.h_buf, b.y)
        torch.cuda.synchronize()
    return b


def _check_rows(inp, sl, b, rows):
    """Compare H and Y of the given dispatched rows with the oracle's
    (O.expert_ffn_segment per expert, bounds in gpu_util.check_ffn_segment)."""
    cfg = inp.cfg
    if len(rows) == 0:
        return
    offs = sl["expert_offsets"]
    experts = np.searchsorted(offs, rows, side="right") - 1
    x64 = host(inp.x)[sl["row_token"][rows]]
    h_round = "bf16" if cfg.dtype == "bf16" else "f32"
    Hg = b.h_buf[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    Yg = b.y[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    for e in np.unique(experts):
        m = experts == e
        check_ffn_segment(h_round, x64[m], host_expert(inp.w1, e), host_expert(inp.b1, e),
                          host_expert(inp.w2, e), host_expert(inp.b2, e), Hg[m], Yg[m])


@pytest.mark.parametrize("cid,packed", [(1, False), (2, False), (2, True), (5, False),
                                        (5, True)])
def test_ffn_full_on_workloads(cid, packed):
    banner(f"ffn full config {cid} packed={packed}")
    inp = device_inputs(cid)
    _, _, cap, sl = _oracle_dispatch(inp)
    b = _run_ffn(inp, cap, sl, packed)
    _check_rows(inp, sl, b, np.arange(sl["R"]))


@pytest.mark.parametrize("cid", [3, 4])
def test_ffn_every_row_full_size(cid):
    """Full-size workloads on row-major weights and x_disp, launched exactly as
    the layer launches them; every accepted row of both GEMMs against the
    oracle, one expert's weights on the host at a time.  (The packed weights
    with the rows gathered inside the first GEMM, the benchmarked path, are
    checked the same way in test_gpu_bench_step.)"""
    banner(f"ffn every row config {cid}")
    inp = device_inputs(cid)
    _, _, cap, sl = _oracle_dispatch(inp)
    b = _run_ffn(inp, cap, sl, False)
    _check_rows(inp, sl, b, np.arange(sl["R"]))


@pytest.mark.parametrize("packed", [False, True])
def test_ffn_large_tiles_ragged(packed):
    """Experts of ~3300 rows (not a multiple of the row tile) and F = 4096:
    the MFMA-bound wide kernels on ragged segments (weights in registers when
    packed, LDS-staged 256 x 256 and 128 x 128 tiles when row-major); sampled
    rows (each expert's first and last, both sides of a 256-row boundary,
    random)."""
    banner(f"ffn tiled ragged packed={packed}")
    cfg = W.custom(T=16384, h=256, E=5, K=1, F=4096, cf=1.0, dtype="bf16", seed=31)
    inp = custom_inputs(cfg)
    _, _, cap, sl = _oracle_dispatch(inp)
    b = _run_ffn(inp, cap, sl, packed)
    offs = sl["expert_offsets"]
    rng = np.random.default_rng(31)
    rows = {int(r) for e in range(cfg.E) if offs[e + 1] > offs[e]
            for r in (offs[e], offs[e + 1] - 1, offs[e] + 255, offs[e] + 256)
            if offs[e] <= r < offs[e + 1]}
    rows.update(rng.integers(0, sl["R"], 64).tolist())
    _check_rows(inp, sl, b, np.array(sorted(rows)))


@pytest.mark.parametrize("T,h,E,K,F,cf", [(1, 64, 1, 1, 64, 1.0), (300, 128, 5, 2, 192, 0.8),
                                          (1000, 256, 16, 2, 320, 1.0),
                                          (513, 64, 64, 6, 128, 1.0),
                                          (2500, 192, 3, 1, 448, 1.5),
                                          (2048, 768, 14, 1, 3072, 1.0),
                                          (3000, 128, 4, 1, 384, 1.3),
                                          (2200, 256, 3, 1, 512, 1.0),
                                          (3000, 64, 4, 1, 256, 1.3),
                                          (2600, 192, 4, 1, 256, 1.3),
                                          (1800, 128, 4, 1, 384, 1.3),
                                          (1800, 192, 4, 1, 448, 1.3),
                                          (4096, 256, 16, 1, 4096, 1.25),
                                          (4096, 256, 16, 1, 2304, 1.25),
                                          (4096, 4096, 16, 1, 256, 1.25)])
@pytest.mark.parametrize("packed", [False, True])
def test_ffn_ragged_segments(T, h, E, K, F, cf, packed):
    banner(f"ffn ragged T={T} h={h} E={E} K={K} F={F} packed={packed}")
    cfg = W.custom(T=T, h=h, E=E, K=K, F=F, cf=cf, dtype="bf16", seed=T * 7 + F)
    inp = custom_inputs(cfg)
    _, _, cap, sl = _oracle_dispatch(inp)
    b = _run_ffn(inp, cap, sl, packed)
    _check_rows(inp, sl, b, np.arange(sl["R"]))


@pytest.mark.parametrize("packed", [False, True])
def test_ffn_static_map_with_empty_experts(packed):
    """Every expert's rows fit one 128-row tile (the static tile map) and a
    strong router bias leaves many experts empty and caps the hot ones: the
    multi-strip streaming kernels (four strips in GEMM1 with packed weights,
    two in GEMM2) on empty, full and partial experts; every accepted row."""
    banner(f"ffn static map, empty experts, packed={packed}")
    cfg = W.custom(T=4096, h=256, E=256, K=8, F=2048, cf=1.0, dtype="bf16", zipf_s=3.0, seed=77)
    inp = custom_inputs(cfg)
    _, _, cap, sl = _oracle_dispatch(inp)
    rows = np.diff(sl["expert_offsets"])
    assert cap == 128 and (rows == 0).sum() > 0 and (rows == cap).sum() > 0
    b = _run_ffn(inp, cap, sl, packed)
    _check_rows(inp, sl, b, np.arange(sl["R"]))


def test_ffn_partial_row_tiles_of_every_size():
    """Weights in registers (packed weights, 521 rows per expert on average):
    experts whose last 256-row tile holds 1, 31, 32, 33, 64, 65, 128, 129,
    255, 256 (none) or 257 (one whole tile and 1) rows, and one of 5000 rows
    (19 whole tiles and 136): the partial tiles run with 2, 4 or 8 of their
    32-row sub-tiles, after each XCD's whole tiles; F = 384 leaves half of
    the first GEMM's second weight tile idle.  Every row against the oracle."""
    banner("ffn partial row tiles of every size")
    sizes = [1, 31, 32, 33, 64, 65, 128, 129, 255, 256, 257, 5000]
    E, T = len(sizes), sum(sizes)
    cfg = W.custom(T=T, h=256, E=E, K=1, F=384, cf=10.0, dtype="bf16", seed=91)
    inp = custom_inputs(cfg)
    rng = np.random.default_rng(91)
    idx = rng.permutation(np.repeat(np.arange(E), sizes)).astype(np.int32)[:, None]
    cap = O.capacity(T, E, cfg.cf)
    sl = O.slot_routes(idx, E, cap)
    assert np.array_equal(np.diff(sl["expert_offsets"]), sizes)
    b = _run_ffn(inp, cap, sl, packed=True)
    _check_rows(inp, sl, b, np.arange(sl["R"]))


@pytest.mark.parametrize("cid,shape,packed", [
    (2, None, True), (2, None, False),                     # gather in the streaming loads
    (None, (2048, 768, 14, 1, 3072, 1.0), True),           # ragged, static tile map
    (None, (1000, 256, 4, 1, 320, 1.0), False),            # 250-row experts: tile search
    (None, (513, 64, 64, 6, 128, 1.0), True),              # many small / empty experts
    (None, (2500, 192, 3, 1, 448, 1.5), False),            # long segments: tiled kernel
    (None, (2500, 192, 3, 1, 448, 1.5), True),             # weights in registers, partial tile
    (None, (4096, 256, 4, 1, 512, 1.0), False),            # wide kernel, 256 x 256 tiles
    (None, (4096, 256, 4, 1, 512, 1.0), True),             # weights in registers
    (None, (1800, 128, 4, 1, 384, 1.3), True),             # wide kernel, 128 x 128 tiles
    (None, (1800, 192, 4, 1, 448, 1.3), True),             # 450-row experts: tiled kernel
    (None, (4096, 256, 16, 1, 4096, 1.25), True),          # two weight strips per wave
    (None, (1, 64, 1, 1, 64, 1.0), False),
    (1, None, False)])                                      # fp32: rows copied into y first
def test_ffn_rows_equals_ffn_on_x_disp(cid, shape, packed):
    """moe_expert_ffn_rows on x and row_token gives the same H and Y, bit for
    bit, as moe_expert_ffn(_packed) on x_disp[r] = x[row_token[r]]."""
    banner(f"ffn rows cid={cid} shape={shape} packed={packed}")
    if cid is not None:
        inp = device_inputs(cid)
    else:
        T, h, E, K, F, cf = shape
        inp = custom_inputs(W.custom(T=T, h=h, E=E, K=K, F=F, cf=cf, dtype="bf16",
                                     seed=T * 3 + F))
    _, _, cap, sl = _oracle_dispatch(inp)
    ref = _run_ffn(inp, cap, sl, packed)
    cfg = inp.cfg
    mc = M.MoeCfg.make(cfg.T, cfg.h, cfg.E, cfg.K, cfg.F, cfg.dtype, cfg.cf)
    b = LayerBuffers(mc, cap)
    R = sl["R"]
    b.row_token.fill_(-7)
    if R:
        b.row_token[:R].copy_(torch.from_numpy(sl["row_token"].astype(np.int32)))
    b.expert_offsets.copy_(torch.from_numpy(sl["expert_offsets"]))
    w1, w2 = (pack_weights(mc, inp.w1, inp.w2) if packed else (inp.w1, inp.w2))
    M.moe_expert_ffn_rows(mc, cap, inp.x, b.row_token, b.expert_offsets, w1, inp.b1, w2, inp.b2,
                          b.h_buf, b.y, packed)
    torch.cuda.synchronize()
    assert torch.equal(b.h_buf[:R], ref.h_buf[:R])
    assert torch.equal(b.y[:R], ref.y[:R])


def test_ffn_fp32_odd_sizes():
    banner("ffn fp32 odd sizes")
    cfg = W.custom(T=50, h=7, E=3, K=2, F=5, cf=1.0, dtype="f32", seed=4)
    inp = custom_inputs(cfg)
    _, _, cap, sl = _oracle_dispatch(inp)
    b = _run_ffn(inp, cap, sl)
    _check_rows(inp, sl, b, np.arange(sl["R"]))


# ------------------------------------------------------------------ combine
def _check_combine(T, K, h, R, drop_frac, seed):
    rng = np.random.default_rng(seed)
    Y = rng.standard_normal((max(R, 1), h)).astype(np.float32)
    gate = rng.random((T, K)).astype(np.float32)
    rows = np.full((T, K), -1, np.int32)
    perm = rng.permutation(R)
    flat = rows.reshape(-1)
    take = min(R, T * K)
    pos = rng.permutation(T * K)[:take]
    flat[pos] = perm[:take]
    flat[rng.random(T * K) < drop_frac] = -1
    if T:
        rows[0, :] = -1
    mc = M.MoeCfg.make(T, h, max(K, 4), K, 64, "f32", 1.0)
    out = torch.full((T, h), 7.0, device="cuda")
    M.moe_combine(mc, to_dev(Y, torch.float32), to_dev(rows, torch.int32),
                  to_dev(gate, torch.float32), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = O.combine(Y, rows, gate)
    mag = np.zeros((T, h))
    for k in range(K):
        m = rows[:, k] >= 0
        mag[m] += np.abs(gate[m, k][:, None].astype(np.float64) * Y[rows[m, k]])
    assert np.all(np.abs(got - want) <= (K + 1) * U32 * mag + 1e-30)
    if T:
        assert np.all(got[0] == 0.0)


@pytest.mark.parametrize("T,K,h,R,drop", [(1, 1, 4, 1, 0.0), (64, 2, 32, 119, 0.1),
                                          (2048, 1, 768, 2048, 0.0), (300, 8, 100, 2000, 0.3),
                                          (1000, 6, 2048, 3000, 0.5), (77, 3, 13, 50, 0.2),
                                          (40, 2, 4100, 60, 0.1), (33, 3, 6000, 80, 0.2),
                                          (20, 8, 8192, 150, 0.0), (9, 4, 8196, 30, 0.3),
                                          # K = 32, the library's limit: 16 tokens per
                                          # workgroup (512 LDS entries) and one per workgroup
                                          (50, 32, 256, 1500, 0.2), (3, 32, 7168, 90, 0.0)])
def test_combine(T, K, h, R, drop):
    banner(f"combine T={T} K={K} h={h}")
    _check_combine(T, K, h, R, drop, seed=T + h)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_combine_on_workload_routing(cid):
    """Combine with the workload's own routing and oracle expert outputs."""
    banner(f"combine config {cid}")
    inp = device_inputs(cid, with_experts=cid in (3, 4))
    idx, gate, cap, sl = _oracle_dispatch(inp)
    cfg = inp.cfg
    R = max(sl["R"], 1)
    rng = np.random.default_rng(cid)
    Y = rng.standard_normal((R, cfg.h)).astype(np.float32)  # stands in for expert outputs
    mc = M.MoeCfg.make(cfg.T, cfg.h, cfg.E, cfg.K, cfg.F, cfg.dtype, cfg.cf)
    out = torch.empty((cfg.T, cfg.h), device="cuda")
    M.moe_combine(mc, to_dev(Y, torch.float32), to_dev(sl["route_row"], torch.int32),
                  to_dev(gate, torch.float32), out)
    torch.cuda.synchronize()
    want = O.combine(Y, sl["route_row"], gate)
    got = out.cpu().numpy()
    mag = np.zeros_like(want)
    for k in range(cfg.K):
        m = sl["route_row"][:, k] >= 0
        mag[m] += np.abs(gate[m, k][:, None].astype(np.float64) * Y[sl["route_row"][m, k]])
    assert np.all(np.abs(got - want) <= (cfg.K + 1) * U32 * mag + 1e-30)

"""FP8 (E4M3) dispatch payload on the GPU vs the oracle: the per-tensor scale,
the quantising dispatch, the receiver's dequantisation (all bit-exact), and
the whole layer fed the dequantised rows (same tolerance as the bf16 layer).
"""
import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
import moe_workloads as W
import oracle as O
from expert_dispatch_combine_amd.runner import LayerBuffers, pack_weights, run_combine, run_ffn
from gpu_util import (banner, bias_np, check_ffn_segment, custom_inputs, device_inputs, host,
                      host_expert, oracle_logits, rms)

pytestmark = pytest.mark.gpu


def _mc(cfg):
    return M.MoeCfg.make(cfg.T, cfg.h, cfg.E, cfg.K, cfg.F, cfg.dtype, cfg.cf)


def _gpu_scale(mc, x):
    scale = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    ws = torch.empty((M.moe_workspace_bytes(mc),), dtype=torch.uint8, device="cuda")
    M.moe_fp8_scale(mc, x, scale, ws)
    torch.cuda.synchronize()
    return float(scale.item()), ws


def _fp8_dispatch(inp, idx, cap, sentinel=0xAB):
    cfg = inp.cfg
    mc = _mc(cfg)
    scale_v, ws = _gpu_scale(mc, inp.x)
    scale = torch.tensor([scale_v], dtype=torch.float32, device="cuda")
    rmax = M.moe_max_rows(mc, cap)
    b = LayerBuffers(mc, cap)
    xq = torch.full((max(rmax, 1), cfg.h), sentinel, dtype=torch.uint8, device="cuda")
    M.moe_dispatch_fp8(mc, inp.x, scale, torch.from_numpy(idx).cuda(), cap, b.expert_offsets,
                       b.route_rank, b.route_row, b.row_token, xq, b.expert_load, ws)
    torch.cuda.synchronize()
    return mc, b, scale, scale_v, xq


@pytest.mark.parametrize("cid", [1, 2, 5])
def test_fp8_scale_bit_exact(cid):
    banner(f"fp8 scale config {cid}")
    inp = device_inputs(cid, with_experts=False)
    if inp.cfg.dtype != "bf16":
        mc = _mc(inp.cfg)
        ws = torch.empty((M.moe_workspace_bytes(mc),), dtype=torch.uint8, device="cuda")
        with pytest.raises(M.MoeError):
            M.moe_fp8_scale(mc, inp.x, torch.empty(1, device="cuda"), ws)
        return
    got, _ = _gpu_scale(_mc(inp.cfg), inp.x)
    assert got == O.fp8_scale(host(inp.x))


@pytest.mark.parametrize("T,h,mag", [(1, 64, 1.0), (37, 128, 1e-4), (500, 192, 250.0),
                                     (4096, 64, 1.0)])
def test_fp8_scale_and_codes_random(T, h, mag):
    """Magnitudes from the E4M3 subnormal range to large values, one odd-sized
    batch; every dispatched code bit-exact (dropless, K = 1, E = 2)."""
    banner(f"fp8 random T={T} h={h} mag={mag}")
    cfg = W.custom(T=T, h=h, E=2, K=1, F=64, cf=2.0, dtype="bf16", seed=T + h)
    inp = custom_inputs(cfg, with_experts=False)
    inp.x.mul_(mag)
    x64 = host(inp.x)
    rng = np.random.default_rng(T)
    idx = rng.integers(0, 2, (T, 1)).astype(np.int32)
    cap = T
    mc, b, scale, scale_v, xq = _fp8_dispatch(inp, idx, cap)
    assert scale_v == O.fp8_scale(x64)
    sl = O.slot_routes(idx, 2, cap)
    R = sl["R"]
    want = O.fp8_quantize(x64[sl["row_token"]], scale_v)
    assert np.array_equal(xq[:R].cpu().numpy(), want)


def test_fp8_codes_beyond_the_format_with_a_caller_scale():
    """A caller-supplied scale four times below max|x| / 448: within one
    16-byte vector some quotients exceed the E4M3 range (NaN code beyond 464,
    448 up to it) and others do not, so the quantiser's out-of-range path and
    its ordinary path meet in the same vectors; every code bit-exact."""
    banner("fp8 caller scale below the amax")
    T, h = 300, 256
    cfg = W.custom(T=T, h=h, E=2, K=1, F=64, cf=2.0, dtype="bf16", seed=41)
    inp = custom_inputs(cfg, with_experts=False)
    x64 = host(inp.x)
    scale_v = O.fp8_scale(x64) / 4.0  # a power-of-two factor: still a bf16 value
    assert scale_v > 0.0 and np.abs(x64 / scale_v).max() > 464.0
    idx = np.random.default_rng(41).integers(0, 2, (T, 1)).astype(np.int32)
    mc = _mc(cfg)
    b = LayerBuffers(mc, T)
    ws = torch.empty((M.moe_workspace_bytes(mc),), dtype=torch.uint8, device="cuda")
    scale = torch.tensor([scale_v], dtype=torch.float32, device="cuda")
    xq = torch.full((max(M.moe_max_rows(mc, T), 1), h), 0xAB, dtype=torch.uint8, device="cuda")
    M.moe_dispatch_fp8(mc, inp.x, scale, torch.from_numpy(idx).cuda(), T, b.expert_offsets,
                       b.route_rank, b.route_row, b.row_token, xq, b.expert_load, ws)
    torch.cuda.synchronize()
    sl = O.slot_routes(idx, 2, T)
    R = sl["R"]
    want = O.fp8_quantize(x64[sl["row_token"]], scale_v)
    assert np.any((want & 0x7F) == 0x7F) and np.any((want & 0x7F) < 0x7F)
    assert np.array_equal(xq[:R].cpu().numpy(), want)


@pytest.mark.parametrize("peak", [448.0, 300.0, 1e-3])
def test_fp8_codes_of_every_bf16_value(peak):
    """The activations hold every finite bf16 value with |v| <= peak (and
    zeros to fill the last row): peak 448 makes the scale exactly 1, so every
    bf16 value up to 448 meets the E4M3 encoding; 300 makes a scale of
    0.66796875, so every pattern goes through the quotient by the scale and
    its rounding to bf16; 1e-3 reaches the bf16 subnormals.  Every code
    bit-exact against the oracle."""
    banner(f"fp8 every bf16 value, peak {peak}")
    pat = np.arange(0, 0x7F80, dtype=np.uint32)          # finite, non-negative bf16 patterns
    vals = (pat << 16).view(np.float32)
    pat = pat[np.abs(vals) <= peak].astype(np.uint16)
    allp = np.concatenate([pat, pat | np.uint16(0x8000)])  # both signs
    h = 256
    T = (allp.size + h - 1) // h
    pad = np.zeros(T * h, np.uint16)
    pad[:allp.size] = allp
    cfg = W.custom(T=T, h=h, E=2, K=1, F=64, cf=2.0, dtype="bf16", seed=11)
    inp = custom_inputs(cfg, with_experts=False)
    inp.x.copy_(torch.from_numpy(pad.view(np.int16).reshape(T, h)).view(torch.bfloat16).cuda())
    x64 = host(inp.x)
    assert float(np.abs(x64).max()) <= peak
    idx = np.random.default_rng(int(peak * 7) % 1000).integers(0, 2, (T, 1)).astype(np.int32)
    mc, b, scale, scale_v, xq = _fp8_dispatch(inp, idx, T)
    assert scale_v == O.fp8_scale(x64)
    sl = O.slot_routes(idx, 2, T)
    want = O.fp8_quantize(x64[sl["row_token"]], scale_v)
    assert np.array_equal(xq[:sl["R"]].cpu().numpy(), want)


@pytest.mark.parametrize("cid", [2, 5])
def test_dispatch_fp8_on_workloads(cid):
    """Routing outputs equal the bf16 dispatch's (and the oracle's); codes of
    every accepted row (workload 2) or of sampled rows (workload 5) equal
    the oracle's; rows beyond R are untouched."""
    banner(f"dispatch fp8 config {cid}")
    inp = device_inputs(cid, with_experts=False)
    cfg = inp.cfg
    logits = oracle_logits(inp)
    idx, _ = O.topk_softmax(logits, cfg.K, bias_np(inp))
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    sl = O.slot_routes(idx, cfg.E, cap)
    mc, b, scale, scale_v, xq = _fp8_dispatch(inp, idx.astype(np.int32), cap)
    assert np.array_equal(b.expert_offsets.cpu().numpy(), sl["expert_offsets"])
    assert np.array_equal(b.route_row.cpu().numpy(), sl["route_row"])
    assert np.array_equal(b.route_rank.cpu().numpy(), sl["route_rank"])
    R = sl["R"]
    assert np.array_equal(b.row_token[:R].cpu().numpy(), sl["row_token"][:R])
    x64 = host(inp.x)
    rows = np.arange(R)
    if cid == 5:
        rows = np.unique(np.concatenate([np.random.default_rng(5).integers(0, R, 384),
                                         [0, R - 1]]))
    want = O.fp8_quantize(x64[sl["row_token"][rows]], scale_v)
    got = xq[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(got, want)
    if R < xq.shape[0]:
        assert bool((xq[R:] == 0xAB).all())


@pytest.mark.parametrize("cid", [2, 5])
def test_fp8_dequantize_bit_exact(cid):
    banner(f"fp8 dequantize config {cid}")
    inp = device_inputs(cid, with_experts=False)
    cfg = inp.cfg
    logits = oracle_logits(inp)
    idx, _ = O.topk_softmax(logits, cfg.K, bias_np(inp))
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    mc, b, scale, scale_v, xq = _fp8_dispatch(inp, idx.astype(np.int32), cap)
    R = int(b.expert_offsets[-1].item())
    b.x_disp.fill_(3.0)
    M.moe_fp8_dequantize(mc, cap, xq, scale, b.expert_offsets, b.x_disp)
    torch.cuda.synchronize()
    rows = np.arange(R) if cid == 2 else np.random.default_rng(7).integers(0, R, 512)
    codes = xq[torch.from_numpy(rows).cuda()].cpu().numpy()
    want = O.fp8_dequantize(codes, scale_v)
    got = b.x_disp[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    assert np.array_equal(got, want)
    if R < b.x_disp.shape[0]:
        assert bool((b.x_disp[R:] == 3.0).all())


def test_fp8_all_zero_activations():
    banner("fp8 zero input")
    cfg = W.custom(T=64, h=64, E=4, K=2, F=64, cf=1.0, dtype="bf16", seed=3)
    inp = custom_inputs(cfg, with_experts=False)
    inp.x.zero_()
    idx = np.stack([np.arange(64) % 4, (np.arange(64) + 1) % 4], 1).astype(np.int32)
    cap = O.capacity(128, 4, 1.0)
    mc, b, scale, scale_v, xq = _fp8_dispatch(inp, idx, cap)
    assert scale_v == 0.0
    R = int(b.expert_offsets[-1].item())
    assert not bool(xq[:R].any())
    M.moe_fp8_dequantize(mc, cap, xq, scale, b.expert_offsets, b.x_disp)
    torch.cuda.synchronize()
    assert not bool(b.x_disp[:R].float().abs().sum().item())


def test_fp8_layer_end_to_end():
    """Workload 2 with the FP8 payload: shared logits give identical routing;
    the experts get the dequantised rows; every token's output within
    2e-2 RMS of the oracle layer run on the same dequantised rows."""
    banner("fp8 layer end to end")
    inp = device_inputs(2)
    cfg = inp.cfg
    logits = oracle_logits(inp)
    idx, gate = O.topk_softmax(logits, cfg.K, bias_np(inp))
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    sl = O.slot_routes(idx, cfg.E, cap)
    mc, b, scale, scale_v, xq = _fp8_dispatch(inp, idx.astype(np.int32), cap)
    M.moe_fp8_dequantize(mc, cap, xq, scale, b.expert_offsets, b.x_disp)
    b.topk_gate.copy_(torch.from_numpy(gate))
    run_ffn(b, inp.w1, inp.b1, inp.w2, inp.b2)
    run_combine(b)
    torch.cuda.synchronize()
    got = b.out.cpu().numpy().astype(np.float64)
    x64 = host(inp.x)
    xd = O.fp8_dequantize(O.fp8_quantize(x64[sl["row_token"]], scale_v), scale_v)
    _, Y = O.expert_ffn(xd, sl["expert_offsets"], host(inp.w1), host(inp.b1), host(inp.w2),
                        host(inp.b2), "bf16")
    want = O.combine(Y, sl["route_row"], gate)
    assert np.max(np.abs(got - want)) <= 2e-2 * rms(want)
    # and the FP8 payload stays close to the bf16 layer (quantisation error only)
    xd16 = x64[sl["row_token"]]
    _, Y16 = O.expert_ffn(xd16, sl["expert_offsets"], host(inp.w1), host(inp.b1), host(inp.w2),
                          host(inp.b2), "bf16")
    assert rms(want - O.combine(Y16, sl["route_row"], gate)) <= 0.1 * rms(want)


@pytest.mark.parametrize("cid,shape,packed", [
    (2, None, True), (2, None, False),                 # streaming, one row tile per expert
    (4, None, True),                                   # streaming, 128-row tiles, 256 experts
    (5, None, True),                                   # weights in registers, partial tile
    (5, None, False),                                  # wide 128 x 128 (hot experts)
    (None, (4096, 256, 4, 1, 512, 1.0), True),         # weights in registers
    (None, (4096, 256, 4, 1, 512, 1.0), False),        # wide 256 x 256 first GEMM
    (None, (1800, 128, 4, 1, 384, 1.3), True),         # wide 128 x 128, 450-row experts
    (None, (4096, 256, 16, 1, 4096, 1.25), True),      # two weight strips per wave, tile search
    (None, (4096, 256, 4, 1, 192, 1.0), True),         # weights in registers, F = 192
    (None, (1000, 256, 4, 1, 320, 1.0), False),        # streaming with the tile search
    (None, (513, 64, 64, 6, 128, 1.0), True)])         # many small / empty experts
def test_fp8_ffn_equals_ffn_on_dequantised_rows(cid, shape, packed):
    """moe_expert_ffn_fp8 (the first GEMM widens the E4M3 codes itself)
    gives the same H and Y, bit for bit, as moe_expert_ffn(_packed) on the
    rows moe_fp8_dequantize writes."""
    banner(f"fp8 ffn cid={cid} shape={shape} packed={packed}")
    if cid is not None:
        inp = device_inputs(cid)
    else:
        T, h, E, K, F, cf = shape
        inp = custom_inputs(W.custom(T=T, h=h, E=E, K=K, F=F, cf=cf, dtype="bf16",
                                     seed=T * 5 + F))
    cfg = inp.cfg
    idx, _ = O.topk_softmax(oracle_logits(inp), cfg.K, bias_np(inp))
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    mc, b, scale, scale_v, xq = _fp8_dispatch(inp, idx.astype(np.int32), cap)
    R = int(b.expert_offsets[-1].item())
    M.moe_fp8_dequantize(mc, cap, xq, scale, b.expert_offsets, b.x_disp)
    w1, w2 = (pack_weights(mc, inp.w1, inp.w2) if packed else (inp.w1, inp.w2))
    fn = M.moe_expert_ffn_packed if packed else M.moe_expert_ffn
    fn(mc, cap, b.x_disp, b.expert_offsets, w1, inp.b1, w2, inp.b2, b.h_buf, b.y)
    torch.cuda.synchronize()
    h_ref, y_ref = b.h_buf[:R].clone(), b.y[:R].clone()
    b.h_buf.fill_(7.0)
    b.y.fill_(float("nan"))
    M.moe_expert_ffn_fp8(mc, cap, xq, scale, b.expert_offsets, w1, inp.b1, w2, inp.b2, b.h_buf,
                         b.y, packed)
    torch.cuda.synchronize()
    assert torch.equal(b.h_buf[:R], h_ref)
    assert torch.equal(b.y[:R], y_ref)


@pytest.mark.parametrize("cid", [2, 5])
def test_fp8_step_end_to_end(cid):
    """The FP8-payload step on the GPU: moe_route (router product), the
    scale, the quantising dispatch, moe_expert_ffn_fp8 (packed weights) and
    the combine, against the oracle fed the same routing (the GPU's ids and
    gates: their own parity is checked elsewhere): every accepted row's H and
    Y against O.expert_ffn_segment on the dequantised rows, and every token's
    output within 2e-2 RMS of the oracle's combine."""
    banner(f"fp8 step config {cid}")
    inp = device_inputs(cid)
    cfg = inp.cfg
    mc = _mc(cfg)
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    b = LayerBuffers(mc, cap)
    M.moe_route(mc, inp.x, inp.w_gate, inp.logit_bias, b.logits, b.topk_idx, b.topk_gate, None,
                b.ws)
    scale = torch.zeros((1,), dtype=torch.float32, device="cuda")
    M.moe_fp8_scale(mc, inp.x, scale, b.ws)
    xq = torch.empty((max(b.r_max, 1), cfg.h), dtype=torch.uint8, device="cuda")
    M.moe_dispatch_fp8(mc, inp.x, scale, b.topk_idx, cap, b.expert_offsets, b.route_rank,
                       b.route_row, b.row_token, xq, None, b.ws)
    w1, w2 = pack_weights(mc, inp.w1, inp.w2)
    M.moe_expert_ffn_fp8(mc, cap, xq, scale, b.expert_offsets, w1, inp.b1, w2, inp.b2, b.h_buf,
                         b.y, True)
    run_combine(b)
    torch.cuda.synchronize()
    del w1, w2
    scale_v = float(scale.item())
    x64 = host(inp.x)
    assert scale_v == O.fp8_scale(x64)
    idx = b.topk_idx.cpu().numpy()
    gate = b.topk_gate.cpu().numpy()
    sl = O.slot_routes(idx, cfg.E, cap)
    assert np.array_equal(b.route_row.cpu().numpy(), sl["route_row"])
    R = sl["R"]
    xd = O.fp8_dequantize(O.fp8_quantize(x64[sl["row_token"]], scale_v), scale_v)
    H_g = b.h_buf[:R].float().cpu().numpy().astype(np.float64)
    Y_g = b.y[:R].cpu().numpy().astype(np.float64)
    offs = sl["expert_offsets"]
    Y_o = np.zeros((R, cfg.h))
    for e in range(cfg.E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            Y_o[lo:hi] = check_ffn_segment("bf16", xd[lo:hi], host_expert(inp.w1, e),
                                           host_expert(inp.b1, e), host_expert(inp.w2, e),
                                           host_expert(inp.b2, e), H_g[lo:hi], Y_g[lo:hi])
    want = O.combine(Y_o, sl["route_row"], gate)
    got = b.out.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - want)) <= 2e-2 * rms(want)


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_ffn_widens_every_code(packed):
    """Dispatched rows made of every finite E4M3 code (all 254 of them, both
    signs, subnormals included), in several orders and scales: the first
    GEMM's in-register widening gives the H and Y of the bf16 FFN on the rows
    that moe_fp8_dequantize writes, bit for bit."""
    banner(f"fp8 every code packed={packed}")
    cfg = W.custom(T=96, h=256, E=3, K=1, F=128, cf=1.0, dtype="bf16", seed=77)
    inp = custom_inputs(cfg)
    mc = _mc(cfg)
    cap = O.capacity(cfg.T, cfg.E, cfg.cf)
    b = LayerBuffers(mc, cap)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] + [0, 0x80], np.uint8)
    rng = np.random.default_rng(78)
    rows = np.stack([rng.permutation(codes) for _ in range(cfg.T)])
    xq = torch.from_numpy(rows).cuda()
    idx = (np.arange(cfg.T) % cfg.E).astype(np.int32)[:, None]
    M.moe_dispatch(mc, None, torch.from_numpy(idx).cuda(), cap, b.expert_offsets, b.route_rank,
                   b.route_row, b.row_token, None, None, b.ws)
    w1, w2 = (pack_weights(mc, inp.w1, inp.w2) if packed else (inp.w1, inp.w2))
    fn = M.moe_expert_ffn_packed if packed else M.moe_expert_ffn
    for scale_v in (1.0, 2.0 ** -9, 0.0078125 * 3):
        scale = torch.tensor([scale_v], dtype=torch.float32, device="cuda")
        M.moe_fp8_dequantize(mc, cap, xq, scale, b.expert_offsets, b.x_disp)
        torch.cuda.synchronize()
        assert np.array_equal(b.x_disp[:cfg.T].double().cpu().numpy(),
                              O.fp8_dequantize(rows, scale_v))
        fn(mc, cap, b.x_disp, b.expert_offsets, w1, inp.b1, w2, inp.b2, b.h_buf, b.y)
        torch.cuda.synchronize()
        h_ref, y_ref = b.h_buf[:cfg.T].clone(), b.y[:cfg.T].clone()
        b.h_buf.fill_(7.0)
        M.moe_expert_ffn_fp8(mc, cap, xq, scale, b.expert_offsets, w1, inp.b1, w2, inp.b2,
                             b.h_buf, b.y, packed)
        torch.cuda.synchronize()
        assert torch.equal(b.h_buf[:cfg.T], h_ref) and torch.equal(b.y[:cfg.T], y_ref)

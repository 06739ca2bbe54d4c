"""moe_route on the GPU vs the oracle.

Shared-logits mode (x = NULL): the oracle's fp32 logits are fed to both sides;
expert ids and loads must be bit-exact, gates within 1e-5 relative.
Product mode (x given): logits within the fp32 accumulation bound; routing
identical except on near-tie tokens."""
import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
import moe_workloads as W
import oracle as O
from expert_dispatch_combine_amd.runner import LayerBuffers, capacity_of, cfg_from
from gpu_util import (banner, bias_np, buffers_for, custom_inputs, device_inputs, host,
                      logit_bound, near_tie_tokens, oracle_logits, to_dev)

pytestmark = pytest.mark.gpu

GATE_RTOL = 1e-5


def _route_logits_in(cfg: W.Config, logits32: np.ndarray, bias):
    b = buffers_for(cfg)
    b.logits.copy_(torch.from_numpy(logits32))
    bias_d = None if bias is None else to_dev(bias, torch.float32)
    M.moe_route(b.cfg, None, None, bias_d, b.logits, b.topk_idx, b.topk_gate, b.expert_load,
                b.ws)
    torch.cuda.synchronize()
    return b.topk_idx.cpu().numpy(), b.topk_gate.cpu().numpy(), b.expert_load.cpu().numpy()


def _assert_route_equal(cfg, logits32, bias):
    idx_o, gate_o = O.topk_softmax(logits32, cfg.K, bias)
    idx_g, gate_g, load_g = _route_logits_in(cfg, logits32, bias)
    assert np.array_equal(idx_g, idx_o)
    np.testing.assert_allclose(gate_g, gate_o, rtol=GATE_RTOL, atol=1e-30)
    assert np.array_equal(load_g.astype(np.int64), O.expert_loads(idx_o, cfg.E))


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_shared_logits_bit_exact(cid):
    banner(f"route shared-logits config {cid}")
    inp = device_inputs(cid, with_experts=cid in (3, 4))
    logits = oracle_logits(inp)
    _assert_route_equal(inp.cfg, logits, bias_np(inp))


@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (17, 3, 2), (300, 4, 4), (129, 8, 8), (77, 33, 5),
                                   (513, 64, 6), (100, 100, 32), (64, 256, 8), (33, 1000, 3),
                                   (70, 1024, 1), (257, 16, 16), (5, 5, 5), (64, 1024, 32)])
def test_tie_heavy_integer_logits(T, E, K):
    banner(f"route ties T={T} E={E} K={K}")
    rng = np.random.default_rng(T * 131 + E)
    logits = rng.integers(-3, 4, (T, E)).astype(np.float32)
    logits[rng.random(logits.shape) < 0.2] = -0.0
    cfg = W.custom(T=T, h=64, E=E, K=K, F=64, dtype="f32")
    _assert_route_equal(cfg, logits, None)
    bias = rng.integers(-1, 2, E).astype(np.float32) * 0.5
    _assert_route_equal(cfg, logits, bias)


def test_wide_logit_spread_and_k_equals_e():
    banner("route wide spread")
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((200, 12)) * 30).astype(np.float32)
    cfg = W.custom(T=200, h=64, E=12, K=12, F=64, dtype="f32")
    _assert_route_equal(cfg, logits, None)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_router_product_and_routing(cid):
    """x given: the GPU computes the logits itself (bf16 MFMA / fp32 FMA)."""
    banner(f"route product config {cid}")
    inp = device_inputs(cid, with_experts=cid in (3, 4))
    cfg = inp.cfg
    x64, wg64 = host(inp.x), host(inp.w_gate)
    logits_o = O.router_logits(x64, wg64)
    b = buffers_for(cfg)
    M.moe_route(b.cfg, inp.x, inp.w_gate, inp.logit_bias, b.logits, b.topk_idx, b.topk_gate,
                b.expert_load, b.ws)
    torch.cuda.synchronize()
    lg = b.logits.cpu().numpy().astype(np.float64)
    err = np.abs(lg - (x64 @ wg64.T))
    bound = logit_bound(x64, wg64)
    assert np.all(err <= bound + 1e-30), float((err - bound).max())
    assert err.max() <= 1e-4, float(err.max())
    bias = bias_np(inp)
    idx_o, gate_o = O.topk_softmax(logits_o, cfg.K, bias)
    idx_g = b.topk_idx.cpu().numpy()
    gate_g = b.topk_gate.cpu().numpy()
    tie = near_tie_tokens(logits_o, bias, cfg.K)
    same = np.all(idx_g == idx_o, axis=1)
    assert np.all(same | tie), np.nonzero(~(same | tie))[0][:10]
    # gate error follows the logit error: |d log g| <= 2 max |d logit|
    tol = 2.0 * float(err.max()) + 2 * GATE_RTOL
    m = same & ~tie
    np.testing.assert_allclose(gate_g[m], gate_o[m], rtol=tol, atol=1e-30)
    # histogram of the GPU's own ids
    assert np.array_equal(b.expert_load.cpu().numpy().astype(np.int64),
                          np.bincount(idx_g.reshape(-1), minlength=cfg.E))


@pytest.mark.parametrize("T,h,E,K", [(1, 64, 4, 2), (37, 128, 16, 1), (300, 192, 64, 6),
                                     (70, 256, 100, 3), (33, 64, 300, 8)])
def test_router_product_ragged_shapes(T, h, E, K):
    banner(f"route product T={T} h={h} E={E} K={K}")
    cfg = W.custom(T=T, h=h, E=E, K=K, F=64, dtype="bf16", seed=T + E)
    inp = custom_inputs(cfg, with_experts=False)
    x64, wg64 = host(inp.x), host(inp.w_gate)
    b = buffers_for(cfg)
    M.moe_route(b.cfg, inp.x, inp.w_gate, None, b.logits, b.topk_idx, b.topk_gate, None, b.ws)
    torch.cuda.synchronize()
    lg = b.logits.cpu().numpy().astype(np.float64)
    err = np.abs(lg - (x64 @ wg64.T))
    assert np.all(err <= logit_bound(x64, wg64) + 1e-30)
    logits_o = O.router_logits(x64, wg64)
    idx_o, _ = O.topk_softmax(logits_o, K)
    tie = near_tie_tokens(logits_o, None, K)
    same = np.all(b.topk_idx.cpu().numpy() == idx_o, axis=1)
    assert np.all(same | tie)


@pytest.mark.parametrize("T,h,E,K,ws", [
    (16390, 128, 64, 6, True),     # 64-token x 64-expert tiles, fused top-k, ragged T
    (16400, 128, 50, 3, True),     # fused top-k on 4-lane groups (K <= 4)
    (16500, 64, 48, 12, True),     # fused top-k on 16-lane groups (8 < K <= 16)
    (16400, 64, 20, 2, True),      # 128 x 32 tiles, E not a multiple of 4
    (300, 512, 32, 20, True),      # K > 16: tiled product, 8 h ranges, separate top-k
    (257, 1024, 256, 8, True),     # 128 x 128 tiles, two expert tiles, 8 h ranges summed
    (257, 1024, 256, 8, False),    # same without workspace: one h range
    (130, 192, 1001, 4, True),     # eight expert tiles, odd E, h not splittable
    (1000, 448, 130, 3, True),     # E just above one 128-expert tile
    (90, 256, 100, 5, True),       # 64 x 128 tiles, 4 h ranges
    (300, 512, 1024, 32, True),    # E = 1024 and K = 32, the library's limits
])
def test_router_tiled_shapes(T, h, E, K, ws):
    """The tiled router product (long batches or E > 64) on shapes that
    exercise each tile shape, the h split with its partial sums, ragged token
    and expert tiles, and the fused and separate top-k; the bias and the
    expert histogram ride along."""
    banner(f"route tiled T={T} h={h} E={E} K={K} ws={ws}")
    cfg = W.custom(T=T, h=h, E=E, K=K, F=64, dtype="bf16", seed=T * 7 + E)
    inp = custom_inputs(cfg, with_experts=False)
    x64, wg64 = host(inp.x), host(inp.w_gate)
    rng = np.random.default_rng(E + K)
    bias = (rng.standard_normal(E) * 0.01).astype(np.float32)
    b = buffers_for(cfg)
    b.logits.fill_(float("nan"))
    M.moe_route(b.cfg, inp.x, inp.w_gate, to_dev(bias, torch.float32), b.logits, b.topk_idx,
                b.topk_gate, b.expert_load, b.ws if ws else None)
    torch.cuda.synchronize()
    lg = b.logits.cpu().numpy().astype(np.float64)
    ref = x64 @ wg64.T
    err = np.abs(lg - ref)
    assert np.all(err <= logit_bound(x64, wg64) + 1e-30), float(np.nanmax(err))
    logits_o = O.router_logits(x64, wg64)
    idx_o, gate_o = O.topk_softmax(logits_o, K, bias)
    idx_g = b.topk_idx.cpu().numpy()
    gate_g = b.topk_gate.cpu().numpy()
    tie = near_tie_tokens(logits_o, bias, K)
    same = np.all(idx_g == idx_o, axis=1)
    assert np.all(same | tie), np.nonzero(~(same | tie))[0][:10]
    # most tokens are compared: each of the K gaps among a token's top K + 1
    # logits may fall under the tie threshold, so the excluded share grows with K
    assert tie.mean() < 0.05 * max(1.0, K / 8)
    m = same & ~tie
    tol = 2.0 * float(err.max()) + 2 * GATE_RTOL
    np.testing.assert_allclose(gate_g[m], gate_o[m], rtol=tol, atol=1e-30)
    # every token's ids are distinct and in range; the histogram is of the GPU's ids
    assert idx_g.min() >= 0 and idx_g.max() < E
    assert np.all(np.sort(idx_g, axis=1)[:, 1:] != np.sort(idx_g, axis=1)[:, :-1])
    assert np.array_equal(b.expert_load.cpu().numpy().astype(np.int64),
                          np.bincount(idx_g.reshape(-1), minlength=E))


def test_router_tiled_is_deterministic():
    """Two calls on the same inputs give the same bits (fixed summation order
    of the h ranges; no atomics on values)."""
    banner("route tiled determinism")
    cfg = W.custom(T=1024, h=1024, E=256, K=8, F=64, dtype="bf16", seed=5)
    inp = custom_inputs(cfg, with_experts=False)
    outs = []
    for _ in range(2):
        b = buffers_for(cfg)
        M.moe_route(b.cfg, inp.x, inp.w_gate, None, b.logits, b.topk_idx, b.topk_gate, None,
                    b.ws)
        torch.cuda.synchronize()
        outs.append((b.logits.cpu().numpy().copy(), b.topk_idx.cpu().numpy().copy(),
                     b.topk_gate.cpu().numpy().copy()))
    for a, c in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              c.view(np.uint32) if c.dtype == np.float32 else c)

"""Aux-loss-free balancing on the GPU vs the oracle: moe_bias_update and the
dropless dispatch.

Routing is made on shared fp32 logits (moe_route with x = NULL), so the
argmax counts and every bias value must be bit-exact: the update is the
page's fp32 arithmetic with one rounding per operation on both sides."""
import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
import moe_workloads as W
import oracle as O
from gpu_util import banner, bias_np, buffers_for, device_inputs, oracle_logits, to_dev

pytestmark = pytest.mark.gpu


def _gpu_step(b, logits32, bias_d, alpha):
    """route on the shared logits with the current bias, then update it"""
    b.logits.copy_(torch.from_numpy(logits32))
    M.moe_route(b.cfg, None, None, bias_d, b.logits, b.topk_idx, b.topk_gate, None, b.ws)
    counts = torch.empty((b.cfg.E,), dtype=torch.int32, device="cuda")
    M.moe_bias_update(b.cfg, b.topk_idx, bias_d, alpha, counts)
    torch.cuda.synchronize()
    return counts.cpu().numpy().astype(np.int64), bias_d.cpu().numpy()


def _oracle_step(logits32, bias32, alpha):
    counts = O.top1_counts(O.add_logit_bias(logits32, bias32))
    return counts, O.expert_bias_update(bias32, counts, alpha).astype(np.float32)


@pytest.mark.parametrize("T,E,K,alpha", [(1, 1, 1, 0.1), (64, 4, 2, 0.1), (1000, 16, 1, 0.1),
                                         (4096, 256, 8, 0.1), (2049, 64, 6, 1e-3),
                                         (300, 1000, 3, 0.37)])
def test_bias_update_bit_exact(T, E, K, alpha):
    banner(f"bias update T={T} E={E} K={K} alpha={alpha}")
    rng = np.random.default_rng(T + E)
    logits = rng.integers(-3, 4, (T, E)).astype(np.float32)  # ties decided by the id rule
    logits += (rng.standard_normal((T, E)) * (rng.random((T, E)) < 0.5)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
    cfg = W.custom(T=T, h=64, E=E, K=K, F=64, dtype="f32")
    b = buffers_for(cfg)
    bias_d = to_dev(bias, torch.float32)
    counts_g, bias_g = _gpu_step(b, logits, bias_d, alpha)
    counts_o, bias_o = _oracle_step(logits, bias, alpha)
    assert np.array_equal(counts_g, counts_o)
    assert np.array_equal(bias_g.view(np.uint32), bias_o.view(np.uint32))


def test_bias_iterations_follow_the_oracle_and_balance_the_hot_expert_workload():
    """Workload 5's router (logits from its x and W_g, Zipf-skewed): 30
    route -> update steps, bias bit-exact with the oracle after every step,
    and the top-1 loads end near balance."""
    banner("bias iterations, hot-expert workload")
    inp = device_inputs(5, with_experts=False)
    cfg = inp.cfg
    logits = O.add_logit_bias(oracle_logits(inp), bias_np(inp)).astype(np.float32)
    b = buffers_for(cfg)
    bias = np.zeros(cfg.E, np.float32)
    bias_d = to_dev(bias, torch.float32)
    ratios = []
    for step in range(30):
        counts_g, bias_g = _gpu_step(b, logits, bias_d, 1e-3)
        counts_o, bias = _oracle_step(logits, bias, 1e-3)
        assert np.array_equal(counts_g, counts_o), step
        assert np.array_equal(bias_g.view(np.uint32), bias.view(np.uint32)), step
        ratios.append(counts_o.max() / (cfg.T / cfg.E))
    assert ratios[0] > 5.0 and ratios[-1] < 1.3


def test_bias_update_empty_batch_and_invalid_ids():
    banner("bias update empty / invalid ids")
    E = 8
    bias = np.arange(E, dtype=np.float32) * 0.25
    cfg0 = M.MoeCfg.make(0, 64, E, 2, 64, "f32", 1.0)
    bias_d = to_dev(bias, torch.float32)
    M.moe_bias_update(cfg0, None, bias_d, 0.1)
    torch.cuda.synchronize()
    assert np.array_equal(bias_d.cpu().numpy(), bias)  # mean 0, counts 0
    # slot-0 ids outside [0, E) are not counted
    T, K = 40, 2
    rng = np.random.default_rng(5)
    idx = rng.integers(0, E, (T, K)).astype(np.int32)
    idx[::7, 0] = -1
    idx[3::11, 0] = E + 2
    cfg = M.MoeCfg.make(T, 64, E, K, 64, "f32", 1.0)
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    M.moe_bias_update(cfg, to_dev(idx, torch.int32), bias_d, 0.1, counts)
    torch.cuda.synchronize()
    valid = idx[:, 0][(idx[:, 0] >= 0) & (idx[:, 0] < E)]
    want_counts = np.bincount(valid, minlength=E)
    assert np.array_equal(counts.cpu().numpy(), want_counts)
    want = O.expert_bias_update(bias, want_counts, 0.1).astype(np.float32)
    assert np.array_equal(bias_d.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("cid", [2, 5])
def test_dropless_dispatch(cid):
    """capacity = T accepts every route: overflow 0, R = T*K, and the slots
    equal the oracle's capacity loop run with that capacity."""
    banner(f"dropless dispatch config {cid}")
    inp = device_inputs(cid, with_experts=False)
    cfg = inp.cfg
    logits = oracle_logits(inp)
    idx, _ = O.topk_softmax(logits, cfg.K, bias_np(inp))
    cap = cfg.T
    sl = O.slot_routes(idx, cfg.E, cap)
    assert sl["R"] == cfg.T * cfg.K
    mc = M.MoeCfg.make(cfg.T, cfg.h, cfg.E, cfg.K, cfg.F, cfg.dtype, cfg.cf)
    rmax = M.moe_max_rows(mc, cap)
    assert rmax == cfg.T * cfg.K
    dev = lambda a: to_dev(a, torch.int32)  # noqa: E731
    offs = torch.empty((cfg.E + 1,), dtype=torch.int32, device="cuda")
    rank = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda")
    row = torch.empty_like(rank)
    row_token = torch.empty((rmax,), dtype=torch.int32, device="cuda")
    xd = torch.empty((rmax, cfg.h), dtype=inp.x.dtype, device="cuda")
    ws = torch.empty((M.moe_workspace_bytes(mc),), dtype=torch.uint8, device="cuda")
    M.moe_dispatch(mc, inp.x, dev(idx), cap, offs, rank, row, row_token, xd, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(offs.cpu().numpy(), sl["expert_offsets"])
    assert np.array_equal(rank.cpu().numpy(), sl["route_rank"])
    assert np.array_equal(row.cpu().numpy(), sl["route_row"])
    assert np.array_equal(row_token.cpu().numpy(), sl["row_token"])
    assert torch.equal(xd, inp.x[torch.from_numpy(sl["row_token"].astype(np.int64)).cuda()])

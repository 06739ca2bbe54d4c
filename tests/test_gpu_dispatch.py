"""moe_dispatch on the GPU vs the oracle: offsets, ranks, rows, row_token and
the gathered rows must be bit-exact (integer and byte work)."""
import itertools

import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
import moe_workloads as W
import oracle as O
from expert_dispatch_combine_amd.runner import LayerBuffers
from gpu_util import banner, bias_np, buffers_for, custom_inputs, device_inputs, host, to_dev

pytestmark = pytest.mark.gpu


def _dispatch(cfg: W.Config, x: torch.Tensor, idx: np.ndarray, cap: int):
    mc = M.MoeCfg.make(cfg.T, cfg.h, cfg.E, cfg.K, cfg.F, cfg.dtype, cfg.cf)
    b = LayerBuffers(mc, cap)
    b.topk_idx.copy_(torch.from_numpy(idx.astype(np.int32)))
    b.row_token.fill_(-7)
    b.x_disp.view(torch.uint8).fill_(0x5A)  # rows past R must keep this
    M.moe_dispatch(mc, x, b.topk_idx, cap, b.expert_offsets, b.route_rank, b.route_row,
                   b.row_token, b.x_disp, b.expert_load, b.ws)
    torch.cuda.synchronize()
    return b


def _check(cfg, x, idx, cap, check_rows=True):
    sl = O.slot_routes(idx, cfg.E, cap)
    b = _dispatch(cfg, x, idx, cap)
    assert np.array_equal(b.expert_offsets.cpu().numpy(), sl["expert_offsets"])
    assert np.array_equal(b.route_rank.cpu().numpy(), sl["route_rank"])
    assert np.array_equal(b.route_row.cpu().numpy(), sl["route_row"])
    R = sl["R"]
    assert np.array_equal(b.row_token.cpu().numpy()[:R], sl["row_token"])
    assert np.array_equal(b.expert_load.cpu().numpy().astype(np.int64),
                          O.expert_loads(idx, cfg.E))
    if check_rows and R:
        # byte-exact copy: compare the raw bits of the rows
        bits = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
        xd_o = O.dispatch(x.cpu().view(bits).numpy(), sl["row_token"])
        got = b.x_disp[:R].cpu().view(bits).numpy()
        assert np.array_equal(got, xd_o)
    if check_rows:
        # the row copy loads every vector position but stores accepted rows only
        assert bool((b.x_disp[R:].view(torch.uint8) == 0x5A).all())
    return b, sl


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_dispatch_on_workloads(cid):
    banner(f"dispatch config {cid}")
    inp = device_inputs(cid, with_experts=cid in (3, 4))
    cfg = inp.cfg
    logits = O.router_logits(host(inp.x), host(inp.w_gate))
    idx, _ = O.topk_softmax(logits, cfg.K, bias_np(inp))
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    _check(cfg, inp.x, idx, cap)


@pytest.mark.parametrize("T,E,K,cf,dtype", [(2048, 16, 1, 1.25, "bf16"), (9000, 64, 2, 1.0, "bf16"),
                                            (300, 5, 2, 0.7, "f32")])
def test_dispatch_metadata_only(T, E, K, cf, dtype):
    """x_disp = NULL (and x = NULL): the same offsets, ranks, rows, row_token and
    loads, no row moved -- the one-launch path (<= 8192 routes) and the
    three-kernel path."""
    banner(f"dispatch metadata only T={T} E={E} K={K}")
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    cfg = W.custom(T=T, h=64, E=E, K=K, F=64, cf=cf, dtype=dtype)
    cap = O.capacity(T * K, E, cf)
    sl = O.slot_routes(idx, E, cap)
    mc = M.MoeCfg.make(T, 64, E, K, 64, dtype, cf)
    b = LayerBuffers(mc, cap)
    b.topk_idx.copy_(torch.from_numpy(idx))
    b.row_token.fill_(-7)
    sentinel = b.x_disp.view(torch.uint8).fill_(0x5A).clone()
    M.moe_dispatch(mc, None, b.topk_idx, cap, b.expert_offsets, b.route_rank, b.route_row,
                   b.row_token, None, b.expert_load, b.ws)
    torch.cuda.synchronize()
    assert np.array_equal(b.expert_offsets.cpu().numpy(), sl["expert_offsets"])
    assert np.array_equal(b.route_rank.cpu().numpy(), sl["route_rank"])
    assert np.array_equal(b.route_row.cpu().numpy(), sl["route_row"])
    assert np.array_equal(b.row_token.cpu().numpy()[:sl["R"]], sl["row_token"])
    assert np.array_equal(b.expert_load.cpu().numpy().astype(np.int64), O.expert_loads(idx, E))
    assert torch.equal(b.x_disp.view(torch.uint8), sentinel)


def _random_idx(rng, T, E, K):
    return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, K), np.int32)


@pytest.mark.parametrize("T,E,K,cf", [(1, 1, 1, 1.0), (3, 2, 2, 1.0), (300, 5, 2, 0.7),
                                      (1025, 8, 3, 1.0), (2049, 64, 6, 1.0), (777, 256, 8, 1.3),
                                      (4000, 1000, 4, 1.0), (1500, 3, 1, 0.2), (64, 7, 7, 1.0),
                                      # the library's limits, E = 1024 and K = 32: one launch
                                      # (6400 routes) and three kernels with drops (48000)
                                      (200, 1024, 32, 1.0), (1500, 1024, 32, 0.5),
                                      # 141 route blocks at E = 64: each of an expert's four
                                      # column readers sums its blocks in two batches
                                      (24000, 64, 6, 1.0)])
def test_dispatch_random_routings(T, E, K, cf):
    banner(f"dispatch random T={T} E={E} K={K} cf={cf}")
    rng = np.random.default_rng(T + E + K)
    cfg = W.custom(T=T, h=64, E=E, K=K, F=64, cf=cf, dtype="bf16", seed=T)
    inp = custom_inputs(cfg, with_experts=False)
    idx = _random_idx(rng, T, E, K)
    cap = O.capacity(T * K, E, cf)
    _check(cfg, inp.x, idx, cap)


@pytest.mark.parametrize("cap", [0, 1, 5, 10 ** 6])
def test_dispatch_capacity_extremes_and_hot_expert(cap):
    banner(f"dispatch hot expert cap={cap}")
    rng = np.random.default_rng(11)
    T, E, K = 3000, 16, 2
    cfg = W.custom(T=T, h=128, E=E, K=K, F=64, dtype="bf16", seed=5)
    inp = custom_inputs(cfg, with_experts=False)
    # every token picks expert 3 first (all tokens -> one expert), then a random other
    idx = np.stack([[3, rng.choice([e for e in range(E) if e != 3])] for _ in range(T)])
    _check(cfg, inp.x, idx.astype(np.int32), cap)


def test_dispatch_fp32_rows_not_multiple_of_16_bytes():
    banner("dispatch fp32 odd h")
    rng = np.random.default_rng(12)
    cfg = W.custom(T=200, h=7, E=5, K=2, F=3, dtype="f32", seed=6)
    inp = custom_inputs(cfg, with_experts=False)
    _check(cfg, inp.x, _random_idx(rng, 200, 5, 2), O.capacity(400, 5, 1.0))


def test_dispatch_brute_force_tiny():
    banner("dispatch brute force")
    cfg = W.custom(T=4, h=64, E=3, K=2, F=64, dtype="bf16", seed=9)
    inp = custom_inputs(cfg, with_experts=False)
    per_token = list(itertools.permutations(range(3), 2))
    n = 0
    for routing in itertools.product(per_token, repeat=4):
        idx = np.array(routing, np.int32)
        for cap in (0, 1, 2, 3, 8):
            _check(cfg, inp.x, idx, cap, check_rows=(cap == 2))
            n += 1
    assert n == 6 ** 4 * 5


def test_dispatch_empty_batch():
    banner("dispatch empty")
    cfg = W.custom(T=0, h=64, E=4, K=2, F=64, dtype="bf16")
    mc = M.MoeCfg.make(0, 64, 4, 2, 64, "bf16", 1.0)
    b = LayerBuffers(mc, 0)
    b.expert_offsets.fill_(-1)
    M.moe_dispatch(mc, None, None, 0, b.expert_offsets, None, None, None, None, b.expert_load,
                   b.ws)
    torch.cuda.synchronize()
    assert b.expert_offsets.cpu().tolist() == [0] * 5
    assert b.expert_load.cpu().tolist() == [0] * 4


def test_dispatch_invalid_ids_are_dropped():
    banner("dispatch invalid ids")
    T, E, K = 50, 4, 2
    cfg = W.custom(T=T, h=64, E=E, K=K, F=64, dtype="bf16", seed=3)
    inp = custom_inputs(cfg, with_experts=False)
    rng = np.random.default_rng(4)
    idx = _random_idx(rng, T, E, K)
    bad = idx.copy()
    bad[5, 1] = E
    bad[9, 0] = -1
    b = _dispatch(cfg, inp.x, bad, 100)
    rr = b.route_row.cpu().numpy()
    assert rr[5, 1] == -1 and rr[9, 0] == -1
    assert b.route_rank.cpu().numpy()[5, 1] == -1
    # the valid routes keep the ranks of the routing without the bad ones
    flat = bad.reshape(-1)
    ranks = b.route_rank.cpu().numpy().reshape(-1)
    for i, e in enumerate(flat):
        if 0 <= e < E:
            assert ranks[i] == int(np.sum(flat[:i] == e))

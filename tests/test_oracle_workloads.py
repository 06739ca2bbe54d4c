"""The oracle on the seeded workloads (CPU): shapes, invariants, and the
properties the workload recipe promises (near-uniform routers, a hot-expert
skew above the max/mean > 2 alarm)."""
import math

import numpy as np
import pytest

import moe_workloads as W
import oracle as O


def _layer(cfg):
    inp = W.make_inputs(cfg, "cpu")
    f = W.host_f64
    h_round = "bf16" if cfg.dtype == "bf16" else "f32"
    L = O.moe_layer(f(inp.x), f(inp.w_gate), f(inp.w1), f(inp.b1), f(inp.w2), f(inp.b2),
                    cfg.K, cfg.cf, logit_bias=None if inp.logit_bias is None
                    else inp.logit_bias.numpy(), h_round=h_round)
    return inp, L


def test_tiny_fp32_layer_invariants():
    cfg = W.CONFIGS[1]
    inp, L = _layer(cfg)
    T, K, E = cfg.T, cfg.K, cfg.E
    assert L["capacity"] == 32
    assert int(L["loads"].sum()) == T * K
    assert L["R"] == int(np.minimum(L["loads"], 32).sum())
    assert L["out"].shape == (T, cfg.h)
    # second formulation
    f = W.host_f64
    out2 = O.moe_layer_per_token(f(inp.x), L["idx"], L["gate"], L["route_row"] >= 0,
                                 f(inp.w1), f(inp.b1), f(inp.w2), f(inp.b2), h_round="f32")
    np.testing.assert_allclose(L["out"], out2, rtol=1e-6, atol=1e-7)
    led = O.ledger(L["idx"], L["gate"], L["route_row"], L["capacity"], inp.src_rank.numpy(),
                   inp.owner_rank.numpy(), cfg.n_ep, cfg.h, cfg.bytes_per_elem)
    assert led["accepted_routes"] == L["R"]
    assert led["local_routes"] + led["cross_rank_routes"] == T * K
    assert math.isclose(led["P"].sum(), 1.0, rel_tol=1e-6)


def test_switch_base_routing_is_near_uniform():
    cfg = W.CONFIGS[2]
    inp = W.make_inputs(cfg, "cpu", with_experts=False)
    logits = O.router_logits(W.host_f64(inp.x), W.host_f64(inp.w_gate))
    idx, gate = O.topk_softmax(logits, cfg.K)
    assert np.all(gate == 1.0)                      # K = 1: the single gate is exactly 1
    loads = O.expert_loads(idx, cfg.E)
    mon = O.load_monitor(loads)
    assert mon["max_over_mean"] < 1.6 and not mon["imbalanced"]
    assert O.capacity(cfg.A, cfg.E, cfg.cf) == 160


@pytest.mark.slow
def test_hot_expert_workload_is_skewed():
    cfg = W.CONFIGS[5]
    inp = W.make_inputs(cfg, "cpu", with_experts=False)
    logits = O.router_logits(W.host_f64(inp.x), W.host_f64(inp.w_gate))
    idx, gate = O.topk_softmax(logits, cfg.K, inp.logit_bias.numpy())
    loads = O.expert_loads(idx, cfg.E)
    cap = O.capacity(cfg.A, cfg.E, cfg.cf)
    mon = O.load_monitor(loads)
    assert mon["imbalanced"] and mon["max_over_mean"] > 2.0
    assert O.overflow(loads, cap) > 0.3 * cfg.A
    src = inp.src_rank.numpy()
    assert src[0] == 0 and src[-1] == cfg.n_ep - 1 and np.all(np.diff(src) >= 0)

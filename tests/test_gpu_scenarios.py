"""The expert-parallel mechanism workload of "46. MoE Expert Parallel" Step 5
(2 ranks x 256 tokens, h 1024, 4 experts, top-2, cf 1.25, bf16) under its
three routing scenarios, through the whole GPU path, vs the oracle.

Routing comes from each scenario's seeded logits (moe_route, logits-in), so
routing, slots and the ledger are bit-exact; the layer output of every token
is within 2e-2 RMS; the plan decision (moe_recommend_plan on the GPU ledger)
equals the oracle's; and each scenario shows what it is meant to show."""
import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
import moe_workloads as W
import oracle as O
from expert_dispatch_combine_amd.runner import (LayerBuffers, capacity_of, cfg_from,
                                                run_combine, run_dispatch, run_ffn, run_ledger)
from gpu_util import banner, host, rms

pytestmark = pytest.mark.gpu

_INPUTS = {}


def _inputs():
    if "x" not in _INPUTS:
        _INPUTS["x"] = W.make_inputs(W.SCENARIO_CONFIG, "cuda")
    return _INPUTS["x"]


@pytest.mark.parametrize("name", W.ROUTING_SCENARIOS)
def test_routing_scenario(name):
    banner(f"routing scenario {name}")
    cfg = W.SCENARIO_CONFIG
    inp = _inputs()
    logits = W.scenario_logits(name)
    mc = cfg_from(cfg)
    b = LayerBuffers(mc, capacity_of(mc))
    b.logits.copy_(torch.from_numpy(logits))
    M.moe_route(mc, None, None, None, b.logits, b.topk_idx, b.topk_gate, None, b.ws)
    run_dispatch(b, inp.x, expert_load=True)
    run_ffn(b, inp.w1, inp.b1, inp.w2, inp.b2)
    run_combine(b)
    led = run_ledger(b, inp.src_rank, inp.owner_rank, cfg.n_ep)
    torch.cuda.synchronize()

    ref = O.moe_layer(host(inp.x), host(inp.w_gate), host(inp.w1), host(inp.b1), host(inp.w2),
                      host(inp.b2), cfg.K, cfg.cf, h_round="bf16", logits32=logits)
    assert np.array_equal(b.topk_idx.cpu().numpy(), ref["idx"])
    assert np.array_equal(b.route_row.cpu().numpy(), ref["route_row"])
    src = inp.src_rank.cpu().numpy()
    owner = inp.owner_rank.cpu().numpy()
    oled = O.ledger(ref["idx"], ref["gate"], ref["route_row"], ref["capacity"], src, owner,
                    cfg.n_ep, hidden_size=cfg.h, bytes_per_elem=2)
    for k in ("total_routes", "overflow", "accepted_routes", "local_routes",
              "cross_rank_routes", "cross_rank_dispatch_bytes", "accepted_local_routes",
              "accepted_cross_rank_routes", "max_load"):
        assert led[k] == oled[k], k
    assert led["balance_ratio"] == oled["balance_ratio"]
    assert led["local_hit_ratio"] == oled["local_hit_ratio"]
    out = b.out.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(out - ref["out"])) <= 2e-2 * rms(ref["out"])

    plan = M.moe_recommend_plan(led)
    assert plan == O.recommend_plan(oled, oled)
    if name == "local_heavy":
        assert led["local_hit_ratio"] > 0.9 and led["overflow"] == 0
    elif name == "balanced":
        assert 0.35 < led["local_hit_ratio"] < 0.65 and plan == "accept"
    else:
        assert led["overflow"] > 0 and led["balance_ratio"] > 1.5 and plan == "reject"

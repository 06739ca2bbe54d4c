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
from gpu_util import banner, compare_ledger, host, rms

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


@pytest.mark.parametrize("loads,cf,want", [([6002, 3998], 1.25, "accept"),
                                           ([9002, 998], 1.8, "tune"),
                                           ([12006, 7994], 1.25, "tune")])
def test_plan_decision_at_the_3_decimal_boundary(loads, cf, want):
    """[EP46] Step 4 / TODO 3: routings whose balance ratio lies just past a
    limit but is stored as round(ratio, 3) on it.  Top-1 routes in a seeded
    order through moe_dispatch, the GPU ledger and moe_recommend_plan decide
    as the oracle (and the page) does."""
    banner(f"plan decision loads={loads} cf={cf}")
    E = len(loads)
    T = sum(loads)
    rng = np.random.default_rng(41)
    ids = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), loads)).reshape(T, 1)
    cfg = W.custom(T, 64, E, 1, 64, cf=cf, n_ep=2)
    mc = cfg_from(cfg)
    b = LayerBuffers(mc, capacity_of(mc))
    b.topk_idx.copy_(torch.from_numpy(ids))
    b.topk_gate.fill_(1.0)
    M.moe_dispatch(mc, None, b.topk_idx, b.capacity, b.expert_offsets, b.route_rank,
                   b.route_row, b.row_token, None, None, b.ws)
    src = torch.from_numpy((np.arange(T) % 2).astype(np.int32)).cuda()
    owner = torch.from_numpy((np.arange(E) % 2).astype(np.int32)).cuda()
    led = run_ledger(b, src, owner, 2)
    torch.cuda.synchronize()
    cap = O.capacity(T, E, cf)
    sl = O.slot_routes(ids, E, cap)
    assert np.array_equal(b.route_row.cpu().numpy(), sl["route_row"])
    oled = O.ledger(ids, np.ones((T, 1)), sl["route_row"], cap, np.arange(T) % 2,
                    np.arange(E) % 2, 2, hidden_size=64, bytes_per_elem=2)
    for k in ("total_routes", "overflow", "accepted_routes", "local_routes",
              "cross_rank_routes", "max_load"):
        assert led[k] == oled[k], k
    assert led["balance_ratio"] == oled["balance_ratio"]
    assert M.moe_recommend_plan(led) == O.recommend_plan(oled, oled) == want


def _placement_case(mc, b, src_rank, n_ep, h, bytes_per_elem):
    """Affinity on the GPU (bit-exact vs the oracle), the host placement (the
    oracle's optimum of local routes, E / n_ep experts per rank), and the
    GPU ledger under that placement against the oracle's ledger of the same
    map.  Returns (round-robin ledger, placed ledger, owner)."""
    E = mc.E
    aff = torch.empty((E, n_ep), dtype=torch.int32, device="cuda")
    M.moe_expert_rank_affinity(mc, b.topk_idx, None, src_rank, n_ep, aff)
    torch.cuda.synchronize()
    idx = b.topk_idx.cpu().numpy()
    src = src_rank.cpu().numpy()
    want = O.expert_rank_affinity(idx, src, E, n_ep)
    aff_h = aff.cpu().numpy()
    assert np.array_equal(aff_h, want)
    row = b.route_row.cpu().numpy()
    aff_acc = torch.empty_like(aff)
    M.moe_expert_rank_affinity(mc, b.topk_idx, b.route_row, src_rank, n_ep, aff_acc)
    torch.cuda.synchronize()
    assert np.array_equal(aff_acc.cpu().numpy(),
                          O.expert_rank_affinity(idx, src, E, n_ep, route_row=row))
    owner = np.asarray(M.moe_place_experts(aff_h, n_ep), np.int32)
    assert sorted(np.bincount(owner, minlength=n_ep).tolist()) == [E // n_ep] * n_ep
    best = O.local_routes_under(want, O.locality_placement(want, n_ep))
    assert O.local_routes_under(want, owner) == best
    rr = np.arange(E, dtype=np.int32) % n_ep
    gate = b.topk_gate.cpu().numpy()
    leds = []
    for own in (rr, owner):
        g = run_ledger(b, src_rank, torch.from_numpy(own).cuda(), n_ep)
        o = O.ledger(idx, gate, row, b.capacity, src, own, n_ep, hidden_size=h,
                     bytes_per_elem=bytes_per_elem)
        compare_ledger(g, o)
        loads = O.rank_loads(idx, row, own, n_ep)
        assert np.array_equal(np.asarray(g["pair_routes"]).sum(axis=0), loads)
        assert M.moe_recommend_plan(g) == O.recommend_plan(o, o)
        leds.append(g)
    assert leds[1]["local_routes"] == best >= leds[0]["local_routes"]
    return leds[0], leds[1], owner


@pytest.mark.parametrize("name", W.ROUTING_SCENARIOS)
def test_locality_placement_on_routing_scenario(name):
    """[EP46] Step 3 (a more local expert placement) on the three routings
    of its Step 5 workload: affinity, placement and the ledgers before and
    after, against the oracle.  Local-heavy routing already favours the
    round-robin owners, so the placement keeps its local routes; balanced
    routing gains a little; the placement never loses local routes."""
    banner(f"locality placement {name}")
    cfg = W.SCENARIO_CONFIG
    inp = _inputs()
    mc = cfg_from(cfg)
    b = LayerBuffers(mc, capacity_of(mc))
    b.logits.copy_(torch.from_numpy(W.scenario_logits(name)))
    M.moe_route(mc, None, None, None, b.logits, b.topk_idx, b.topk_gate, None, b.ws)
    run_dispatch(b, inp.x, expert_load=True)
    before, after, owner = _placement_case(mc, b, inp.src_rank, cfg.n_ep, cfg.h, 2)
    if name == "local_heavy":
        assert after["local_routes"] == before["local_routes"]
    print(f"[placement] {name}: local hit {before['local_hit_ratio']:.4f} -> "
          f"{after['local_hit_ratio']:.4f}, owner {owner.tolist()}", flush=True)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_locality_placement_on_workloads(cid):
    """The same on the five workloads' own routing (GPU router)."""
    banner(f"locality placement config {cid}")
    from gpu_util import buffers_for, device_inputs
    inp = device_inputs(cid, with_experts=cid in (3, 4))
    cfg = inp.cfg
    mc = cfg_from(cfg)
    b = buffers_for(cfg)
    M.moe_route(mc, inp.x, inp.w_gate, inp.logit_bias, b.logits, b.topk_idx, b.topk_gate, None,
                b.ws)
    M.moe_dispatch(mc, None, b.topk_idx, b.capacity, b.expert_offsets, b.route_rank,
                   b.route_row, b.row_token, None, None, b.ws)
    _placement_case(mc, b, inp.src_rank, cfg.n_ep, cfg.h, cfg.bytes_per_elem)

"""The pre-marshalled step (LayerPlan) and its HIP-graph replay.

A captured graph is replayed several times, with eager work and host
synchronisation between replays, and every replay's outputs (layer output,
routing, slots and ledger) must equal the eager call sequence bit for bit.
The asynchronous ledger (moe_ledger_launch + moe_ledger_finalize) must equal
the synchronous moe_ledger."""
import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
from expert_dispatch_combine_amd.runner import LayerPlan, pack_weights, run_layer, run_ledger
from gpu_util import banner, buffers_for, device_inputs

pytestmark = pytest.mark.gpu


def _snapshot(b, led):
    return {"out": b.out.clone(), "idx": b.topk_idx.clone(), "gate": b.topk_gate.clone(),
            "row": b.route_row.clone(), "offs": b.expert_offsets.clone(),
            "acc": led["accepted_routes"], "P": list(led["P"]), "loads": list(led["loads"])}


def _same(a, c):
    for k in ("out", "idx", "gate", "row", "offs"):
        assert torch.equal(a[k], c[k]), k
    assert a["acc"] == c["acc"] and a["P"] == c["P"] and a["loads"] == c["loads"]


@pytest.mark.parametrize("cid,packed,tail,gather", [
    (1, False, "side", False), (2, False, "side", False), (2, True, "side", False),
    (3, True, "side", False), (4, True, "side", False), (5, True, "side", False),
    (1, False, "fused", True), (2, True, "fused", True), (3, True, "fused", True),
    (4, True, "fused", True),
    (5, True, "fused", True)])
def test_plan_and_graph_replay_match_eager(cid, packed, tail, gather):
    """tail "side": the ledger on a second stream beside the FFN; "fused":
    combine and ledger in one moe_combine_ledger call (one launch for
    workloads 1 and 2, two for workload 5's 98304 routes).  gather: the
    dispatch moves no row and moe_expert_ffn_rows gathers them (in the first
    GEMM's loads for the bf16 workloads, by a copy into y first for the fp32
    workload 1)."""
    banner(f"plan/graph config {cid} packed={packed} tail={tail} gather={gather}")
    inp = device_inputs(cid)
    cfg = inp.cfg
    b = buffers_for(cfg)
    w1, w2 = (pack_weights(b.cfg, inp.w1, inp.w2) if packed else (inp.w1, inp.w2))
    args = (inp.x, inp.w_gate, inp.logit_bias, w1, inp.b1, w2, inp.b2)
    # reference: plain eager calls on the default stream
    run_layer(b, *args, packed=packed)
    ref_led = run_ledger(b, inp.src_rank, inp.owner_rank, cfg.n_ep)
    torch.cuda.synchronize()
    ref = _snapshot(b, ref_led)

    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    plan = LayerPlan(b, *args, inp.src_rank, inp.owner_rank, cfg.n_ep, main=main,
                     side=side if tail == "side" else None, packed=packed,
                     fused_tail=tail == "fused", gather_in_ffn=gather)
    b.out.zero_()
    with torch.cuda.stream(main):
        plan.launch()
    torch.cuda.synchronize()
    _same(ref, _snapshot(b, plan.ledger()))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=main):
        plan.launch()
    torch.cuda.synchronize()
    for rep in range(4):
        b.out.fill_(float(rep + 1))       # eager work between replays
        b.topk_idx.fill_(-1)
        b.route_row.fill_(-5)
        plan.stage.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(main):
            g.replay()
        torch.cuda.synchronize()
        _same(ref, _snapshot(b, plan.ledger()))


def test_async_ledger_equals_sync_ledger():
    banner("async ledger")
    inp = device_inputs(5)
    cfg = inp.cfg
    b = buffers_for(cfg)
    run_layer(b, inp.x, inp.w_gate, inp.logit_bias, inp.w1, inp.b1, inp.w2, inp.b2)
    sync = run_ledger(b, inp.src_rank, inp.owner_rank, cfg.n_ep, alpha=0.03)
    stage = torch.empty((M.moe_ledger_stage_bytes(b.cfg, cfg.n_ep),), dtype=torch.uint8,
                        pin_memory=True)
    M.moe_ledger_launch(b.cfg, b.topk_idx, b.topk_gate, b.route_row, inp.src_rank,
                        inp.owner_rank, cfg.n_ep, stage, b.ws)
    torch.cuda.synchronize()
    asy = M.moe_ledger_finalize(b.cfg, b.capacity, cfg.n_ep, 0.03, stage)
    assert sync == asy

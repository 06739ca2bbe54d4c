"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code path: page worked
examples (tests/golden), closed forms, library routines the method reduces to,
brute force over tiny inputs, and invariants.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- page examples
def test_ep47_worked_examples():
    g = _load("ep47_ledger_cases.json")
    for case in g["cases"]:
        s = O.summarize_routes(case["routes"], case["num_experts"], case["hidden_size"],
                               case["bytes_per_elem"], case["capacity_factor"])
        for key, want in case["expect"].items():
            if key == "balance_ratio_3dp":
                assert round(s["balance_ratio"], 3) == want, case["name"]
            elif key == "balance_ratio_gt":
                assert s["balance_ratio"] > want, case["name"]
            else:
                assert s[key] == want, (case["name"], key, s[key], want)
        assert s["all_to_all_bytes"] == 2 * s["dispatch_bytes"]


def test_ep46_contracts():
    g = _load("ep46_contract_cases.json")
    c = g["capacity"]
    s = O.summarize_routes(c["routes"], c["num_experts"], c["hidden_size"])
    for key, want in c["expect"].items():
        if key == "balance_ratio_3dp":
            assert round(s["balance_ratio"], 3) == want
        else:
            assert s[key] == want, key
    e = g["empty"]
    s = O.summarize_routes(e["routes"], e["num_experts"], e["hidden_size"])
    for key, want in e["expect"].items():
        assert s[key] == want
    assert s["balance_ratio"] == 0.0
    for bad in g["invalid"]:
        with pytest.raises(ValueError):
            O.summarize_routes(bad["routes"], bad["num_experts"], bad["hidden_size"])
    tt = g["two_token_capacity"]
    s = O.summarize_routes(tt["routes"], tt["num_experts"], tt["hidden_size"])
    assert s["overflow"] == tt["expect"]["overflow"]
    assert s["balance_ratio"] <= tt["expect"]["balance_ratio_le"]
    loc = g["locality"]
    owners = {int(k): v for k, v in loc["expert_owner_ranks"].items()}
    d = O.dispatch_locality(loc["routes"], loc["token_source_ranks"], owners,
                            loc["hidden_size"], loc["bytes_per_elem"])
    assert d == loc["expect"]
    with pytest.raises(ValueError):
        O.dispatch_locality([[0]], [0, 1], owners, 8)
    with pytest.raises(ValueError):
        O.dispatch_locality([[2]], [0], owners, 8)
    cb = g["combine"]
    out = O.combine_index_add(cb["token_indices"], cb["expert_outputs"],
                              cb["routing_weights"], cb["num_tokens"])
    np.testing.assert_allclose(out, np.asarray(cb["expect"]), rtol=0, atol=1e-12)


def test_capacity_rounds_up():
    # 11 routes on 2 experts at cf 1.0: 5.5 -> 6 (the page's rejected case)
    assert O.capacity(11, 2, 1.0) == 6
    assert O.capacity(0, 4, 1.25) == 0
    assert O.capacity(2048, 16, 1.25) == 160
    assert O.capacity(8192, 8, 1.25) == 1280
    assert O.capacity(32768, 256, 1.0) == 128
    assert O.capacity(98304, 64, 1.0) == 1536
    assert O.capacity(128, 4, 1.0) == 32
    assert O.capacity(3, 2, 1.0) == 2
    assert O.capacity(1, 3, 0.5) == 1
    for bad in [(4, 0, 1.0), (4, 2, 0.0), (4, 2, -1.0), (4, 2, float("nan"))]:
        with pytest.raises(ValueError):
            O.capacity(*bad)


def test_epc_pair_bytes_table():
    g = _load("epc_pair_bytes.json")
    rng = np.random.default_rng(0)
    for c in g["cases"]:
        # any routing of B tokens with K experts each has A = B*K routes
        T, K, h, n = c["B"], c["K"], c["h"], c["N_EP"]
        E = 256 if c["model"] == "DeepSeek-V3" else 16
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        s = O.summarize_routes(O.routes_from_idx(idx), E, h, c["dtype_bytes"])
        per_pair = s["logical_route_bytes"] / n
        assert per_pair == c["expect_bytes"]
        if c["compare"].startswith("bytes/1e6"):
            assert f"{per_pair / 1e6:.1f} MB" == c["page_value"]
        else:
            assert f"{per_pair / 2**20:.2f} MB" == c["page_value"]


def test_round_robin_placement_example():
    g = _load("dsv3_placement.json")
    p = O.uniform_expert_placement(g["num_experts"], g["num_devices"])
    for dev, experts in g["expect"].items():
        assert p[int(dev)] == experts
    assert all(len(v) == g["experts_per_device"] for v in p.values())
    assert sorted(sum(p.values(), [])) == list(range(g["num_experts"]))


# ---------------------------------------------------------------- closed forms
def test_aux_loss_closed_forms():
    alpha = 0.01
    rng = np.random.default_rng(1)
    # perfectly balanced selections: every expert in exactly T*K/E tokens
    E, K, T = 8, 2, 64
    idx = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])
    gate = rng.random((T, K))
    gate /= gate.sum(1, keepdims=True)
    a = O.aux_loss_terms(idx, gate, E, alpha)
    assert np.allclose(a["f"], K / E)
    assert math.isclose(a["l_aux"], alpha * K / E, rel_tol=1e-12)
    assert math.isclose(a["l_aux_norm"], alpha, rel_tol=1e-12)
    assert math.isclose(a["P"].sum(), 1.0, rel_tol=1e-12)
    # every token on expert 0 with K = 1
    idx = np.zeros((T, 1), int)
    a = O.aux_loss_terms(idx, np.ones((T, 1)), E, alpha)
    assert math.isclose(a["l_aux"], alpha, rel_tol=1e-12)
    assert math.isclose(a["l_aux_norm"], alpha * E, rel_tol=1e-12)
    a = O.aux_loss_terms(np.zeros((0, 2), int), np.zeros((0, 2)), E, alpha)
    assert a["l_aux"] == 0.0 and a["l_aux_norm"] == 0.0


def test_round_bf16_special_values_and_torch():
    one = 1.0
    assert O.round_bf16(one) == 1.0
    assert O.round_bf16(1 + 2 ** -8) == 1.0                 # tie -> even (down)
    assert O.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6      # tie -> even (up)
    assert O.round_bf16(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7
    assert O.round_bf16(-0.0) == 0.0
    assert O.round_bf16(3.0) == 3.0
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(v.astype(np.float64)), ref)
    np.testing.assert_array_equal(O.round_f32(np.float64(1 + 2 ** -40)), 1.0)


def test_gelu_tanh_matches_torch():
    u = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(u), ref, rtol=1e-14, atol=1e-15)
    assert O.gelu_tanh(0.0) == 0.0


# ---------------------------------------------------------------- router
def test_router_logits_exact_integers():
    rng = np.random.default_rng(3)
    x = rng.integers(-4, 5, (13, 7)).astype(np.float64)
    w = rng.integers(-3, 4, (5, 7)).astype(np.float64)
    got = O.router_logits(x, w)
    for t in range(13):
        for e in range(5):
            assert got[t, e] == sum(int(x[t, j]) * int(w[e, j]) for j in range(7))
    # W_g acts on x as a column: logits[t] = W_g @ x[t], not W_g^T
    x = rng.standard_normal((3, 4))
    w = rng.standard_normal((6, 4))
    np.testing.assert_allclose(O.router_logits(x, w), (w @ x.T).T.astype(np.float32))


def test_topk_softmax_matches_torch_without_ties():
    rng = np.random.default_rng(4)
    for E, K in [(4, 2), (16, 1), (8, 2), (64, 6), (256, 8), (5, 5)]:
        l = rng.standard_normal((50, E)).astype(np.float32)
        idx, g = O.topk_softmax(l, K)
        tv, ti = torch.topk(torch.from_numpy(l).double(), K, dim=-1)
        assert np.array_equal(idx, ti.numpy())
        ref = torch.softmax(tv, dim=-1).numpy()
        np.testing.assert_allclose(g, ref.astype(np.float32), rtol=2e-7, atol=0)
        np.testing.assert_allclose(g.astype(np.float64).sum(1), 1.0, rtol=1e-6)
        if K == 1:
            assert np.all(g == 1.0)


def test_topk_ties_brute_force():
    rng = np.random.default_rng(5)
    for E, K in [(4, 2), (6, 3), (8, 8), (3, 1)]:
        l = rng.integers(-2, 3, (200, E)).astype(np.float32)
        l[rng.random(l.shape) < 0.1] = -0.0
        idx, g = O.topk_softmax(l, K)
        for t in range(l.shape[0]):
            # brute force: the K smallest (-logit, id) pairs, in that order
            pairs = sorted((-float(l[t, e]) + 0.0, e) for e in range(E))
            assert [e for _, e in pairs[:K]] == list(idx[t])
            sel = [float(l[t, e]) for e in idx[t]]
            den = sum(math.exp(v) for v in sel)
            for k in range(K):
                assert abs(g[t, k] - math.exp(sel[k]) / den) <= 1e-7 * g[t, k] + 1e-12
    with pytest.raises(ValueError):
        O.topk_softmax(np.zeros((2, 3), np.float32), 4)


def test_logit_bias_changes_the_routing_and_is_kept_in_the_softmax():
    l = np.array([[1.0, 0.5, 0.0]], np.float32)
    b = np.array([0.0, 1.0, 0.0], np.float32)
    idx, g = O.topk_softmax(l, 2, b)
    assert list(idx[0]) == [1, 0]
    e = math.exp(1.5) + math.exp(1.0)
    assert abs(g[0, 0] - math.exp(1.5) / e) < 1e-7


# ---------------------------------------------------------------- slotting
def _all_routings(T, E, K):
    per_token = list(itertools.permutations(range(E), K))
    return itertools.product(per_token, repeat=T)


@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (2, 2, 1), (3, 2, 2), (4, 3, 1), (3, 3, 2), (4, 3, 2)])
def test_slotting_brute_force(T, E, K):
    A = T * K
    for routing in _all_routings(T, E, K):
        idx = np.array(routing, dtype=np.int32).reshape(T, K)
        flat = idx.reshape(-1)
        loads = [int((flat == e).sum()) for e in range(E)]
        for cap in range(0, A + 1):
            sl = O.slot_routes(idx, E, cap)
            # independent formulation: rank = earlier routes (row-major) to the same expert
            rank = np.array([int((flat[:i] == flat[i]).sum()) for i in range(A)]).reshape(T, K)
            assert np.array_equal(sl["route_rank"], rank)
            acc = [min(l, cap) for l in loads]
            off = np.concatenate([[0], np.cumsum(acc)])
            assert np.array_equal(sl["expert_offsets"], off)
            want_row = np.where(rank < cap, off[idx] + rank, -1)
            assert np.array_equal(sl["route_row"], want_row)
            R = int(off[-1])
            assert sl["R"] == R and R + O.overflow(loads, cap) == A
            rows = sorted(int(r) for r in sl["route_row"].reshape(-1) if r >= 0)
            assert rows == list(range(R))
            for e in range(E):
                seg = sl["row_token"][off[e]:off[e + 1]]
                assert np.all(np.diff(seg) > 0)          # token order inside a segment
            for t in range(T):
                for k in range(K):
                    if sl["route_row"][t, k] >= 0:
                        assert sl["row_token"][sl["route_row"][t, k]] == t


def test_slotting_rejects_bad_ids():
    with pytest.raises(ValueError):
        O.slot_routes(np.array([[3]]), 3, 1)
    with pytest.raises(ValueError):
        O.expert_loads(np.array([[-1]]), 3)


# ---------------------------------------------------------------- FFN, combine, layer
def test_expert_ffn_matches_torch_linear_gelu():
    rng = np.random.default_rng(6)
    E, F, h = 3, 12, 5
    w1 = rng.standard_normal((E, F, h)); b1 = rng.standard_normal((E, F))
    w2 = rng.standard_normal((E, h, F)); b2 = rng.standard_normal((E, h))
    offsets = np.array([0, 4, 4, 9])
    xd = rng.standard_normal((9, h))
    H, Y = O.expert_ffn(xd, offsets, w1, b1, w2, b2)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        a = torch.from_numpy(xd[lo:hi])
        hh = torch.nn.functional.gelu(torch.nn.functional.linear(a, torch.from_numpy(w1[e]),
                                                                 torch.from_numpy(b1[e])),
                                      approximate="tanh")
        y = torch.nn.functional.linear(hh, torch.from_numpy(w2[e]), torch.from_numpy(b2[e]))
        np.testing.assert_allclose(H[lo:hi], hh.numpy(), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(Y[lo:hi], y.numpy().astype(np.float32), rtol=1e-6, atol=1e-6)
    # sampled-row form agrees with the segment form
    rows_e = np.array([0, 0, 2, 2, 2, 0])
    rows = np.array([0, 3, 4, 8, 5, 1])
    H2, Y2 = O.expert_ffn_rows(xd[rows], rows_e, w1, b1, w2, b2)
    np.testing.assert_allclose(Y2, Y[rows], rtol=1e-6, atol=1e-7)
    # bf16 rounding of H moves it to the bf16 grid
    Hb, _ = O.expert_ffn(xd, offsets, w1, b1, w2, b2, h_round="bf16")
    assert np.array_equal(Hb, O.round_bf16(Hb))
    assert np.max(np.abs(Hb - H)) <= np.max(np.abs(H)) * 2 ** -8


def test_combine_gather_equals_index_add():
    rng = np.random.default_rng(7)
    T, K, h, R = 20, 3, 6, 70
    Y = rng.standard_normal((R, h)).astype(np.float32)
    gate = rng.random((T, K)).astype(np.float32)
    rows = rng.permutation(R)[:T * K].reshape(T, K).astype(np.int32)
    rows[rng.random((T, K)) < 0.3] = -1
    rows[0, :] = -1                                  # a token with every route dropped
    out = O.combine(Y, rows, gate)
    m = rows.reshape(-1) >= 0
    tok = np.repeat(np.arange(T), K)[m]
    ref = O.combine_index_add(tok, Y[rows.reshape(-1)[m]], gate.reshape(-1)[m], T)
    np.testing.assert_allclose(out, ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    assert np.all(out[0] == 0.0)


def _small_layer(T=40, h=16, E=5, K=2, F=24, seed=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, h))
    wg = rng.standard_normal((E, h)) / math.sqrt(h)
    w1 = rng.standard_normal((E, F, h)) / math.sqrt(h)
    b1 = 0.1 * rng.standard_normal((E, F))
    w2 = rng.standard_normal((E, h, F)) / math.sqrt(F)
    b2 = 0.1 * rng.standard_normal((E, h))
    return x, wg, w1, b1, w2, b2


@pytest.mark.parametrize("cf", [0.5, 1.0, 1e9])
def test_layer_two_formulations_agree(cf):
    x, wg, w1, b1, w2, b2 = _small_layer()
    K = 2
    L = O.moe_layer(x, wg, w1, b1, w2, b2, K, cf)
    acc = L["route_row"] >= 0
    out2 = O.moe_layer_per_token(x, L["idx"], L["gate"], acc, w1, b1, w2, b2)
    np.testing.assert_allclose(L["out"], out2, rtol=1e-6, atol=1e-7)
    if cf == 1e9:
        assert acc.all()
        # with nothing dropped the layer is the dense top-k MoE: sum_k g_k FFN_k(x)
        xt = torch.from_numpy(x)
        dense = torch.zeros_like(xt)
        for t in range(x.shape[0]):
            for k in range(K):
                e = int(L["idx"][t, k])
                hh = torch.nn.functional.gelu(xt[t] @ torch.from_numpy(w1[e]).T
                                              + torch.from_numpy(b1[e]), approximate="tanh")
                dense[t] += float(L["gate"][t, k]) * (hh @ torch.from_numpy(w2[e]).T
                                                      + torch.from_numpy(b2[e]))
        np.testing.assert_allclose(L["out"], dense.numpy(), rtol=1e-5, atol=1e-6)
    else:
        assert (~acc).any()


def test_ledger_invariants_and_empty():
    x, wg, w1, b1, w2, b2 = _small_layer(T=64, E=6, K=2)
    L = O.moe_layer(x, wg, w1, b1, w2, b2, 2, 0.8)
    src = np.arange(64) % 3
    owner = np.arange(6) % 3
    led = O.ledger(L["idx"], L["gate"], L["route_row"], L["capacity"], src, owner, 3, 16, 2)
    A = 128
    assert led["total_routes"] == A and int(led["expert_loads"].sum()) == A
    assert led["local_routes"] + led["cross_rank_routes"] == A
    assert led["all_to_all_bytes"] == 2 * led["dispatch_bytes"]
    assert led["accepted_routes"] + led["overflow"] == A
    assert led["accepted_local_routes"] + led["accepted_cross_rank_routes"] == led["accepted_routes"]
    assert int(led["pair_routes"].sum()) == led["accepted_routes"]
    assert int(np.trace(led["pair_routes"])) == led["accepted_local_routes"]
    assert math.isclose(led["f"].sum(), 2.0, rel_tol=1e-12)
    assert math.isclose(led["P"].sum(), 1.0, rel_tol=1e-6)
    assert led["local_hit_ratio"] == led["local_routes"] / A
    assert led["cross_rank_roundtrip_bytes"] == 2 * led["cross_rank_dispatch_bytes"]
    assert led["balance_ratio"] == led["max_load"] / (A / 6)
    # empty batch: zero ledger
    z = O.ledger(np.zeros((0, 2), np.int32), np.zeros((0, 2), np.float32),
                 np.zeros((0, 2), np.int32), 0, np.zeros(0, int), owner, 3, 16, 2)
    assert z["total_routes"] == 0 and z["capacity"] == 0 and z["balance_ratio"] == 0.0
    assert z["local_hit_ratio"] == 0.0 and z["l_aux"] == 0.0
    with pytest.raises(ValueError):
        O.ledger(L["idx"], L["gate"], L["route_row"], 1, src, np.arange(6) % 4, 3, 16, 2)


def test_load_monitor_alarm():
    m = O.load_monitor([10, 1])
    assert math.isclose(m["max_over_mean"], 10 / 5.5)
    assert not m["imbalanced"]
    m = O.load_monitor([30, 1, 1, 0])
    assert m["imbalanced"]
    assert math.isclose(m["var_over_mean"], float(np.var([30, 1, 1, 0], ddof=1)) / 8.0)


# ------------------------------------------------- aux-loss-free bias update
def test_top1_counts_match_argmax_bincount():
    """[DSV3] section 八 counts tokens by bincount(argmax(adjusted logits));
    torch's argmax returns the first maximum, i.e. the lower id on ties."""
    rng = np.random.default_rng(11)
    for T, E in [(1, 1), (50, 3), (200, 7), (333, 16)]:
        logits = rng.integers(-2, 3, (T, E)).astype(np.float32)  # many ties
        want = torch.bincount(torch.from_numpy(logits).argmax(-1), minlength=E).numpy()
        assert np.array_equal(O.top1_counts(logits), want)


def test_bias_update_closed_forms():
    rng = np.random.default_rng(12)
    E = 8
    bias = rng.standard_normal(E).astype(np.float32)
    # balanced counts: mean == count for every expert, the bias does not move
    new = O.expert_bias_update(bias, np.full(E, 125), alpha=0.1)
    assert np.array_equal(new, bias.astype(np.float64))
    # every token on expert 0 (T = 1000): steps 0.1 * (125 - 1000) and 0.1 * 125
    counts = np.zeros(E, np.int64)
    counts[0] = 1000
    new = O.expert_bias_update(bias, counts, alpha=0.1)
    exact = bias.astype(np.float64) + 0.1 * (125.0 - counts)
    ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(new - exact) <= 2 * ulp + 1e-6)
    assert new[0] < bias[0] and np.all(new[1:] > bias[1:])
    # the steps cancel: sum(mean - count) = 0
    counts = rng.integers(0, 500, E)
    new = O.expert_bias_update(bias, counts, alpha=0.1)
    assert abs(float(np.sum(new - bias))) <= 1e-3


def test_bias_update_balances_a_skewed_router():
    """The rule's purpose ([DSV3] 3.3 / section 八): iterating route -> count
    -> update drives a Zipf-skewed top-1 routing toward equal loads.  The step
    acts on raw token counts, so it must be small against them: with the
    page's alpha = 0.1 and 2048 tokens the bias overshoots by tens of logits
    per step (checked too); alpha = 1e-3 settles."""
    rng = np.random.default_rng(13)
    T, E = 2048, 16
    perm = rng.permutation(E)
    logits = (rng.standard_normal((T, E)) - 1.2 * np.log(perm + 1.0)).astype(np.float32)

    def run(alpha, steps):
        bias = np.zeros(E, np.float32)
        ratios = []
        for _ in range(steps):
            counts = O.top1_counts(O.add_logit_bias(logits, bias))
            ratios.append(counts.max() / (T / E))
            bias = O.expert_bias_update(bias, counts, alpha=alpha).astype(np.float32)
        return ratios

    r = run(1e-3, 40)
    assert r[0] > 3.0 and max(r[-5:]) < 1.2
    r = run(0.1, 12)
    assert max(r[-6:]) > 3.0  # oscillates: every token flips to one expert


# ------------------------------------------------------- FP8 dispatch payload
def test_e4m3_codes_match_torch_float8():
    """[DSV3] 4.3 converts with torch's float8_e4m3fn; the oracle's E4M3
    rounding is checked against it on every code and on values across the
    whole range (subnormals, ties, the 448/464 edge, overflow to NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(want), np.isnan(got))
    assert np.array_equal(want[~np.isnan(want)], got[~np.isnan(got)])
    rng = np.random.default_rng(21)
    vals = rng.standard_normal(50000) * np.exp2(rng.integers(-14, 10, 50000))
    vals = np.concatenate([vals, want[~np.isnan(want)],  # every finite code, and
                           (want[1:120] + want[:119]) / 2,  # every midpoint (ties)
                           [448, 449, 463, 464, 465, 480, 1e6, -464, -465, 0.0, -0.0]])
    vals = vals.astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(vals.astype(np.float64)), ref)


def test_fp8_payload_matches_the_pages_torch_expression():
    """scale = x.abs().max() / 448; q = (x / scale).to(float8_e4m3fn);
    back = q.to(bfloat16) * scale, all on bf16 tensors ([DSV3] 4.3)."""
    rng = np.random.default_rng(22)
    for shape, mag in [((64, 96), 1.0), ((7, 33), 1e-3), ((128, 64), 300.0), ((1, 16), 1.0)]:
        x = torch.from_numpy((rng.standard_normal(shape) * mag).astype(np.float32)).to(
            torch.bfloat16)
        scale_t = x.abs().max() / 448.0
        q_t = (x / scale_t).to(torch.float8_e4m3fn)
        back_t = q_t.to(torch.bfloat16) * scale_t
        x64 = x.to(torch.float64).numpy()
        scale = O.fp8_scale(x64)
        assert scale == float(scale_t)
        q = O.fp8_quantize(x64, scale)
        assert np.array_equal(q, q_t.view(torch.uint8).numpy())
        assert np.array_equal(O.fp8_dequantize(q, scale), back_t.to(torch.float64).numpy())


def test_fp8_round_trip_error_and_zero_input():
    rng = np.random.default_rng(23)
    x = O.round_bf16(rng.standard_normal((50, 128)))
    scale = O.fp8_scale(x)
    back = O.fp8_dequantize(O.fp8_quantize(x, scale), scale)
    # E4M3 keeps 3 mantissa bits: half a step is 2^-4 relative for normals, 2^-10
    # scale absolute in the subnormal range; plus the bf16 roundings
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scale + 2.0 ** -7 * np.abs(x)
    assert np.all(np.abs(back - x) <= bound)
    assert np.max(np.abs(x)) <= 448.0 * scale * (1 + 2.0 ** -7)
    z = np.zeros((4, 16))
    assert O.fp8_scale(z) == 0.0
    assert not np.any(O.fp8_quantize(z, 0.0)) and not np.any(O.fp8_dequantize(O.fp8_quantize(z, 0.0), 0.0))


# -------------------------------------------------------------- plan decision
def test_plan_decision_page_contract():
    g = _load("ep46_decision_cases.json")
    assert O.PLAN_THRESHOLDS == g["source"]["thresholds"]
    for case in g["cases"]:
        s = O.summarize_routes(case["routes"], case["num_experts"], case["hidden_size"])
        assert O.recommend_plan(s, case["locality"]) == case["expect"], case["name"]


def test_plan_decision_boundaries():
    """Each limit is inclusive, and crossing any one of them moves the plan."""
    def summ(A, overflow, bal):
        return {"total_routes": A, "overflow": overflow, "balance_ratio": bal}

    def loc(cross, total=100):
        return {"total_routes": total, "local_routes": total - cross, "cross_rank_routes": cross}

    assert O.recommend_plan(summ(0, 0, 0.0)) == "reject"
    assert O.recommend_plan(summ(100, 0, 1.2), loc(50)) == "accept"
    # the balance ratio is compared as the summary stores it, round(., 3)
    assert O.recommend_plan(summ(100, 0, 1.2004), loc(50)) == "accept"
    assert O.recommend_plan(summ(100, 0, 1.2006), loc(50)) == "tune"
    assert O.recommend_plan(summ(100, 0, 1.0), loc(51)) == "tune"
    assert O.recommend_plan(summ(100, 1, 1.0), loc(0)) == "tune"
    assert O.recommend_plan(summ(100, 25, 1.8), loc(90)) == "tune"
    assert O.recommend_plan(summ(100, 26, 1.0), loc(0)) == "reject"
    assert O.recommend_plan(summ(100, 0, 1.8004), loc(0)) == "tune"
    assert O.recommend_plan(summ(100, 0, 1.8006), loc(0)) == "reject"
    assert O.recommend_plan(summ(100, 0, 1.0), loc(91)) == "reject"
    assert O.recommend_plan(summ(100, 0, 1.0), loc(0, total=0)) == "accept"


def test_plan_decision_reads_the_stored_3_decimal_balance():
    """[EP46] Step 4 reference code: the summary stores round(balance_ratio, 3)
    and the joint decision (TODO 3) compares that stored value with its
    limits.  Routings whose exact ratio lies just past a limit but rounds onto
    it decide as on the page.  The page's decision is evaluated here by its
    own rule on the rounded value."""
    def page(loads, E, cf):
        routes = [[e] for e in range(E) for _ in range(loads[e])]
        return O.summarize_routes(routes, E, 8, 2, cf)

    # 6002 / 3998 routes over 2 experts, cf 1.25: cap 6250, no overflow,
    # balance 1.2004 -> stored 1.2 -> accept (the unrounded value would tune)
    s = page([6002, 3998], 2, 1.25)
    assert s["overflow"] == 0 and s["balance_ratio"] > 1.2
    assert O.recommend_plan(s) == "accept"
    # 9002 / 998 routes, cf 1.8: cap 9000, overflow 2 (share 2e-4), balance
    # 1.8004 -> stored 1.8 -> tune (the unrounded value would reject)
    s = page([9002, 998], 2, 1.8)
    assert s["overflow"] == 2 and s["balance_ratio"] > 1.8
    assert O.recommend_plan(s) == "tune"
    # 12005 / 7995: the double nearest 1.2005 lies below the decimal
    # midpoint, so it rounds to 1.2 and accepts; 12006 / 7994 rounds to 1.201
    s = page([12005, 7995], 2, 1.25)
    assert round(s["balance_ratio"], 3) == 1.2 and O.recommend_plan(s) == "accept"
    s = page([12006, 7994], 2, 1.25)
    assert round(s["balance_ratio"], 3) == 1.201 and O.recommend_plan(s) == "tune"


def test_expert_loads_match_the_pages_worked_examples():
    """[EP47] 测试: the route ledgers of the worked examples assert the loads
    [2, 2, 2], [3, 1], [10, 1] and [0, 0] (empty)."""
    g = _load("ep47_ledger_cases.json")
    for case in g["cases"]:
        E = case["num_experts"]
        routes = case["routes"]
        want = case["expect"]["expert_loads"]
        if routes:
            K = len(routes[0])
            if all(len(r) == K for r in routes):
                idx = np.asarray(routes, np.int64).reshape(len(routes), K)
                assert O.expert_loads(idx, E).tolist() == want, case["name"]
        flat = np.asarray([e for r in routes for e in r], np.int64).reshape(-1, 1)
        assert O.expert_loads(flat, E).tolist() == want, case["name"]


def test_expert_loads_against_an_independent_count():
    """Every routing with T <= 4 tokens, E <= 3 experts and K <= 2 distinct
    experts per token, plus random large ones: the loads equal numpy's
    bincount of the ids (a library count, independent of the oracle's loop)."""
    import itertools
    for E in (1, 2, 3):
        for K in range(1, min(E, 2) + 1):
            choices = list(itertools.permutations(range(E), K))
            for T in range(0, 5 if E < 3 else 4):
                for combo in itertools.product(choices, repeat=T):
                    idx = np.asarray(combo, np.int64).reshape(T, K)
                    want = np.bincount(idx.reshape(-1), minlength=E)
                    assert np.array_equal(O.expert_loads(idx, E), want)
    rng = np.random.default_rng(31)
    for T, E, K in [(1000, 16, 1), (513, 64, 6), (77, 256, 8)]:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        want = np.bincount(idx.reshape(-1), minlength=E)
        assert np.array_equal(O.expert_loads(idx, E), want)


def test_bias_update_bit_exact_against_the_pages_torch_expression():
    """[DSV3] section 八 DeepSeekV3Gate: with fp32 tensors, expert_count =
    bincount(...).float(); mean_count = expert_count.mean(); expert_bias.data
    += alpha * (mean_count - expert_count).  The page's expression, run by
    torch on the CPU, equals the oracle's update bit for bit."""
    rng = np.random.default_rng(32)
    for trial in range(300):
        E = int(rng.choice([1, 2, 3, 8, 16, 64, 256]))
        T = int(rng.integers(0, 20000))
        alpha = float(rng.choice([0.1, 1e-3, 0.37, 2.0 ** -7]))
        bias = (rng.standard_normal(E) * rng.choice([1e-3, 1.0, 30.0])).astype(np.float32)
        counts = rng.multinomial(T, rng.dirichlet(np.ones(E) * 0.3)) if E > 1 else np.array([T])
        expert_bias = torch.from_numpy(bias.copy())
        expert_count = torch.zeros(E)
        expert_count += torch.from_numpy(counts.astype(np.int64)).float()
        mean_count = expert_count.mean()
        expert_bias.data += alpha * (mean_count - expert_count)
        got = O.expert_bias_update(bias, counts, alpha=alpha)
        assert np.array_equal(got, expert_bias.numpy().astype(np.float64)), (trial, E, T, alpha)


# ------------------------------------------------ locality-aware placement
def _all_equal_count_maps(E, n):
    """Every expert -> rank map with E / n experts per rank (brute force)."""
    import itertools
    per = E // n
    for owner in itertools.product(range(n), repeat=E):
        if all(owner.count(r) == per for r in range(n)):
            yield owner


def test_placement_reaches_the_brute_force_optimum():
    """[DSV3] 2.2 matches experts to devices on an affinity matrix; the
    placement must keep E / n_ep experts per rank and reach the largest
    number of local routes over all such maps (enumerated)."""
    rng = np.random.default_rng(51)
    for E, n in [(2, 2), (4, 2), (6, 2), (6, 3), (8, 4), (8, 2), (4, 4), (3, 1)]:
        maps = list(_all_equal_count_maps(E, n))
        for trial in range(6):
            aff = rng.integers(0, 9, (E, n))
            if trial == 0:
                aff[:] = 3            # all maps tie
            owner = O.locality_placement(aff, n)
            assert sorted(np.bincount(owner, minlength=n).tolist()) == [E // n] * n
            best = max(sum(int(aff[e, m[e]]) for e in range(E)) for m in maps)
            assert O.local_routes_under(aff, owner) == best


def test_affinity_and_locality_agree_with_the_page_contract():
    """sum_e affinity[e, owner[e]] is the local-route count of [EP46]'s
    dispatch-locality summary for any placement; the rows sum to the expert
    loads and the whole matrix to the routes (accepted routes when route_row
    is given)."""
    rng = np.random.default_rng(52)
    T, E, K, n = 300, 8, 2, 4
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    src = rng.integers(0, n, T)
    aff = O.expert_rank_affinity(idx, src, E, n)
    assert aff.sum() == T * K
    assert np.array_equal(aff.sum(axis=1), O.expert_loads(idx, E))
    for owner in [np.arange(E) % n, O.locality_placement(aff, n), rng.integers(0, n, E)]:
        loc = O.dispatch_locality(O.routes_from_idx(idx), src.tolist(),
                                  {e: int(owner[e]) for e in range(E)}, 16)
        assert O.local_routes_under(aff, owner) == loc["local_routes"]
    cap = O.capacity(T * K, E, 0.8)
    sl = O.slot_routes(idx, E, cap)
    acc = O.expert_rank_affinity(idx, src, E, n, route_row=sl["route_row"])
    assert acc.sum() == sl["R"]
    assert np.array_equal(O.rank_loads(idx, sl["route_row"], np.arange(E) % n, n),
                          np.bincount(np.arange(E) % n, weights=acc.sum(axis=1),
                                      minlength=n).astype(np.int64))


def test_placement_follows_rank_local_routing():
    """Tokens of rank r route only to the experts of a hidden block of E / n
    experts (a permuted local-heavy routing): the placement recovers that
    block for every rank, so every route is local, where round robin keeps
    only what the permutation happens to leave on each rank."""
    rng = np.random.default_rng(53)
    E, n, K, T = 8, 4, 2, 400
    perm = rng.permutation(E)
    home = {int(perm[e]): e // (E // n) for e in range(E)}  # expert -> hidden rank
    src = rng.integers(0, n, T)
    idx = np.stack([rng.permutation(perm[(E // n) * s:(E // n) * (s + 1)])[:K] for s in src])
    aff = O.expert_rank_affinity(idx, src, E, n)
    owner = O.locality_placement(aff, n)
    assert O.local_routes_under(aff, owner) == T * K
    assert all(int(owner[e]) == home[e] for e in range(E))

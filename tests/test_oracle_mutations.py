"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in an oracle function (on the CPU, through
monkeypatch: the oracle's files are untouched) and runs the pins aimed at
that function from test_oracle_pins.py.  At least one of them must fail;
a mistake that every pin lets through would mean the oracle is not pinned
where it matters.  The mistakes are the kind a rewrite could make: a wrong
constant, a dropped term, a flipped sign, an off-by-one, a transposed loop
order, truncation instead of rounding, a wrong tie order.
"""
import math

import numpy as np
import pytest

import oracle as O
import oracle.moe_oracle as OM
import test_oracle_pins as P

_NAMES = ("gelu_tanh", "topk_softmax", "capacity", "slot_routes", "combine", "router_logits",
          "expert_ffn_segment", "expert_loads", "aux_loss_terms", "expert_bias_update",
          "e4m3_encode", "round_bf16", "dispatch_locality", "recommend_plan")
ORIG = {n: getattr(OM, n) for n in _NAMES}


# ------------------------------------------------------------------ mistakes
def gelu_wrong_cubic(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.0447 * u ** 3)))


def gelu_erf_form(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.vectorize(math.erf)(u / math.sqrt(2.0)))


def topk_ties_to_higher_id(logits32, K, bias32=None):
    l = np.asarray(logits32)
    E = l.shape[1]
    b = None if bias32 is None else np.asarray(bias32)[::-1]
    idx, g = ORIG["topk_softmax"](np.ascontiguousarray(l[:, ::-1]), K, b)
    return E - 1 - idx, g


def topk_softmax_over_all_experts(logits32, K, bias32=None):
    idx, _ = ORIG["topk_softmax"](logits32, K, bias32)
    l = OM.add_logit_bias(np.asarray(logits32, np.float32), bias32).astype(np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return idx, np.take_along_axis(p, idx, axis=1).astype(np.float32)


def capacity_floor(A, E, cf):
    if E <= 0 or not cf > 0:
        raise ValueError("bad")
    return 0 if A == 0 else int(math.floor((A / E) * cf))


def slot_accepts_one_more(idx, E, cap):
    return ORIG["slot_routes"](idx, E, cap + 1)


def slot_k_major(idx, E, cap):
    idx = np.asarray(idx)
    T, K = idx.shape
    r = ORIG["slot_routes"](idx.T.reshape(-1, 1), E, cap)  # routes ranked k-major
    out = dict(r)
    out["route_rank"] = np.asarray(r["route_rank"]).reshape(K, T).T
    out["route_row"] = np.asarray(r["route_row"]).reshape(K, T).T
    out["row_token"] = np.asarray(r["row_token"]) % T
    return out


def combine_renormalised(Y, route_row, gate):
    g = np.asarray(gate, np.float64).copy()
    acc = np.asarray(route_row) >= 0
    s = (g * acc).sum(axis=1, keepdims=True)
    s[s == 0] = 1.0
    return ORIG["combine"](Y, route_row, g / s)


def router_drops_last_column(x, w_gate):
    return ORIG["router_logits"](np.asarray(x)[:, :-1], np.asarray(w_gate)[:, :-1])


def ffn_without_b2(rows_x, w1_e, b1_e, w2_e, b2_e, h_round=None):
    return ORIG["expert_ffn_segment"](rows_x, w1_e, b1_e, w2_e,
                                      np.zeros_like(np.asarray(b2_e, np.float64)), h_round)


def ffn_w2_transposed_slice(rows_x, w1_e, b1_e, w2_e, b2_e, h_round=None):
    # W2 read as if it were [F, h] and square-cropped: the classic layout slip
    w2 = np.asarray(w2_e, np.float64)
    n = min(w2.shape)
    w2t = w2.copy()
    w2t[:n, :n] = w2[:n, :n].T
    return ORIG["expert_ffn_segment"](rows_x, w1_e, b1_e, w2t, b2_e, h_round)


def loads_off_by_one(idx, E):
    return ORIG["expert_loads"](idx, E) + (np.arange(E) == 0)


def aux_without_alpha(idx, gate, num_experts, alpha=0.01):
    d = dict(ORIG["aux_loss_terms"](idx, gate, num_experts, alpha))
    d["l_aux"] = d["l_aux"] / alpha
    return d


def bias_update_sign_flipped(bias32, counts, alpha=0.1):
    return ORIG["expert_bias_update"](bias32, counts, -alpha)


def e4m3_scaled_slightly(v):
    return ORIG["e4m3_encode"](np.asarray(v, np.float64) * (1.0 - 2.0 ** -6))


def bf16_truncating(a):
    f = np.asarray(a, np.float64).astype(np.float32)
    u = f.view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def locality_swapped(*args, **kw):
    d = dict(ORIG["dispatch_locality"](*args, **kw))
    d["local_routes"], d["cross_rank_routes"] = d["cross_rank_routes"], d["local_routes"]
    return d


def plan_rounds_balance_up(summary, locality=None, **thresholds):
    s = dict(summary)
    s["balance_ratio"] = math.ceil(s["balance_ratio"] * 1000.0) / 1000.0
    return ORIG["recommend_plan"](s, locality, **thresholds)


# ------------------------------------------------------------------ cases
def _slot_pins():
    return [(P.test_slotting_brute_force, (3, 2, 2)), (P.test_slotting_brute_force, (4, 3, 2)),
            (P.test_slotting_brute_force, (4, 3, 1)), (P.test_layer_two_formulations_agree, (0.5,))]


CASES = {
    "gelu: wrong cubic coefficient": ("gelu_tanh", gelu_wrong_cubic,
                                      [(P.test_gelu_tanh_matches_torch, ())]),
    "gelu: erf form instead of tanh form": ("gelu_tanh", gelu_erf_form,
                                            [(P.test_gelu_tanh_matches_torch, ())]),
    "top-k: ties to the higher id": ("topk_softmax", topk_ties_to_higher_id,
                                     [(P.test_topk_ties_brute_force, ())]),
    "top-k: softmax over all experts": ("topk_softmax", topk_softmax_over_all_experts,
                                        [(P.test_topk_softmax_matches_torch_without_ties, ()),
                                         (P.test_topk_ties_brute_force, ())]),
    "capacity: floor instead of ceil": ("capacity", capacity_floor,
                                        [(P.test_capacity_rounds_up, ()),
                                         (P.test_ep47_worked_examples, ())]),
    "slots: accepts one route too many": ("slot_routes", slot_accepts_one_more, _slot_pins()),
    "slots: ranks routes k-major": ("slot_routes", slot_k_major, _slot_pins()),
    "combine: renormalises over accepted gates": ("combine", combine_renormalised,
                                                  [(P.test_combine_gather_equals_index_add, ()),
                                                   (P.test_layer_two_formulations_agree, (0.5,))]),
    "router: drops the last hidden column": ("router_logits", router_drops_last_column,
                                             [(P.test_router_logits_exact_integers, ())]),
    "FFN: second bias dropped": ("expert_ffn_segment", ffn_without_b2,
                                 [(P.test_expert_ffn_matches_torch_linear_gelu, ())]),
    "FFN: second weight read transposed": ("expert_ffn_segment", ffn_w2_transposed_slice,
                                           [(P.test_expert_ffn_matches_torch_linear_gelu, ())]),
    "loads: off by one": ("expert_loads", loads_off_by_one,
                          [(P.test_expert_loads_match_the_pages_worked_examples, ()),
                           (P.test_expert_loads_against_an_independent_count, ())]),
    "L_aux: alpha dropped": ("aux_loss_terms", aux_without_alpha,
                             [(P.test_aux_loss_closed_forms, ())]),
    "bias update: sign flipped": ("expert_bias_update", bias_update_sign_flipped,
                                  [(P.test_bias_update_closed_forms, ()),
                                   (P.test_bias_update_bit_exact_against_the_pages_torch_expression, ())]),
    "E4M3: input scaled slightly": ("e4m3_encode", e4m3_scaled_slightly,
                                    [(P.test_e4m3_codes_match_torch_float8, ())]),
    "bf16: truncation instead of round-to-nearest-even": ("round_bf16", bf16_truncating,
                                                          [(P.test_round_bf16_special_values_and_torch, ())]),
    "locality: local and cross swapped": ("dispatch_locality", locality_swapped,
                                          [(P.test_ep46_contracts, ())]),
    "plan: balance rounded up": ("recommend_plan", plan_rounds_balance_up,
                                 [(P.test_plan_decision_boundaries, ()),
                                  (P.test_plan_decision_reads_the_stored_3_decimal_balance, ())]),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_a_planted_mistake_fails_a_pin(case, monkeypatch):
    name, mutant, pins = CASES[case]
    monkeypatch.setattr(OM, name, mutant)
    monkeypatch.setattr(O, name, mutant)
    caught = []
    for fn, args in pins:
        try:
            fn(*args)
        except (AssertionError, pytest.fail.Exception):  # a pin's own check failed
            caught.append(fn.__name__)
    assert caught, f"no pin fails with the mistake '{case}' planted in {name}"


def test_the_pins_pass_on_the_oracle_as_it_is():
    """The same pins, unmutated, pass (so a failure above is the mistake's)."""
    for name, _, pins in CASES.values():
        assert getattr(O, name) is ORIG[name]
        for fn, args in pins:
            fn(*args)

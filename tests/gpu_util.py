"""Shared helpers of the GPU parity tests: cached device inputs, oracle
results computed from host copies of the same inputs, and tolerance formulas.

Nothing here computes an expected value from the HIP path: every expected
value comes from `oracle` applied to the seeded inputs."""
from __future__ import annotations

import functools
import math

import numpy as np
import torch

import moe_workloads as W
import oracle as O
from expert_dispatch_combine_amd.runner import LayerBuffers, capacity_of, cfg_from

U32 = 2.0 ** -24  # unit roundoff of fp32


def banner(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


@functools.lru_cache(maxsize=2)
def device_inputs(cid: int, with_experts: bool = True) -> W.Inputs:
    return W.make_inputs(W.CONFIGS[cid], "cuda", with_experts=with_experts)


def custom_inputs(cfg: W.Config, with_experts=True) -> W.Inputs:
    return W.make_inputs(cfg, "cuda", with_experts=with_experts)


def host(t):
    return W.host_f64(t)


def bias_np(inp: W.Inputs):
    return None if inp.logit_bias is None else inp.logit_bias.cpu().numpy()


def oracle_logits(inp: W.Inputs) -> np.ndarray:
    return O.router_logits(host(inp.x), host(inp.w_gate))


def oracle_route(inp: W.Inputs, logits32: np.ndarray):
    cfg = inp.cfg
    idx, gate = O.topk_softmax(logits32, cfg.K, bias_np(inp))
    cap = O.capacity(cfg.T * cfg.K, cfg.E, cfg.cf)
    return idx, gate, cap


def near_tie_tokens(logits32: np.ndarray, bias, K: int, thr: float = 1e-4) -> np.ndarray:
    """Tokens where two consecutive ranks k, k+1 (k = 1..K) of the sorted
    (biased) oracle logits lie within `thr`: their top-k set or slot order is
    not decided at the accuracy of an fp32-accumulated bf16 router product."""
    l = O.add_logit_bias(logits32, bias).astype(np.float64)
    n = min(K + 1, l.shape[1])
    if n < 2:
        return np.zeros(l.shape[0], bool)
    s = -np.sort(-l, axis=1)[:, :n]
    return np.any((s[:, :-1] - s[:, 1:]) < thr, axis=1)


def logit_bound(x64: np.ndarray, wg64: np.ndarray) -> np.ndarray:
    """Rigorous bound of an fp32-accumulated dot product of exactly
    representable products: h * u * sum_j |x_j w_j|."""
    h = x64.shape[1]
    return h * U32 * (np.abs(x64) @ np.abs(wg64).T)


def rms(a) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def buffers_for(cfg: W.Config, device="cuda") -> LayerBuffers:
    mc = cfg_from(cfg)
    return LayerBuffers(mc, capacity_of(mc), device)


def to_dev(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def host_expert(t: torch.Tensor, e: int) -> np.ndarray:
    """Float64 host copy of one expert's slice of a device weight tensor (one
    expert at a time keeps host memory bounded on the 256-expert workload)."""
    return host(t[int(e)])


def check_ffn_segment(h_round: str, xe: np.ndarray, w1, b1, w2, b2, Hg: np.ndarray,
                      Yg: np.ndarray):
    """One expert's H and Y from the GPU against the oracle's
    (O.expert_ffn_segment on the same rows).  Returns the oracle's Y.

    Derived bounds (u = 2^-24, fp32 accumulation of exactly representable
    products; Cauchy-Schwarz bounds each sum |a_j b_j| by ||a|| ||b||):
      pre-activation: |du| <= h u ||x_r|| ||W1_f|| + u |pre|, and
                    |pre| <= ||x_r|| ||W1_f|| + |b1_f|;
      H: one unit of the storage grid (2^-7 |H| for bf16, 2^-23 for fp32)
         plus GELU' (<= 1.13) times |du|;
      Y: ||M_r|| ||W2_n|| + F u ||H_r|| ||W2_n|| + u |Y|, M = the H bound;
      and in RMS, dY below 2^-8 RMS(Y) per expert."""
    H, Y = O.expert_ffn_segment(xe, w1, b1, w2, b2, h_round)
    h = xe.shape[1]
    F = H.shape[1]
    b1 = np.asarray(b1, np.float64)
    nx = np.linalg.norm(xe, axis=1)
    nw1 = np.linalg.norm(w1, axis=1)
    du = (h + 1) * U32 * np.outer(nx, nw1) + U32 * np.abs(b1)[None, :]
    ulp = 2.0 ** -7 if h_round == "bf16" else 2.0 ** -23
    tolH = ulp * np.abs(H) + 1.13 * du + 1e-6
    dH = np.abs(Hg - H)
    assert np.all(dH <= tolH), float((dH - tolH).max())
    if h_round == "bf16":
        assert np.mean(dH > 0) < 0.02
    nw2 = np.linalg.norm(w2, axis=1)
    nM = np.linalg.norm(ulp * np.abs(H) + 1.13 * du, axis=1)
    nH = np.linalg.norm(H, axis=1)
    tolY = np.outer(nM + F * U32 * nH, nw2) + U32 * np.abs(Y) + 1e-6
    dY = np.abs(Yg - Y)
    assert np.all(dY <= tolY), float((dY - tolY).max())
    assert rms(Yg - Y) <= 2.0 ** -8 * rms(Y) + 1e-7
    return Y


INT_FIELDS = ["total_tokens", "total_routes", "capacity", "accepted_routes", "overflow",
              "max_load", "logical_route_bytes", "all_to_all_bytes", "accepted_route_bytes",
              "local_routes", "cross_rank_routes", "cross_rank_dispatch_bytes",
              "cross_rank_roundtrip_bytes", "accepted_local_routes",
              "accepted_cross_rank_routes", "accepted_cross_rank_dispatch_bytes",
              "accepted_cross_rank_roundtrip_bytes"]
EXACT_FLOATS = ["balance_ratio", "local_hit_ratio", "accepted_local_hit_ratio",
                "pair_bytes_uniform"]


def compare_ledger(g: dict, o: dict) -> None:
    """A decoded GPU ledger against O.ledger of the same routing: integer
    fields and the float64 values computed from them equal; P (fixed-point
    gate sums on the device, each gate rounded to a multiple of 2^-32) within
    load_e * 2^-33 / T, and L_aux within alpha * sum_e f_e * that bound."""
    for k in INT_FIELDS:
        assert g[k] == o[k], (k, g[k], o[k])
    for k in EXACT_FLOATS:
        assert g[k] == o[k], (k, g[k], o[k])
    assert g["loads"] == [int(v) for v in o["expert_loads"]]
    assert np.array_equal(np.array(g["f"]), o["f"])
    T = max(o["total_tokens"], 1)
    dP = np.asarray(o["expert_loads"], np.float64) * 2.0 ** -33 / T + 1e-15 * np.abs(o["P"])
    assert np.all(np.abs(np.array(g["P"]) - o["P"]) <= dP)
    d_aux = g["alpha"] * float(np.sum(np.asarray(o["f"]) * dP)) + 1e-15 * abs(o["l_aux"])
    assert abs(g["l_aux"] - o["l_aux"]) <= d_aux
    scale = o["num_experts"] / max(o["total_routes"] / T, 1)  # E / K
    assert abs(g["l_aux_norm"] - o["l_aux_norm"]) <= scale * d_aux + 1e-15 * abs(o["l_aux_norm"])
    np.testing.assert_allclose(g["load_var_over_mean"], o["load_var_over_mean"], rtol=1e-12)
    assert bool(g["imbalanced"]) == o["imbalanced"]
    assert np.array_equal(np.array(g["pair_routes"]), o["pair_routes"])

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

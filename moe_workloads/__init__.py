"""Seeded synthetic workloads for the MoE route -> dispatch -> FFN -> combine path.

This module only *draws inputs*: shapes, seeds and value distributions.  It holds
none of the method's arithmetic (no routing, capacity, slotting, FFN or combine),
so both the CPU oracle's tests and the GPU library's tests/bench can use it
without sharing any implementation with each other.

Shapes follow the layer shapes the pages name: a Switch-Base-like layer and the
DeepSeek-V3 all-to-all example in the "通信量分析" table of "专家并行（Expert
Parallelism）", the Mixtral 8-expert top-2 example of "MoE 与专家并行", and the
256-expert top-8 layer of "MoE大模型专家并行与动态路由优化" (section 一).

Recipe (every tensor has its own seed, derived from the workload seed):
  x ~ N(0, 1);  W_g, W1 ~ N(0, 1/h);  W2 ~ N(0, 1/F);  b1, b2 ~ N(0, 0.01)
  (0.01 is the variance, i.e. std 0.1).  Values are drawn in fp32 and rounded
  to bf16 (round-to-nearest-even, torch's conversion) for bf16 workloads;
  biases stay fp32.  The hot-expert workload adds a per-expert router-logit
  bias  -s*ln(pi(e)+1), s = 1.2, with pi a seeded permutation of the experts
  (a log-Zipf popularity profile; the Zipf normaliser is a uniform shift and
  is dropped).
Token source ranks: t % N_EP (round robin), or floor(t*N_EP/T) (contiguous
blocks) for the hot-expert workload.  Expert owner ranks: e % N_EP.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "custom", "make_inputs", "Inputs", "host_f64",
           "seed_for", "ROUTING_SCENARIOS", "SCENARIO_CONFIG", "scenario_logits"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    h: int
    E: int
    K: int
    F: int
    cf: float
    dtype: str            # "f32" or "bf16"
    n_ep: int
    src_rank: str = "mod"  # "mod": t % n_ep ; "block": floor(t * n_ep / T)
    zipf_s: Optional[float] = None
    seed: int = 0

    @property
    def bytes_per_elem(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def A(self) -> int:
        return self.T * self.K


CONFIGS = {
    1: Config("tiny-fp32", T=64, h=32, E=4, K=2, F=64, cf=1.0, dtype="f32",
              n_ep=2, src_rank="mod", seed=1001),
    2: Config("switch-base-bf16", T=2048, h=768, E=16, K=1, F=3072, cf=1.25,
              dtype="bf16", n_ep=16, src_rank="mod", seed=1002),
    3: Config("mixtral-bf16", T=4096, h=4096, E=8, K=2, F=14336, cf=1.25,
              dtype="bf16", n_ep=4, src_rank="mod", seed=1003),
    4: Config("deepseek-v3-bf16", T=4096, h=7168, E=256, K=8, F=2048, cf=1.0,
              dtype="bf16", n_ep=8, src_rank="mod", seed=1004),
    5: Config("hot-expert-bf16", T=16384, h=2048, E=64, K=6, F=1408, cf=1.0,
              dtype="bf16", n_ep=8, src_rank="block", zipf_s=1.2, seed=1005),
}


def custom(T, h, E, K, F, cf=1.0, dtype="bf16", n_ep=2, src_rank="mod",
           zipf_s=None, seed=7, name="custom") -> Config:
    return Config(name, T=T, h=h, E=E, K=K, F=F, cf=cf, dtype=dtype, n_ep=n_ep,
                  src_rank=src_rank, zipf_s=zipf_s, seed=seed)


# tensor ids: one child stream per tensor (and per expert for W1/W2)
_TID = {"x": 0, "w_gate": 1, "w1": 2, "b1": 3, "w2": 4, "b2": 5, "perm": 6, "logits": 7}


def seed_for(seed: int, tensor: str, expert: int = -1) -> int:
    """64-bit seed of one tensor's (or one expert slice's) own stream."""
    ss = np.random.SeedSequence([seed, _TID[tensor], expert + 1])
    return int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def _normal(shape, std, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


@dataclasses.dataclass
class Inputs:
    cfg: Config
    x: torch.Tensor            # [T, h]   f32 or bf16
    w_gate: torch.Tensor       # [E, h]
    w1: torch.Tensor           # [E, F, h]
    b1: torch.Tensor           # [E, F]   f32
    w2: torch.Tensor           # [E, h, F]
    b2: torch.Tensor           # [E, h]   f32
    logit_bias: Optional[torch.Tensor]  # [E] f32 or None
    src_rank: torch.Tensor     # [T] int32
    owner_rank: torch.Tensor   # [E] int32


def make_inputs(cfg: Config, device="cpu", with_experts: bool = True) -> Inputs:
    """Draw every tensor of one workload on `device` (seeded, reproducible)."""
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    T, h, E, F = cfg.T, cfg.h, cfg.E, cfg.F
    s = cfg.seed
    # router inputs are drawn on the CPU (device-independent values, so the
    # routing can be reproduced anywhere); expert weights on `device`
    x = _normal((T, h), 1.0, seed_for(s, "x"), "cpu").to(dt).to(device)
    w_gate = _normal((E, h), 1.0 / math.sqrt(h), seed_for(s, "w_gate"), "cpu").to(dt).to(device)
    if with_experts:
        w1 = torch.empty((E, F, h), dtype=dt, device=device)
        w2 = torch.empty((E, h, F), dtype=dt, device=device)
        for e in range(E):
            w1[e] = _normal((F, h), 1.0 / math.sqrt(h), seed_for(s, "w1", e), device).to(dt)
            w2[e] = _normal((h, F), 1.0 / math.sqrt(F), seed_for(s, "w2", e), device).to(dt)
        b1 = _normal((E, F), 0.1, seed_for(s, "b1"), device)
        b2 = _normal((E, h), 0.1, seed_for(s, "b2"), device)
    else:
        w1 = w2 = b1 = b2 = None
    logit_bias = None
    if cfg.zipf_s is not None:
        g = torch.Generator(device="cpu")
        g.manual_seed(seed_for(s, "perm"))
        perm = torch.randperm(E, generator=g)
        logit_bias = (-cfg.zipf_s * torch.log(perm.to(torch.float64) + 1.0)).to(
            torch.float32).to(device)
    t = torch.arange(T, dtype=torch.int64)
    if cfg.src_rank == "mod":
        src = t % cfg.n_ep
    else:
        src = (t * cfg.n_ep) // max(T, 1)
    owner = torch.arange(E, dtype=torch.int64) % cfg.n_ep
    return Inputs(cfg, x, w_gate, w1, b1, w2, b2, logit_bias,
                  src.to(torch.int32).to(device), owner.to(torch.int32).to(device))


def host_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact float64 host copy of a stored tensor (bf16/f32 widen exactly)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# routing scenarios of the expert-parallel mechanism benchmark
# ----------------------------------------------------------------------------
# "46. MoE Expert Parallel" Step 5 fixes the workload (2 ranks, 256 tokens per
# rank, hidden 1024, 4 experts, top-2, capacity factor 1.25, bf16) and varies
# only the routing: local-heavy, balanced, skewed.  The page does not say how
# each routing is drawn; here the router logits are seeded N(0, 1) plus a
# per-scenario bias: +4 on the experts owned by the token's source rank
# (local_heavy), none (balanced), +3 on expert 0 (skewed).  Experts are owned
# round robin (e % 2); tokens come from ranks in contiguous blocks of 256.
# The FFN width (not given) is 4 * hidden.
ROUTING_SCENARIOS = ("local_heavy", "balanced", "skewed")
SCENARIO_CONFIG = Config("ep-mechanism-bf16", T=512, h=1024, E=4, K=2, F=4096, cf=1.25,
                         dtype="bf16", n_ep=2, src_rank="block", seed=1046)


def scenario_logits(name: str, cfg: Config = SCENARIO_CONFIG) -> np.ndarray:
    """fp32 router logits [T, E] of one routing scenario (seeded)."""
    if name not in ROUTING_SCENARIOS:
        raise ValueError(f"unknown routing scenario {name!r}")
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(cfg.seed, "logits", ROUTING_SCENARIOS.index(name)))
    logits = torch.randn((cfg.T, cfg.E), generator=g, dtype=torch.float32)
    t = torch.arange(cfg.T)
    src = (t * cfg.n_ep) // cfg.T
    owner = torch.arange(cfg.E) % cfg.n_ep
    if name == "local_heavy":
        logits += 4.0 * (owner[None, :] == src[:, None]).to(torch.float32)
    elif name == "skewed":
        logits[:, 0] += 3.0
    return logits.numpy()


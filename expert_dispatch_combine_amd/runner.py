"""Device buffers for one MoE layer and the call sequence of the C ABI.

`LayerBuffers` allocates every output/scratch tensor the five entry points
need (sizes from moe_max_rows / moe_workspace_bytes); `run_layer` issues
moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine on one stream.
No arithmetic of the method happens here.
"""
from __future__ import annotations

import torch

from ._binding import (MOE_BF16, MoeCfg, moe_capacity, moe_combine, moe_dispatch,
                       moe_expert_ffn, moe_ledger, moe_max_rows, moe_route,
                       moe_workspace_bytes)


class LayerBuffers:
    def __init__(self, cfg: MoeCfg, capacity: int, device="cuda"):
        T, h, E, K, F = cfg.T, cfg.h, cfg.E, cfg.K, cfg.F
        act = torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32
        i32, f32 = torch.int32, torch.float32
        self.cfg = cfg
        self.capacity = int(capacity)
        self.r_max = moe_max_rows(cfg, capacity)
        rm = max(self.r_max, 1)
        self.logits = torch.empty((T, E), dtype=f32, device=device)
        self.topk_idx = torch.empty((T, K), dtype=i32, device=device)
        self.topk_gate = torch.empty((T, K), dtype=f32, device=device)
        self.expert_load = torch.empty((E,), dtype=i32, device=device)
        self.expert_offsets = torch.empty((E + 1,), dtype=i32, device=device)
        self.route_rank = torch.empty((T, K), dtype=i32, device=device)
        self.route_row = torch.empty((T, K), dtype=i32, device=device)
        self.row_token = torch.empty((rm,), dtype=i32, device=device)
        self.x_disp = torch.empty((rm, h), dtype=act, device=device)
        self.h_buf = torch.empty((rm, F), dtype=act, device=device)
        self.y = torch.empty((rm, h), dtype=f32, device=device)
        self.out = torch.empty((T, h), dtype=f32, device=device)
        self.ws = torch.empty((moe_workspace_bytes(cfg),), dtype=torch.uint8, device=device)


def cfg_from(workload) -> MoeCfg:
    """MoeCfg of a moe_workloads.Config."""
    return MoeCfg.make(workload.T, workload.h, workload.E, workload.K, workload.F,
                       workload.dtype, workload.cf)


def capacity_of(cfg: MoeCfg) -> int:
    return moe_capacity(cfg.T * cfg.K, cfg.E, cfg.capacity_factor)


def run_route(b: LayerBuffers, x, w_gate, logit_bias=None, expert_load=True, stream=None):
    moe_route(b.cfg, x, w_gate, logit_bias, b.logits, b.topk_idx, b.topk_gate,
              b.expert_load if expert_load else None, b.ws, stream)


def run_dispatch(b: LayerBuffers, x, expert_load=False, stream=None):
    moe_dispatch(b.cfg, x, b.topk_idx, b.capacity, b.expert_offsets, b.route_rank, b.route_row,
                 b.row_token, b.x_disp, b.expert_load if expert_load else None, b.ws, stream)


def run_ffn(b: LayerBuffers, w1, b1, w2, b2, stream=None):
    moe_expert_ffn(b.cfg, b.capacity, b.x_disp, b.expert_offsets, w1, b1, w2, b2, b.h_buf, b.y,
                   stream)


def run_combine(b: LayerBuffers, stream=None):
    moe_combine(b.cfg, b.y, b.route_row, b.topk_gate, b.out, stream)


def run_ledger(b: LayerBuffers, src_rank, owner_rank, n_ep, alpha=0.01, stream=None, **kw):
    return moe_ledger(b.cfg, b.topk_idx, b.topk_gate, b.route_row, b.capacity, src_rank,
                      owner_rank, n_ep, alpha, b.ws, stream, **kw)


def run_layer(b: LayerBuffers, x, w_gate, logit_bias, w1, b1, w2, b2, stream=None):
    """route -> dispatch -> expert FFN -> combine (asynchronous on `stream`)."""
    run_route(b, x, w_gate, logit_bias, expert_load=False, stream=stream)
    run_dispatch(b, x, expert_load=True, stream=stream)
    run_ffn(b, w1, b1, w2, b2, stream=stream)
    run_combine(b, stream=stream)

"""expert_dispatch_combine_amd: one MoE layer hot path on an MI355X (gfx950).

route -> capacity-limited dispatch -> expert FFN -> weighted combine, plus a
counters-only ledger, implemented as hand-written HIP kernels behind the C ABI
of include/moe.h (libmoe.so).  This module is the thin Python binding: it only
marshals torch tensors (device memory) and the current HIP stream into the C
calls, which have the same names.  Every step of the path runs in the library;
there is no fallback: if libmoe.so is missing or fails to load, every call
raises.
"""
from ._binding import (  # noqa: F401
    EXPORTED_SYMBOLS, MOE_BF16, MOE_F32, MoeCfg, MoeError, MoeLedger, library_path,
    load_library, moe_bias_update, moe_capacity, moe_combine, moe_combine_ledger, moe_dispatch,
    moe_dispatch_noalloc, moe_dispatch_fp8, moe_expert_rank_affinity, moe_place_experts,
    moe_expert_ffn_fp8, moe_expert_ffn, moe_fp8_dequantize, moe_fp8_scale, moe_recommend_plan, PLAN_NAMES,
    moe_expert_ffn_packed, moe_expert_ffn_rows, moe_ledger, moe_ledger_finalize,
    moe_ledger_launch,
    moe_ledger_stage_bytes, moe_max_rows, moe_pack_expert_weights, moe_route,
    moe_status_string, moe_workspace_bytes,
)

__all__ = [
    "EXPORTED_SYMBOLS", "MOE_BF16", "MOE_F32", "MoeCfg", "MoeError", "MoeLedger",
    "library_path", "load_library", "moe_bias_update", "moe_capacity", "moe_combine",
    "moe_combine_ledger",
    "moe_dispatch", "moe_dispatch_noalloc", "moe_dispatch_fp8", "moe_fp8_dequantize",
    "moe_expert_rank_affinity", "moe_place_experts", "moe_expert_ffn_fp8",
    "moe_fp8_scale",
    "moe_recommend_plan", "PLAN_NAMES",
    "moe_expert_ffn", "moe_expert_ffn_packed", "moe_expert_ffn_rows", "moe_ledger",
    "moe_ledger_finalize",
    "moe_ledger_launch", "moe_ledger_stage_bytes", "moe_max_rows", "moe_pack_expert_weights",
    "moe_route", "moe_status_string", "moe_workspace_bytes",
]

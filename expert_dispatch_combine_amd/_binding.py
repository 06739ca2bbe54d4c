"""ctypes binding of libmoe.so (argument marshalling only).

Each function takes torch tensors (or None for optional arguments), checks
that they are contiguous device tensors of the expected dtype, and passes
their device pointers, the shape struct and the current HIP stream to the C
function of the same name (see include/moe.h for the contracts).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads the HIP runtime that libmoe then binds to

MOE_F32 = 0
MOE_BF16 = 1

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoe.so"

EXPORTED_SYMBOLS = (
    "moe_status_string", "moe_capacity", "moe_max_rows", "moe_workspace_bytes",
    "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_ledger",
    "moe_ledger_stage_bytes", "moe_ledger_launch", "moe_ledger_finalize",
    "moe_dispatch_noalloc", "moe_expert_rank_affinity", "moe_place_experts",
    "moe_expert_ffn_fp8",
    "moe_expert_ffn_packed", "moe_pack_expert_weights", "moe_bias_update",
    "moe_fp8_scale", "moe_dispatch_fp8", "moe_fp8_dequantize", "moe_recommend_plan",
    "moe_combine_ledger", "moe_expert_ffn_rows",
)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {moe_status_string(status)} ({status})")


class MoeCfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("h", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("F", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity_factor", ctypes.c_double)]

    @classmethod
    def make(cls, T, h, E, K, F, dtype, capacity_factor):
        if isinstance(dtype, str):
            dtype = MOE_BF16 if dtype == "bf16" else MOE_F32
        return cls(int(T), int(h), int(E), int(K), int(F), int(dtype), float(capacity_factor))


_I64 = ctypes.c_int64
_F64 = ctypes.c_double


class MoeLedger(ctypes.Structure):
    _fields_ = [(n, _I64) for n in (
        "total_tokens", "total_routes", "num_experts", "capacity", "accepted_routes",
        "overflow", "max_load", "invalid_routes", "logical_route_bytes", "all_to_all_bytes",
        "accepted_route_bytes", "local_routes", "cross_rank_routes",
        "cross_rank_dispatch_bytes", "cross_rank_roundtrip_bytes", "accepted_local_routes",
        "accepted_cross_rank_routes", "accepted_cross_rank_dispatch_bytes",
        "accepted_cross_rank_roundtrip_bytes", "n_ep")] + [(n, _F64) for n in (
        "balance_ratio", "local_hit_ratio", "accepted_local_hit_ratio", "pair_bytes_uniform",
        "l_aux", "l_aux_norm", "alpha", "load_var_over_mean")] + [
        ("imbalanced", ctypes.c_int32), ("status", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def library_path() -> str:
    return os.environ.get("MOE_LIBRARY", os.path.join(_PKG, _LIB_NAME))


def load_library():
    """Load libmoe.so once; raise if it is missing (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with "
                           "`python -m expert_dispatch_combine_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(MoeCfg)
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_capacity.restype = _I64
    lib.moe_capacity.argtypes = [_I64, ctypes.c_int32, _F64]
    lib.moe_max_rows.restype = _I64
    lib.moe_max_rows.argtypes = [cfgp, _I64]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_bytes.argtypes = [cfgp]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route.argtypes = [cfgp, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_dispatch.restype = ctypes.c_int
    lib.moe_dispatch.argtypes = [cfgp, P, P, _I64, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_dispatch_noalloc.restype = ctypes.c_int
    lib.moe_dispatch_noalloc.argtypes = [cfgp, P, P, _I64, P, P, P, P, P, P, P]
    lib.moe_expert_ffn.restype = ctypes.c_int
    lib.moe_expert_ffn.argtypes = [cfgp, _I64, P, P, P, P, P, P, P, P, P]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_combine.argtypes = [cfgp, P, P, P, P, P]
    lib.moe_ledger.restype = ctypes.c_int
    lib.moe_ledger.argtypes = [cfgp, P, P, P, _I64, P, P, ctypes.c_int32, _F64,
                               ctypes.POINTER(MoeLedger), P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_ledger_stage_bytes.restype = ctypes.c_size_t
    lib.moe_ledger_stage_bytes.argtypes = [cfgp, ctypes.c_int32]
    lib.moe_ledger_launch.restype = ctypes.c_int
    lib.moe_ledger_launch.argtypes = [cfgp, P, P, P, P, P, ctypes.c_int32, P, ctypes.c_size_t,
                                      P, ctypes.c_size_t, P]
    lib.moe_combine_ledger.restype = ctypes.c_int
    lib.moe_combine_ledger.argtypes = [cfgp, P, P, P, P, P, P, P, ctypes.c_int32, P,
                                       ctypes.c_size_t, P, ctypes.c_size_t, P]
    lib.moe_ledger_finalize.restype = ctypes.c_int
    lib.moe_ledger_finalize.argtypes = [cfgp, _I64, ctypes.c_int32, _F64, P,
                                        ctypes.POINTER(MoeLedger), P, P, P, P]
    lib.moe_expert_ffn_rows.restype = ctypes.c_int
    lib.moe_expert_ffn_rows.argtypes = [cfgp, _I64, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P]
    lib.moe_expert_ffn_packed.restype = ctypes.c_int
    lib.moe_expert_ffn_packed.argtypes = [cfgp, _I64, P, P, P, P, P, P, P, P, P]
    lib.moe_pack_expert_weights.restype = ctypes.c_int
    lib.moe_pack_expert_weights.argtypes = [cfgp, P, P, P, P, P]
    lib.moe_bias_update.restype = ctypes.c_int
    lib.moe_bias_update.argtypes = [cfgp, P, P, ctypes.c_float, P, P]
    lib.moe_fp8_scale.restype = ctypes.c_int
    lib.moe_fp8_scale.argtypes = [cfgp, P, P, P, ctypes.c_size_t, P]
    lib.moe_dispatch_fp8.restype = ctypes.c_int
    lib.moe_dispatch_fp8.argtypes = [cfgp, P, P, P, _I64, P, P, P, P, P, P, P, ctypes.c_size_t,
                                     P]
    lib.moe_recommend_plan.restype = ctypes.c_int
    lib.moe_recommend_plan.argtypes = [ctypes.POINTER(MoeLedger), ctypes.POINTER(_F64),
                                       ctypes.c_int32]
    lib.moe_expert_ffn_fp8.restype = ctypes.c_int
    lib.moe_expert_ffn_fp8.argtypes = [cfgp, _I64, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P]
    lib.moe_expert_rank_affinity.restype = ctypes.c_int
    lib.moe_expert_rank_affinity.argtypes = [cfgp, P, P, P, ctypes.c_int32, P, P]
    lib.moe_place_experts.restype = ctypes.c_int
    lib.moe_place_experts.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P]
    lib.moe_fp8_dequantize.restype = ctypes.c_int
    lib.moe_fp8_dequantize.argtypes = [cfgp, _I64, P, P, P, P, P]
    _lib = lib
    return lib


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(int(status)).decode()


# ----------------------------------------------------------------- marshalling
_WANT = {
    "act": None,  # activation dtype: checked against cfg.dtype
    "f32": torch.float32,
    "i32": torch.int32,
    "u8": torch.uint8,
}


def _act_dtype(cfg: MoeCfg):
    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor], kind: str, cfg: MoeCfg, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    want = _act_dtype(cfg) if kind == "act" else _WANT[kind]
    if t.dtype != want:
        raise ValueError(f"{name}: expected {want}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("ws: expected a contiguous device tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


# ----------------------------------------------------------------- entry points
def moe_capacity(A: int, E: int, capacity_factor: float) -> int:
    return int(load_library().moe_capacity(int(A), int(E), float(capacity_factor)))


def moe_max_rows(cfg: MoeCfg, capacity: int) -> int:
    return int(load_library().moe_max_rows(ctypes.byref(cfg), int(capacity)))


def moe_workspace_bytes(cfg: MoeCfg) -> int:
    return int(load_library().moe_workspace_bytes(ctypes.byref(cfg)))


def moe_route(cfg: MoeCfg, x, w_gate, logit_bias, logits, topk_idx, topk_gate,
              expert_load=None, ws=None, stream=None) -> None:
    lib = load_library()
    wsp, wsb = _ws(ws)
    st = lib.moe_route(ctypes.byref(cfg), _ptr(x, "act", cfg, "x"),
                       _ptr(w_gate, "act", cfg, "w_gate"), _ptr(logit_bias, "f32", cfg, "logit_bias"),
                       _ptr(logits, "f32", cfg, "logits"), _ptr(topk_idx, "i32", cfg, "topk_idx"),
                       _ptr(topk_gate, "f32", cfg, "topk_gate"),
                       _ptr(expert_load, "i32", cfg, "expert_load"), wsp, wsb, _stream(stream))
    _check("moe_route", st)


def moe_bias_update(cfg: MoeCfg, topk_idx, expert_bias, alpha: float = 0.1, counts=None,
                    stream=None) -> None:
    """expert_bias (fp32 [E], device) += alpha * (mean_count - count), in place."""
    lib = load_library()
    st = lib.moe_bias_update(ctypes.byref(cfg), _ptr(topk_idx, "i32", cfg, "topk_idx"),
                             _ptr(expert_bias, "f32", cfg, "expert_bias"), float(alpha),
                             _ptr(counts, "i32", cfg, "counts"), _stream(stream))
    _check("moe_bias_update", st)


def moe_fp8_scale(cfg: MoeCfg, x, scale, ws, stream=None) -> None:
    """scale[0] = bf16(max|x| / 448) (fp32 device tensor of one element)."""
    lib = load_library()
    wsp, wsb = _ws(ws)
    st = lib.moe_fp8_scale(ctypes.byref(cfg), _ptr(x, "act", cfg, "x"),
                           _ptr(scale, "f32", cfg, "scale"), wsp, wsb, _stream(stream))
    _check("moe_fp8_scale", st)


def moe_dispatch_fp8(cfg: MoeCfg, x, scale, topk_idx, capacity: int, expert_offsets,
                     route_rank, route_row, row_token, x_disp_q, expert_load=None, ws=None,
                     stream=None) -> None:
    """moe_dispatch sending E4M3 codes: x_disp_q is a uint8 [R_max, h] tensor."""
    lib = load_library()
    wsp, wsb = _ws(ws)
    st = lib.moe_dispatch_fp8(ctypes.byref(cfg), _ptr(x, "act", cfg, "x"),
                              _ptr(scale, "f32", cfg, "scale"),
                              _ptr(topk_idx, "i32", cfg, "topk_idx"), int(capacity),
                              _ptr(expert_offsets, "i32", cfg, "expert_offsets"),
                              _ptr(route_rank, "i32", cfg, "route_rank"),
                              _ptr(route_row, "i32", cfg, "route_row"),
                              _ptr(row_token, "i32", cfg, "row_token"),
                              _ptr(x_disp_q, "u8", cfg, "x_disp_q"),
                              _ptr(expert_load, "i32", cfg, "expert_load"), wsp, wsb,
                              _stream(stream))
    _check("moe_dispatch_fp8", st)


def moe_fp8_dequantize(cfg: MoeCfg, capacity: int, x_disp_q, scale, expert_offsets, x_disp,
                       stream=None) -> None:
    """x_disp[r] = bf16(value(x_disp_q[r]) * scale) for the accepted rows."""
    lib = load_library()
    st = lib.moe_fp8_dequantize(ctypes.byref(cfg), int(capacity),
                                _ptr(x_disp_q, "u8", cfg, "x_disp_q"),
                                _ptr(scale, "f32", cfg, "scale"),
                                _ptr(expert_offsets, "i32", cfg, "expert_offsets"),
                                _ptr(x_disp, "act", cfg, "x_disp"), _stream(stream))
    _check("moe_fp8_dequantize", st)


def moe_dispatch_noalloc(cfg: MoeCfg, x, topk_idx, capacity: int, expert_offsets, route_rank,
                         route_row, row_token, x_disp, expert_load=None, stream=None) -> None:
    """moe_dispatch with its scratch in the library's static device array (no
    workspace argument, nothing allocated); see include/moe.h."""
    lib = load_library()
    st = lib.moe_dispatch_noalloc(ctypes.byref(cfg), _ptr(x, "act", cfg, "x"),
                                  _ptr(topk_idx, "i32", cfg, "topk_idx"), int(capacity),
                                  _ptr(expert_offsets, "i32", cfg, "expert_offsets"),
                                  _ptr(route_rank, "i32", cfg, "route_rank"),
                                  _ptr(route_row, "i32", cfg, "route_row"),
                                  _ptr(row_token, "i32", cfg, "row_token"),
                                  _ptr(x_disp, "act", cfg, "x_disp"),
                                  _ptr(expert_load, "i32", cfg, "expert_load"), _stream(stream))
    _check("moe_dispatch_noalloc", st)


def moe_dispatch(cfg: MoeCfg, x, topk_idx, capacity: int, expert_offsets, route_rank,
                 route_row, row_token, x_disp, expert_load=None, ws=None, stream=None) -> None:
    lib = load_library()
    wsp, wsb = _ws(ws)
    st = lib.moe_dispatch(ctypes.byref(cfg), _ptr(x, "act", cfg, "x"),
                          _ptr(topk_idx, "i32", cfg, "topk_idx"), int(capacity),
                          _ptr(expert_offsets, "i32", cfg, "expert_offsets"),
                          _ptr(route_rank, "i32", cfg, "route_rank"),
                          _ptr(route_row, "i32", cfg, "route_row"),
                          _ptr(row_token, "i32", cfg, "row_token"),
                          _ptr(x_disp, "act", cfg, "x_disp"),
                          _ptr(expert_load, "i32", cfg, "expert_load"), wsp, wsb,
                          _stream(stream))
    _check("moe_dispatch", st)


def moe_expert_ffn(cfg: MoeCfg, capacity: int, x_disp, expert_offsets, w1, b1, w2, b2, h_buf,
                   y, stream=None) -> None:
    lib = load_library()
    st = lib.moe_expert_ffn(ctypes.byref(cfg), int(capacity), _ptr(x_disp, "act", cfg, "x_disp"),
                            _ptr(expert_offsets, "i32", cfg, "expert_offsets"),
                            _ptr(w1, "act", cfg, "w1"), _ptr(b1, "f32", cfg, "b1"),
                            _ptr(w2, "act", cfg, "w2"), _ptr(b2, "f32", cfg, "b2"),
                            _ptr(h_buf, "act", cfg, "h_buf"), _ptr(y, "f32", cfg, "y"),
                            _stream(stream))
    _check("moe_expert_ffn", st)


def moe_expert_ffn_packed(cfg: MoeCfg, capacity: int, x_disp, expert_offsets, w1_packed, b1,
                          w2_packed, b2, h_buf, y, stream=None) -> None:
    lib = load_library()
    st = lib.moe_expert_ffn_packed(ctypes.byref(cfg), int(capacity),
                                   _ptr(x_disp, "act", cfg, "x_disp"),
                                   _ptr(expert_offsets, "i32", cfg, "expert_offsets"),
                                   _ptr(w1_packed, "act", cfg, "w1_packed"),
                                   _ptr(b1, "f32", cfg, "b1"),
                                   _ptr(w2_packed, "act", cfg, "w2_packed"),
                                   _ptr(b2, "f32", cfg, "b2"), _ptr(h_buf, "act", cfg, "h_buf"),
                                   _ptr(y, "f32", cfg, "y"), _stream(stream))
    _check("moe_expert_ffn_packed", st)


def moe_expert_ffn_rows(cfg: MoeCfg, capacity: int, x, row_token, expert_offsets, w1, b1, w2,
                        b2, h_buf, y, packed: bool = False, stream=None) -> None:
    """The expert FFN on x[row_token[r]] (the dispatch gather done by the FFN)."""
    lib = load_library()
    st = lib.moe_expert_ffn_rows(ctypes.byref(cfg), int(capacity), _ptr(x, "act", cfg, "x"),
                                 _ptr(row_token, "i32", cfg, "row_token"),
                                 _ptr(expert_offsets, "i32", cfg, "expert_offsets"),
                                 _ptr(w1, "act", cfg, "w1"), _ptr(b1, "f32", cfg, "b1"),
                                 _ptr(w2, "act", cfg, "w2"), _ptr(b2, "f32", cfg, "b2"),
                                 _ptr(h_buf, "act", cfg, "h_buf"), _ptr(y, "f32", cfg, "y"),
                                 int(bool(packed)), _stream(stream))
    _check("moe_expert_ffn_rows", st)


def moe_pack_expert_weights(cfg: MoeCfg, w1, w2, w1_packed, w2_packed, stream=None) -> None:
    lib = load_library()
    st = lib.moe_pack_expert_weights(ctypes.byref(cfg), _ptr(w1, "act", cfg, "w1"),
                                     _ptr(w2, "act", cfg, "w2"),
                                     _ptr(w1_packed, "act", cfg, "w1_packed"),
                                     _ptr(w2_packed, "act", cfg, "w2_packed"), _stream(stream))
    _check("moe_pack_expert_weights", st)


def moe_combine(cfg: MoeCfg, y, route_row, topk_gate, out, stream=None) -> None:
    lib = load_library()
    st = lib.moe_combine(ctypes.byref(cfg), _ptr(y, "f32", cfg, "y"),
                         _ptr(route_row, "i32", cfg, "route_row"),
                         _ptr(topk_gate, "f32", cfg, "topk_gate"), _ptr(out, "f32", cfg, "out"),
                         _stream(stream))
    _check("moe_combine", st)


def moe_ledger(cfg: MoeCfg, topk_idx, topk_gate, route_row, capacity: int, src_rank,
               owner_rank, n_ep: int, alpha: float = 0.01, ws=None, stream=None,
               raise_on_error: bool = True) -> dict:
    """Returns the ledger fields plus 'loads', 'f', 'P' (lists) and
    'pair_routes' (n_ep x n_ep nested list); synchronises the stream."""
    lib = load_library()
    wsp, wsb = _ws(ws)
    E = int(cfg.E)
    out = MoeLedger()
    out.status = -1  # moe_ledger fills `out` (status included) only once it has counted
    loads = (_I64 * E)()
    f = (_F64 * E)()
    P = (_F64 * E)()
    pair = (_I64 * (n_ep * n_ep))()
    st = lib.moe_ledger(ctypes.byref(cfg), _ptr(topk_idx, "i32", cfg, "topk_idx"),
                        _ptr(topk_gate, "f32", cfg, "topk_gate"),
                        _ptr(route_row, "i32", cfg, "route_row"), int(capacity),
                        _ptr(src_rank, "i32", cfg, "src_rank"),
                        _ptr(owner_rank, "i32", cfg, "owner_rank"), int(n_ep), float(alpha),
                        ctypes.byref(out), loads, f, P, pair, wsp, wsb, _stream(stream))
    if st != 0 and (raise_on_error or st not in (2, 1) or out.status != st):
        raise MoeError("moe_ledger", st)
    d = out.as_dict()
    d["loads"] = list(loads)
    d["f"] = list(f)
    d["P"] = list(P)
    d["pair_routes"] = [list(pair[i * n_ep:(i + 1) * n_ep]) for i in range(n_ep)]
    d["return_status"] = st
    return d


def moe_ledger_stage_bytes(cfg: MoeCfg, n_ep: int) -> int:
    return int(load_library().moe_ledger_stage_bytes(ctypes.byref(cfg), int(n_ep)))


def _host_ptr(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous host tensor")
    return ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size()


def moe_ledger_launch(cfg: MoeCfg, topk_idx, topk_gate, route_row, src_rank, owner_rank,
                      n_ep: int, host_stage: torch.Tensor, ws=None, stream=None) -> None:
    """Enqueue the ledger's kernels and the copy of its counters into
    `host_stage` (a page-locked host tensor of moe_ledger_stage_bytes bytes)."""
    lib = load_library()
    wsp, wsb = _ws(ws)
    hp, hb = _host_ptr(host_stage, "host_stage")
    st = lib.moe_ledger_launch(ctypes.byref(cfg), _ptr(topk_idx, "i32", cfg, "topk_idx"),
                               _ptr(topk_gate, "f32", cfg, "topk_gate"),
                               _ptr(route_row, "i32", cfg, "route_row"),
                               _ptr(src_rank, "i32", cfg, "src_rank"),
                               _ptr(owner_rank, "i32", cfg, "owner_rank"), int(n_ep), hp, hb,
                               wsp, wsb, _stream(stream))
    _check("moe_ledger_launch", st)


def moe_combine_ledger(cfg: MoeCfg, y, route_row, topk_gate, out, topk_idx, src_rank,
                       owner_rank, n_ep: int, host_stage: torch.Tensor, ws=None,
                       stream=None) -> None:
    """moe_combine and moe_ledger_launch in one call (one launch up to 4096
    routes); `host_stage` as for moe_ledger_launch."""
    lib = load_library()
    wsp, wsb = _ws(ws)
    hp, hb = _host_ptr(host_stage, "host_stage")
    st = lib.moe_combine_ledger(ctypes.byref(cfg), _ptr(y, "f32", cfg, "y"),
                                _ptr(route_row, "i32", cfg, "route_row"),
                                _ptr(topk_gate, "f32", cfg, "topk_gate"),
                                _ptr(out, "f32", cfg, "out"),
                                _ptr(topk_idx, "i32", cfg, "topk_idx"),
                                _ptr(src_rank, "i32", cfg, "src_rank"),
                                _ptr(owner_rank, "i32", cfg, "owner_rank"), int(n_ep), hp, hb,
                                wsp, wsb, _stream(stream))
    _check("moe_combine_ledger", st)


def moe_ledger_finalize(cfg: MoeCfg, capacity: int, n_ep: int, alpha: float,
                        host_stage: torch.Tensor, raise_on_error: bool = True) -> dict:
    """Decode a completed stage into the ledger dict (pure host call)."""
    lib = load_library()
    hp, _ = _host_ptr(host_stage, "host_stage")
    E = int(cfg.E)
    out = MoeLedger()
    loads = (_I64 * E)()
    f = (_F64 * E)()
    P = (_F64 * E)()
    pair = (_I64 * (n_ep * n_ep))()
    out.status = -1  # finalize fills `out` (status included) only for a decoded stage
    st = lib.moe_ledger_finalize(ctypes.byref(cfg), int(capacity), int(n_ep), float(alpha), hp,
                                 ctypes.byref(out), loads, f, P, pair)
    if st != 0 and (raise_on_error or st not in (2, 1) or out.status != st):
        raise MoeError("moe_ledger_finalize", st)
    d = out.as_dict()
    d["loads"] = list(loads)
    d["f"] = list(f)
    d["P"] = list(P)
    d["pair_routes"] = [list(pair[i * n_ep:(i + 1) * n_ep]) for i in range(n_ep)]
    d["return_status"] = st
    return d


PLAN_NAMES = ("accept", "tune", "reject")


def moe_recommend_plan(ledger: dict, thresholds=None, use_locality: bool = True) -> str:
    """Joint plan decision over a ledger dict (as moe_ledger returns):
    'accept' / 'tune' / 'reject'.  thresholds: None (the page's limits) or
    5 numbers (accept balance, accept cross share, tune overflow share, tune
    balance, tune cross share)."""
    lib = load_library()
    L = MoeLedger()
    for name, _ in MoeLedger._fields_:
        setattr(L, name, ledger[name])
    th = None if thresholds is None else (_F64 * 5)(*[float(v) for v in thresholds])
    r = lib.moe_recommend_plan(ctypes.byref(L), th, int(bool(use_locality)))
    if r < 0:
        raise MoeError("moe_recommend_plan", 1)
    return PLAN_NAMES[r]



def moe_expert_ffn_fp8(cfg: MoeCfg, capacity: int, x_disp_q, scale, expert_offsets, w1, b1,
                       w2, b2, h_buf, y, packed: bool = False, stream=None) -> None:
    """The expert FFN on the E4M3 dispatch payload (x_disp_q uint8 [R_max, h],
    scale fp32 [1] on the device); packed: w1/w2 in the packed layout."""
    lib = load_library()
    if not isinstance(x_disp_q, torch.Tensor) or x_disp_q.dtype != torch.uint8:
        raise ValueError("x_disp_q: expected a uint8 device tensor")
    if x_disp_q.device.type != "cuda" or not x_disp_q.is_contiguous():
        raise ValueError("x_disp_q: expected a contiguous device tensor")
    st = lib.moe_expert_ffn_fp8(ctypes.byref(cfg), int(capacity),
                                ctypes.c_void_p(x_disp_q.data_ptr()),
                                _ptr(scale, "f32", cfg, "scale"),
                                _ptr(expert_offsets, "i32", cfg, "expert_offsets"),
                                _ptr(w1, "act", cfg, "w1"), _ptr(b1, "f32", cfg, "b1"),
                                _ptr(w2, "act", cfg, "w2"), _ptr(b2, "f32", cfg, "b2"),
                                _ptr(h_buf, "act", cfg, "h_buf"), _ptr(y, "f32", cfg, "y"),
                                int(bool(packed)), _stream(stream))
    _check("moe_expert_ffn_fp8", st)


def moe_expert_rank_affinity(cfg: MoeCfg, topk_idx, route_row, src_rank, n_ep: int, affinity,
                             stream=None) -> None:
    """affinity [E, n_ep] int32 (device): routes to expert e from source rank r
    (accepted routes only when route_row is given)."""
    lib = load_library()
    st = lib.moe_expert_rank_affinity(ctypes.byref(cfg), _ptr(topk_idx, "i32", cfg, "topk_idx"),
                                      _ptr(route_row, "i32", cfg, "route_row"),
                                      _ptr(src_rank, "i32", cfg, "src_rank"), int(n_ep),
                                      _ptr(affinity, "i32", cfg, "affinity"), _stream(stream))
    _check("moe_expert_rank_affinity", st)


def moe_place_experts(affinity, n_ep: int):
    """Expert -> rank map (list of E ints) with E / n_ep experts per rank that
    maximises the local routes (pure host call on a host copy of `affinity`)."""
    lib = load_library()
    a = torch.as_tensor(affinity).to("cpu", torch.int32).contiguous()
    E = int(a.shape[0])
    owner = (ctypes.c_int32 * E)()
    st = lib.moe_place_experts(ctypes.c_void_p(a.data_ptr()), E, int(n_ep), owner)
    _check("moe_place_experts", st)
    return list(owner)

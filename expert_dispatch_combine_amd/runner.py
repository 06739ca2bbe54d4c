"""Device buffers for one MoE layer and the call sequence of the C ABI.

`LayerBuffers` allocates every output/scratch tensor the entry points need
(sizes from moe_max_rows / moe_workspace_bytes); `run_layer` issues
moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine on one stream.
`LayerPlan` marshals the same calls once for fixed tensors and a fixed stream,
so a serving loop (or a HIP-graph capture) pays only the bare C calls per
step.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import ctypes

import torch

from ._binding import (_F64, _I64, MOE_BF16, MoeCfg, MoeError, MoeLedger, _ptr, _ws,
                       load_library, moe_capacity,
                       moe_combine, moe_dispatch, moe_expert_ffn, moe_expert_ffn_packed,
                       moe_ledger, moe_ledger_finalize, moe_ledger_stage_bytes, moe_max_rows,
                       moe_pack_expert_weights, moe_route, moe_workspace_bytes)


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


def run_ffn(b: LayerBuffers, w1, b1, w2, b2, stream=None, packed=False):
    fn = moe_expert_ffn_packed if packed else moe_expert_ffn
    fn(b.cfg, b.capacity, b.x_disp, b.expert_offsets, w1, b1, w2, b2, b.h_buf, b.y, stream)


def pack_weights(cfg: MoeCfg, w1, w2, stream=None):
    """Packed copies of W1 and W2 (moe_pack_expert_weights)."""
    w1p, w2p = torch.empty_like(w1), torch.empty_like(w2)
    moe_pack_expert_weights(cfg, w1, w2, w1p, w2p, stream)
    return w1p, w2p


def run_combine(b: LayerBuffers, stream=None):
    moe_combine(b.cfg, b.y, b.route_row, b.topk_gate, b.out, stream)


def run_ledger(b: LayerBuffers, src_rank, owner_rank, n_ep, alpha=0.01, stream=None, **kw):
    return moe_ledger(b.cfg, b.topk_idx, b.topk_gate, b.route_row, b.capacity, src_rank,
                      owner_rank, n_ep, alpha, b.ws, stream, **kw)


def run_layer(b: LayerBuffers, x, w_gate, logit_bias, w1, b1, w2, b2, stream=None,
              packed=False):
    """route -> dispatch -> expert FFN -> combine (asynchronous on `stream`);
    `packed`: w1/w2 are in the packed fragment layout."""
    run_route(b, x, w_gate, logit_bias, expert_load=False, stream=stream)
    run_dispatch(b, x, expert_load=True, stream=stream)
    run_ffn(b, w1, b1, w2, b2, stream=stream, packed=packed)
    run_combine(b, stream=stream)


class LayerPlan:
    """The whole step -- route, dispatch, expert FFN, combine, and the ledger's
    device half with the copy of its counters to a page-locked host stage --
    marshalled once.  `launch()` enqueues it with bare C calls; the ledger
    runs on `side` (after the dispatch, beside the FFN) when given, joined back
    into `main` before launch() returns; with fused_tail it runs with the
    combine in one moe_combine_ledger call.  gather_in_ffn: moe_dispatch
    moves no row and moe_expert_ffn_rows reads x[row_token[r]] itself (b.x_disp
    is then left untouched).  After the work has completed,
    `ledger()` decodes the stage on the host.

    The plan does not own the tensors: they must outlive it and keep their
    storage (a HIP graph captured from launch() replays these addresses).
    logits_in: route from the logits already in `b.logits` (moe_route with
    x = NULL) instead of the router product."""

    def __init__(self, b: LayerBuffers, x, w_gate, logit_bias, w1, b1, w2, b2, src_rank,
                 owner_rank, n_ep: int, alpha: float = 0.01, main=None, side=None,
                 ledger_ws=None, packed: bool = False, logits_in: bool = False,
                 fused_tail: bool = False, gather_in_ffn: bool = False):
        lib = load_library()
        cfg = b.cfg
        self.b, self.cfg, self.n_ep, self.alpha = b, cfg, int(n_ep), float(alpha)
        self.main = main if main is not None else torch.cuda.current_stream()
        self.side = side
        if fused_tail and side is not None:
            raise ValueError("fused_tail runs the ledger with the combine on `main`: no side "
                             "stream")
        self.fused_tail = bool(fused_tail)
        self.stage = torch.empty((moe_ledger_stage_bytes(cfg, n_ep),), dtype=torch.uint8,
                                 pin_memory=True)
        self.ledger_ws = ledger_ws if ledger_ws is not None else (
            torch.empty_like(b.ws) if side is not None else b.ws)
        ms = ctypes.c_void_p(self.main.cuda_stream)
        ls = ctypes.c_void_p((side or self.main).cuda_stream)
        c = ctypes.byref(cfg)
        wsp, wsb = _ws(b.ws)
        lwsp, lwsb = _ws(self.ledger_ws)
        self._cfg_ref = cfg  # byref() keeps no reference of its own
        self._keep = (x, w_gate, logit_bias, w1, b1, w2, b2, src_rank, owner_rank)
        p = lambda t, k, n: _ptr(t, k, cfg, n)  # noqa: E731
        rx, rw = (None, None) if logits_in else (x, w_gate)  # logits_in: b.logits is the input
        self.route = (lib.moe_route, (c, p(rx, "act", "x"), p(rw, "act", "w_gate"),
                                      p(logit_bias, "f32", "logit_bias"),
                                      p(b.logits, "f32", "logits"),
                                      p(b.topk_idx, "i32", "topk_idx"),
                                      p(b.topk_gate, "f32", "topk_gate"), None, wsp, wsb, ms))
        xd = None if gather_in_ffn else p(b.x_disp, "act", "x_disp")
        self.dispatch = (lib.moe_dispatch, (c, p(x, "act", "x"), p(b.topk_idx, "i32", "topk_idx"),
                                            b.capacity, p(b.expert_offsets, "i32", "offsets"),
                                            p(b.route_rank, "i32", "route_rank"),
                                            p(b.route_row, "i32", "route_row"),
                                            p(b.row_token, "i32", "row_token"), xd,
                                            p(b.expert_load, "i32", "expert_load"), wsp, wsb, ms))
        wargs = (p(b.expert_offsets, "i32", "offsets"), p(w1, "act", "w1"), p(b1, "f32", "b1"),
                 p(w2, "act", "w2"), p(b2, "f32", "b2"), p(b.h_buf, "act", "h_buf"),
                 p(b.y, "f32", "y"))
        if gather_in_ffn:  # the FFN's loads gather x[row_token[r]]; no x_disp
            self.ffn = (lib.moe_expert_ffn_rows, (c, b.capacity, p(x, "act", "x"),
                                                  p(b.row_token, "i32", "row_token"), *wargs,
                                                  int(bool(packed)), ms))
        else:
            ffn_fn = lib.moe_expert_ffn_packed if packed else lib.moe_expert_ffn
            self.ffn = (ffn_fn, (c, b.capacity, p(b.x_disp, "act", "x_disp"), *wargs, ms))
        self.combine = (lib.moe_combine, (c, p(b.y, "f32", "y"), p(b.route_row, "i32", "route_row"),
                                          p(b.topk_gate, "f32", "topk_gate"),
                                          p(b.out, "f32", "out"), ms))
        self.ledger_launch = (lib.moe_ledger_launch, (
            c, p(b.topk_idx, "i32", "topk_idx"), p(b.topk_gate, "f32", "topk_gate"),
            p(b.route_row, "i32", "route_row"), p(src_rank, "i32", "src_rank"),
            p(owner_rank, "i32", "owner_rank"), self.n_ep,
            ctypes.c_void_p(self.stage.data_ptr()), self.stage.numel(), lwsp, lwsb, ls))
        self.combine_ledger = (lib.moe_combine_ledger, (
            c, p(b.y, "f32", "y"), p(b.route_row, "i32", "route_row"),
            p(b.topk_gate, "f32", "topk_gate"), p(b.out, "f32", "out"),
            p(b.topk_idx, "i32", "topk_idx"), p(src_rank, "i32", "src_rank"),
            p(owner_rank, "i32", "owner_rank"), self.n_ep,
            ctypes.c_void_p(self.stage.data_ptr()), self.stage.numel(), lwsp, lwsb, ms))
        # moe_ledger_finalize into buffers allocated once (decode() per step)
        E, ne = int(cfg.E), self.n_ep
        self._fin = (MoeLedger(), (_I64 * E)(), (_F64 * E)(), (_F64 * E)(), (_I64 * (ne * ne))())
        self.finalize = (lib.moe_ledger_finalize, (
            c, int(b.capacity), ne, self.alpha, ctypes.c_void_p(self.stage.data_ptr()),
            ctypes.byref(self._fin[0]), *self._fin[1:]))
        self.ev_dispatched = torch.cuda.Event()
        self.ev_ledger = torch.cuda.Event()

    @staticmethod
    def _call(name, fa):
        st = fa[0](*fa[1])
        if st != 0:
            raise MoeError(name, st)

    def launch(self, events=None):
        """Enqueue one step.  `events` (optional, 5 timing events) are recorded
        on the main stream before route / dispatch / FFN / combine and after."""
        m = self.main
        if events:
            events[0].record(m)
        self._call("moe_route", self.route)
        if events:
            events[1].record(m)
        self._call("moe_dispatch", self.dispatch)
        if events:
            events[2].record(m)
        if self.side is not None:
            self.ev_dispatched.record(m)
            self.side.wait_event(self.ev_dispatched)
            self._call("moe_ledger_launch", self.ledger_launch)
            self.ev_ledger.record(self.side)
        self._call("moe_expert_ffn", self.ffn)
        if events:
            events[3].record(m)
        if self.fused_tail:  # combine and ledger in one call (one launch when small)
            self._call("moe_combine_ledger", self.combine_ledger)
            if events:
                events[4].record(m)
            return
        self._call("moe_combine", self.combine)
        if events:
            events[4].record(m)
        if self.side is None:
            self._call("moe_ledger_launch", self.ledger_launch)
        else:
            m.wait_event(self.ev_ledger)

    def decode(self) -> int:
        """moe_ledger_finalize of the completed stage into the plan's own host
        buffers (no Python objects built); returns its status (0, or 1/2
        when the batch held invalid ranks / expert ids, with the ledger
        filled).  A stage holding no completed ledger, or an argument error,
        raises."""
        fn, args = self.finalize
        self._fin[0].status = -1  # written by finalize only for a decoded stage
        st = fn(*args)
        if st != 0 and (st not in (1, 2) or self._fin[0].status != st):
            raise MoeError("moe_ledger_finalize", st)
        return st

    def ledger(self, **kw) -> dict:
        """Decode the host stage (the step's work must have completed)."""
        return moe_ledger_finalize(self.cfg, self.b.capacity, self.n_ep, self.alpha, self.stage,
                                   **kw)

"""The C-ABI library on the CPU: it loads, exports every function include/moe.h
declares, and its pure-host functions and argument checks behave (no GPU call
is made here: every invalid argument is rejected before any HIP call)."""
import ctypes
import math
import os
import random
import re

import numpy as np
import pytest

import expert_dispatch_combine_amd as M
import oracle as O
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(moe_[a-z_0-9]+)\s*\(", src,
                                 flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.library_path()):
        pytest.fail("libmoe.so is not built: run `python -m expert_dispatch_combine_amd.build`")
    return M.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert set(names) == set(M.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert M.moe_status_string(0) == "MOE_OK"
    assert M.moe_status_string(2) == "MOE_ERR_EXPERT_ID"
    assert M.moe_status_string(99) == "MOE_ERR_UNKNOWN"


def test_capacity_matches_oracle_bit_for_bit(lib):
    rng = random.Random(0)
    cases = [(11, 2, 1.0), (0, 4, 1.25), (2048, 16, 1.25), (8192, 8, 1.25), (32768, 256, 1.0),
             (98304, 64, 1.0), (128, 4, 1.0), (7, 3, 1.1), (1, 1024, 0.01)]
    for _ in range(3000):
        cases.append((rng.randrange(0, 1 << 22), rng.randrange(1, 1025),
                      rng.choice([1.0, 1.25, 2.0, 0.5, rng.uniform(0.01, 4.0)])))
    for A, E, cf in cases:
        assert M.moe_capacity(A, E, cf) == O.capacity(A, E, cf), (A, E, cf)
    assert M.moe_capacity(4, 0, 1.0) == -1
    assert M.moe_capacity(4, 2, 0.0) == -1
    assert M.moe_capacity(4, 2, float("nan")) == -1
    assert M.moe_capacity(-1, 2, 1.0) == -1


def test_max_rows_and_workspace(lib):
    cfg = M.MoeCfg.make(4096, 7168, 256, 8, 2048, "bf16", 1.0)
    assert M.moe_max_rows(cfg, 128) == min(4096 * 8, 256 * 128)
    assert M.moe_max_rows(cfg, 1000) == 4096 * 8
    assert M.moe_max_rows(cfg, -1) == -1
    assert M.moe_workspace_bytes(cfg) > 0
    bad = M.MoeCfg.make(4, 64, 2, 3, 64, "bf16", 1.0)   # K > E
    assert M.moe_workspace_bytes(bad) == 0


def _call_route(lib, cfg):
    return lib.moe_route(ctypes.byref(cfg), None, None, None, None, None, None, None, None, 0,
                         None)


def test_invalid_arguments_are_rejected_on_the_host(lib):
    mk = M.MoeCfg.make
    assert _call_route(lib, mk(4, 64, 2, 3, 64, "bf16", 1.0)) == 1          # K > E
    assert _call_route(lib, mk(4, 64, 0, 1, 64, "bf16", 1.0)) == 1          # E = 0
    assert _call_route(lib, mk(4, 0, 2, 1, 64, "bf16", 1.0)) == 1           # h = 0
    assert _call_route(lib, mk(-1, 64, 2, 1, 64, "bf16", 1.0)) == 1         # T < 0
    assert _call_route(lib, mk(4, 64, 2, 1, 64, "bf16", 0.0)) == 1          # cf = 0
    assert _call_route(lib, mk(4, 64, 2, 1, 64, "bf16", float("inf"))) == 1
    assert _call_route(lib, M.MoeCfg(4, 64, 2, 1, 64, 7, 1.0)) == 1          # dtype
    assert _call_route(lib, mk(4, 64, 2000, 1, 64, "bf16", 1.0)) == 5       # E > 1024
    assert _call_route(lib, mk(4, 64, 64, 33, 64, "bf16", 1.0)) == 5        # K > 32
    assert _call_route(lib, mk(4, 96, 2, 1, 64, "bf16", 1.0)) == 5          # h % 64
    assert _call_route(lib, mk(4, 64, 2, 1, 64, "bf16", 1.0)) == 1          # NULL outputs
    cfg = mk(4, 64, 2, 1, 64, "bf16", 1.0)
    # dispatch: negative capacity, missing workspace
    assert lib.moe_dispatch(ctypes.byref(cfg), None, None, -1, None, None, None, None, None,
                            None, None, 0, None) == 1
    assert lib.moe_dispatch(ctypes.byref(cfg), None, None, 2, None, None, None, None, None,
                            None, None, 0, None) == 1
    # ffn: negative capacity, NULL operands
    assert lib.moe_expert_ffn(ctypes.byref(cfg), -1, None, None, None, None, None, None, None,
                              None, None) == 1
    assert lib.moe_expert_ffn(ctypes.byref(cfg), 2, None, None, None, None, None, None, None,
                              None, None) == 1
    # combine: NULL outputs
    assert lib.moe_combine(ctypes.byref(cfg), None, None, None, None, None) == 1
    # ledger: n_ep out of range, NULL out
    out = M.MoeLedger()
    assert lib.moe_ledger(ctypes.byref(cfg), None, None, None, 2, None, None, 65, 0.01,
                          ctypes.byref(out), None, None, None, None, None, 0, None) == 1
    assert lib.moe_ledger(ctypes.byref(cfg), None, None, None, 2, None, None, 2, 0.01,
                          None, None, None, None, None, None, 0, None) == 1
    # bias update: NULL bias, non-finite alpha
    assert lib.moe_bias_update(ctypes.byref(cfg), None, None, 0.1, None, None) == 1
    assert lib.moe_bias_update(ctypes.byref(cfg), None, ctypes.c_void_p(16),
                               float("nan"), None, None) == 1
    # FP8 payload: fp32 configurations are unsupported; NULL scale / workspace
    cfg32 = mk(4, 64, 2, 1, 64, "f32", 1.0)
    assert lib.moe_fp8_scale(ctypes.byref(cfg32), None, None, None, 0, None) == 5
    assert lib.moe_dispatch_fp8(ctypes.byref(cfg32), None, None, None, 2, None, None, None,
                                None, None, None, None, 0, None) == 5
    assert lib.moe_fp8_dequantize(ctypes.byref(cfg32), 2, None, None, None, None, None) == 5
    assert lib.moe_fp8_scale(ctypes.byref(cfg), None, None, None, 0, None) == 1
    assert lib.moe_dispatch_fp8(ctypes.byref(cfg), None, None, None, 2, None, None, None,
                                None, None, None, None, 0, None) == 1
    assert lib.moe_fp8_dequantize(ctypes.byref(cfg), 2, None, None, None, None, None) == 1
    # ffn on gathered rows: NULL cfg, NULL row_token, packed fp32 weights
    assert lib.moe_expert_ffn_rows(None, 2, None, None, None, None, None, None, None, None,
                                   None, 0, None) == 1
    assert lib.moe_expert_ffn_rows(ctypes.byref(cfg), 2, None, None, None, None, None, None,
                                   None, None, None, 0, None) == 1
    assert lib.moe_expert_ffn_rows(ctypes.byref(cfg32), 2, None, ctypes.c_void_p(16), None,
                                   None, None, None, None, None, None, 1, None) == 5
    # combine + ledger: NULL workspace, n_ep out of range, stage too small
    fake = ctypes.c_void_p(256)
    assert lib.moe_combine_ledger(ctypes.byref(cfg), None, None, None, None, None, None, fake,
                                  2, fake, 1 << 20, None, 0, None) == 1
    ws_b = lib.moe_workspace_bytes(ctypes.byref(cfg))
    assert lib.moe_combine_ledger(ctypes.byref(cfg), None, fake, fake, fake, fake, fake, fake,
                                  65, fake, 1 << 20, fake, ws_b, None) == 1
    assert lib.moe_combine_ledger(ctypes.byref(cfg), None, fake, fake, fake, fake, fake, fake,
                                  2, fake, 8, fake, ws_b, None) == 3


def test_empty_batch_needs_no_device_work(lib):
    cfg = M.MoeCfg.make(0, 64, 4, 2, 64, "bf16", 1.0)
    # T = 0 with no expert_load requested: nothing is enqueued
    assert lib.moe_route(ctypes.byref(cfg), None, None, None, None, None, None, None, None, 0,
                         None) == 0
    assert lib.moe_expert_ffn(ctypes.byref(cfg), 0, None, None, None, None, None, None, None,
                              None, None) == 0
    assert lib.moe_combine(ctypes.byref(cfg), None, None, None, None, None) == 0


def test_ledger_struct_layout_matches_header(lib):
    # 20 int64 + 8 double + 2 int32
    assert ctypes.sizeof(M.MoeLedger) == 20 * 8 + 8 * 8 + 2 * 4
    assert ctypes.sizeof(M.MoeCfg) == 6 * 4 + 8


def test_recommend_plan_matches_the_oracle(lib):
    """The library's decision equals the oracle's on the page's contract cases
    and on random ledgers around every limit (pure host function)."""
    import json
    import random
    import oracle as O
    from conftest import GOLDEN
    g = json.load(open(os.path.join(GOLDEN, "ep46_decision_cases.json")))
    for case in g["cases"]:
        s = O.summarize_routes(case["routes"], case["num_experts"], case["hidden_size"])
        led = {name: 0 for name, _ in M.MoeLedger._fields_}
        led.update(total_routes=s["total_routes"], overflow=s["overflow"],
                   balance_ratio=s["balance_ratio"])
        loc = case["locality"]
        if loc is not None:
            led.update(local_routes=loc["local_routes"], cross_rank_routes=loc["cross_rank_routes"])
        assert M.moe_recommend_plan(led, use_locality=loc is not None) == case["expect"]
    rng = random.Random(9)
    for _ in range(3000):
        A = rng.choice([0, 1, 7, 100, 1000])
        ovf = rng.randint(0, A)
        bal = rng.choice([1.0, 1.2, 1.2000001, 1.2004, 1.2005, 1.2006, 1.5, 1.8, 1.8000001,
                          1.8004, 1.8005, 1.8006, 2.5,
                          # the exact ratio of integer loads, max * E / A
                          rng.randint(1, 20000) * 2 / 20000, rng.randint(6000, 6010) / 5000,
                          rng.randint(9000, 9010) / 5000])
        cross = rng.randint(0, A)
        led = {name: 0 for name, _ in M.MoeLedger._fields_}
        led.update(total_routes=A, overflow=ovf, balance_ratio=bal, local_routes=A - cross,
                   cross_rank_routes=cross)
        want = O.recommend_plan({"total_routes": A, "overflow": ovf, "balance_ratio": bal},
                                {"total_routes": A, "local_routes": A - cross,
                                 "cross_rank_routes": cross})
        assert M.moe_recommend_plan(led) == want
    th = [1.0, 0.1, 0.5, 3.0, 1.0]
    led = {name: 0 for name, _ in M.MoeLedger._fields_}
    led.update(total_routes=10, overflow=0, balance_ratio=1.1, local_routes=9,
               cross_rank_routes=1)
    assert M.moe_recommend_plan(led, th) == O.recommend_plan(
        {"total_routes": 10, "overflow": 0, "balance_ratio": 1.1},
        {"total_routes": 10, "local_routes": 9, "cross_rank_routes": 1},
        max_accept_balance=1.0, max_accept_cross_rank=0.1, max_tune_overflow_ratio=0.5,
        max_tune_balance=3.0, max_tune_cross_rank=1.0)


def test_finalize_rejects_a_stage_without_a_ledger(lib):
    """A zeroed (never written, or torn) stage holds no part count: finalize
    returns MOE_ERR_SHAPE and leaves every output unwritten."""
    cfg = M.MoeCfg.make(16, 64, 4, 2, 64, "bf16", 1.0)
    n_ep = 2
    nbytes = lib.moe_ledger_stage_bytes(ctypes.byref(cfg), n_ep)
    assert nbytes > 8
    stage = (ctypes.c_uint8 * nbytes)()
    out = M.MoeLedger()
    out.status = -7
    out.total_routes = -7
    loads = (ctypes.c_int64 * 4)(-1, -1, -1, -1)
    st = lib.moe_ledger_finalize(ctypes.byref(cfg), 8, n_ep, 0.01, stage, ctypes.byref(out),
                                 loads, None, None, None)
    assert st == 3  # MOE_ERR_SHAPE
    assert out.status == -7 and out.total_routes == -7 and list(loads) == [-1] * 4
    # a part count beyond the stage's capacity is refused the same way
    ctypes.c_int64.from_buffer(stage).value = 5
    assert lib.moe_ledger_finalize(ctypes.byref(cfg), 8, n_ep, 0.01, stage, ctypes.byref(out),
                                   loads, None, None, None) == 3
    # one part of all-zero counters is a valid (empty) ledger
    ctypes.c_int64.from_buffer(stage).value = 1
    assert lib.moe_ledger_finalize(ctypes.byref(cfg), 8, n_ep, 0.01, stage, ctypes.byref(out),
                                   loads, None, None, None) == 0
    assert out.status == 0 and out.total_routes == 32 and list(loads) == [0] * 4
    # the Python decoder raises on a zeroed stage instead of returning zeros
    import torch
    with pytest.raises(M.MoeError):
        M.moe_ledger_finalize(cfg, 8, n_ep, 0.01, torch.zeros(nbytes, dtype=torch.uint8))


def test_noalloc_dispatch_checks_on_the_host(lib):
    """moe_dispatch_noalloc rejects, before any HIP call, arguments that are
    invalid and sizes whose counting scratch (ceil(T*K/1024) * (E+1) int32,
    rounded up to 256 bytes) exceeds its 4 MiB static array."""
    fake = ctypes.c_void_p(256)
    assert lib.moe_dispatch_noalloc(None, fake, fake, 8, fake, fake, fake, fake, None, None,
                                    None) == 1
    cfg = M.MoeCfg.make(2048, 64, 1024, 1, 64, "bf16", 1.0)
    assert lib.moe_dispatch_noalloc(ctypes.byref(cfg), fake, fake, -1, fake, fake, fake, fake,
                                    None, None, None) == 1
    assert lib.moe_dispatch_noalloc(ctypes.byref(cfg), fake, fake, 8, None, fake, fake, fake,
                                    None, None, None) == 1
    # one route more than the largest batch that fits, at E = 1024 and E = 64
    for E, A_fit in ((1024, 1_047_552), (64, 16_518_144)):
        cfg = M.MoeCfg.make(A_fit + 1, 64, E, 1, 64, "bf16", 1.0)
        assert lib.moe_dispatch_noalloc(ctypes.byref(cfg), fake, fake, 8, fake, fake, fake, fake,
                                        None, None, None) == 5, E


def test_place_experts_reaches_the_oracle_optimum(lib):
    """moe_place_experts (host Hungarian method) against the oracle's
    locality placement: the same number of local routes (the optimum is
    unique, the map need not be), E / n_ep experts per rank, on random and
    structured affinity matrices up to 256 experts."""
    rng = np.random.default_rng(61)
    cases = [(2, 2), (4, 2), (8, 4), (16, 16), (64, 8), (256, 8), (12, 3), (5, 1)]
    for E, n in cases:
        for kind in ("random", "tied", "local", "skewed"):
            if kind == "random":
                aff = rng.integers(0, 1000, (E, n))
            elif kind == "tied":
                aff = np.full((E, n), 7)
            elif kind == "local":   # expert e gets its routes from rank perm(e) // (E/n)
                perm = rng.permutation(E)
                aff = rng.integers(0, 3, (E, n))
                aff[np.arange(E), perm // (E // n)] += 500
            else:                   # every rank prefers rank 0's experts
                aff = rng.integers(0, 50, (E, n))
                aff[:, 0] += rng.integers(0, 5000, E)
            owner = M.moe_place_experts(aff.astype(np.int32), n)
            assert sorted(np.bincount(owner, minlength=n).tolist()) == [E // n] * n
            want = O.locality_placement(aff, n)
            assert O.local_routes_under(aff, owner) == O.local_routes_under(aff, want), (E, n, kind)


def test_place_experts_argument_checks(lib):
    aff = np.zeros((6, 4), np.int32)
    owner = (ctypes.c_int32 * 6)()
    assert lib.moe_place_experts(ctypes.c_void_p(aff.ctypes.data), 6, 4, owner) == 1  # 6 % 4
    assert lib.moe_place_experts(None, 6, 3, owner) == 1
    aff[2, 1] = -1
    assert lib.moe_place_experts(ctypes.c_void_p(aff.ctypes.data), 6, 3, owner) == 1
    assert lib.moe_expert_rank_affinity(None, None, None, None, 2, None, None) == 1
    cfg = M.MoeCfg.make(4, 64, 4, 2, 64, "bf16", 1.0)
    assert lib.moe_expert_rank_affinity(ctypes.byref(cfg), None, None, None, 2, None, None) == 1
    assert lib.moe_expert_rank_affinity(ctypes.byref(cfg), None, None, None, 65,
                                        ctypes.c_void_p(256), None) == 1


def test_fp8_ffn_checks_on_the_host(lib):
    """moe_expert_ffn_fp8: bf16 only, and unsupported where the first GEMM
    would take the tiled shape (rows per expert >= 384, F not a multiple of
    128, row-major weights or fewer than 512 rows per expert); both refused
    before any HIP call."""
    fake = ctypes.c_void_p(256)
    cfg32 = M.MoeCfg.make(64, 64, 4, 2, 64, "f32", 1.0)
    assert lib.moe_expert_ffn_fp8(ctypes.byref(cfg32), 32, fake, fake, fake, fake, fake, fake,
                                  fake, fake, fake, 0, None) == 5
    cfg = M.MoeCfg.make(4096, 256, 4, 1, 192, "bf16", 1.0)   # 1024 rows per expert, F = 192
    assert lib.moe_expert_ffn_fp8(ctypes.byref(cfg), 1024, fake, fake, fake, fake, fake, fake,
                                  fake, fake, fake, 0, None) == 5
    cfg = M.MoeCfg.make(1800, 256, 4, 1, 192, "bf16", 1.3)   # 450 rows per expert, packed
    assert lib.moe_expert_ffn_fp8(ctypes.byref(cfg), 585, fake, fake, fake, fake, fake, fake,
                                  fake, fake, fake, 1, None) == 5
    cfg = M.MoeCfg.make(64, 64, 4, 2, 64, "bf16", 1.0)
    assert lib.moe_expert_ffn_fp8(ctypes.byref(cfg), 32, None, fake, fake, fake, fake, fake,
                                  fake, fake, fake, 0, None) == 1

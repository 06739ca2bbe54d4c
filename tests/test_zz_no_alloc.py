"""moe_dispatch_noalloc (the dispatch for callers that cannot allocate: its
scratch is a static device array, not a caller workspace) against
moe_dispatch, called through the C ABI.

Two calls in a row on one stream, the second with a smaller batch (fewer
routes, and more experts, so the second call's counts overlap what the first
left in the array), each compared bit for bit with moe_dispatch on the same
inputs: expert offsets, ranks, rows, row_token, the dispatched rows and the
loads.  Both batches exceed the one-launch dispatch (8192 routes), so the
counting kernels use the scratch; the last case is below it (no scratch).
Sizes whose scratch exceeds the array are refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import expert_dispatch_combine_amd as M
import moe_workloads as W
from gpu_util import banner

pytestmark = pytest.mark.gpu


def _routing(T, E, K, seed, zipf=None):
    rng = np.random.default_rng(seed)
    if zipf is None:
        return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    p = 1.0 / (np.arange(E) + 1.0) ** zipf
    p /= p.sum()
    return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _outputs(T, h, E, K, cap, dtype):
    i32 = dict(dtype=torch.int32, device="cuda")
    rmax = min(T * K, E * cap)
    return {"off": torch.full((E + 1,), -9, **i32), "rank": torch.full((T, K), -9, **i32),
            "row": torch.full((T, K), -9, **i32), "tok": torch.full((max(rmax, 1),), -9, **i32),
            "xd": torch.full((max(rmax, 1), h), 7, dtype=dtype, device="cuda"),
            "load": torch.full((E,), -9, **i32)}


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _call_both(lib, T, h, E, K, cf, seed, zipf=None):
    cfg = M.MoeCfg.make(T, h, E, K, 64, "bf16", cf)
    cap = M.moe_capacity(T * K, E, cf)
    idx = torch.from_numpy(_routing(T, E, K, seed, zipf)).cuda()
    x = torch.randn(T, h, device="cuda").to(torch.bfloat16)
    ref = _outputs(T, h, E, K, cap, torch.bfloat16)
    got = _outputs(T, h, E, K, cap, torch.bfloat16)
    ws = torch.empty(M.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.moe_dispatch(ctypes.byref(cfg), _p(x), _p(idx), cap, _p(ref["off"]),
                          _p(ref["rank"]), _p(ref["row"]), _p(ref["tok"]), _p(ref["xd"]),
                          _p(ref["load"]), _p(ws), ws.numel(), stream)
    assert st == 0
    st = lib.moe_dispatch_noalloc(ctypes.byref(cfg), _p(x), _p(idx), cap, _p(got["off"]),
                                  _p(got["rank"]), _p(got["row"]), _p(got["tok"]),
                                  _p(got["xd"]), _p(got["load"]), stream)
    assert st == 0
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k], got[k]), k
    return int(ref["off"][-1])


def test_noalloc_dispatch_equals_dispatch_twice_in_a_row():
    lib = M.load_library()
    banner("noalloc dispatch: 98304 routes, E 64 (hot experts)")
    R1 = _call_both(lib, 16384, 256, 64, 6, 1.0, seed=1, zipf=1.2)
    banner("noalloc dispatch: 12000 routes, E 256, second call")
    R2 = _call_both(lib, 1500, 128, 256, 8, 1.0, seed=2)
    assert R1 > 0 and R2 > 0
    banner("noalloc dispatch: 3000 routes (one-launch path, no scratch)")
    _call_both(lib, 1000, 64, 16, 3, 1.25, seed=3)


def test_noalloc_dispatch_refuses_sizes_beyond_its_scratch():
    lib = M.load_library()
    banner("noalloc dispatch: oversize refused")
    # ceil(A / 1024) * (E + 1) * 4 bytes > 4 MiB: refused before any launch
    cfg = M.MoeCfg.make(2_000_000, 64, 1024, 1, 64, "bf16", 1.0)
    fake = ctypes.c_void_p(256)
    assert lib.moe_dispatch_noalloc(ctypes.byref(cfg), fake, fake, 8, fake, fake, fake, fake,
                                    None, None, None) == 5

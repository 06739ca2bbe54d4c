"""bench.py pieces that run without a GPU: the one-GPU guard, the algorithmic
byte and flop counts behind `roofline.achieved`, and the reader of the
committed counter summary behind `roofline.traffic`."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

import moe_workloads as W


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line on refusal


def test_algorithmic_bytes_and_flops_of_the_switch_base_layer():
    # expert FFN: weights of the 16 non-empty experts (2 h F b each), x_disp
    # read (R h b), H written and read (2 R F b), Y written in fp32 (4 R h);
    # flops 4 h F R.  R = 2048 accepted rows (no overflow at cf 1.25).
    b = _bench()
    wl = W.CONFIGS[2]
    a = b.algorithmic(wl, R=2048, E_nz=16)
    h, F, R = 768, 3072, 2048
    assert a["ffn_bytes"] == 16 * 2 * h * F * 2 + R * h * 2 + 2 * R * F * 2 + R * h * 4
    assert a["ffn_bytes"] == 185_597_952
    assert a["ffn_flops"] == 4 * h * F * R == 19_327_352_832
    # the arithmetic intensity that puts this FFN under the HBM roof
    assert a["ffn_flops"] / a["ffn_bytes"] < 2500e12 / 8000e9
    # combine: Y rows in fp32, out rows in fp32, route rows and gates
    assert a["combine_bytes"] == R * h * 4 + 2048 * h * 4 + 2048 * 1 * 8


def test_committed_traffic_applies_only_to_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_text("kernel source v1\n")
    import hashlib
    rec = {"kernel": "expert_ffn", "workload": "w", "sources": ["k.hip"],
           "sources_sha256": hashlib.sha256(b"kernel source v1\n").hexdigest(),
           "bytes_per_call": 1234}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "x.md").write_text("# summary\n\ntraffic-json: " + json.dumps(rec) + "\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.committed_traffic("expert_ffn", "w") == 1234
    assert b.committed_traffic("expert_ffn", "other workload") is None
    assert b.committed_traffic("combine", "w") is None
    src.write_text("kernel source v2\n")  # the kernel changed since the counters
    assert b.committed_traffic("expert_ffn", "w") is None


def test_the_committed_headline_summary_parses():
    # the real profiles/ entry for the headline FFN (the DeepSeek-V3-shaped
    # workload): well formed, and its bytes within 2% of the algorithmic bytes
    # it is compared against (R = 31456 accepted rows, all 256 experts)
    b = _bench()
    path = os.path.join(ROOT, "profiles", "kernels_deepseek_v3_4096tok.md")
    lines = [l for l in open(path, encoding="utf-8") if l.startswith("traffic-json: ")]
    assert len(lines) == 1
    rec = json.loads(lines[0][len("traffic-json: "):])
    assert rec["kernel"] == "expert_ffn" and rec["workload"] == W.CONFIGS[4].name
    assert all(os.path.exists(os.path.join(ROOT, s)) for s in rec["sources"])
    alg = b.algorithmic(W.CONFIGS[4], R=31456, E_nz=256)["ffn_bytes"]
    assert alg == 16_642_932_736
    assert abs(rec["bytes_per_call"] / alg - 1) < 0.02


def test_default_workload_is_the_largest_single_gpu_one():
    b = _bench()
    import sys as _sys
    argv = _sys.argv
    try:
        _sys.argv = ["bench.py"]
        args = b.parse()
    finally:
        _sys.argv = argv
    wl = W.CONFIGS[args.config]
    weights = lambda c: c.E * 2 * c.h * c.F  # noqa: E731
    assert weights(wl) == max(weights(c) for c in W.CONFIGS.values())

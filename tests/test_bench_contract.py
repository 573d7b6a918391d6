"""CPU checks of bench.py's command-line contract and of the pieces of its JSON line that do not
need a GPU: more than one GPU is refused with a message, the measured-traffic lookup follows the
kernel code (comments aside), and the algorithmic byte counts match their definitions."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_quant_bytes_definition():
    # read the input once, write one code per element and one scale per group
    assert bench.quant_bytes(4096, 7168, 128, 2, 1, False) == 4096 * (2 * 7168 + 7168 + 56)
    assert bench.quant_bytes(8192, 2048, 128, 2, 4, True) == 8192 * (2 * 4096 + 2048 + 16 * 4)
    assert bench.quant_bytes(4096, 7168, 7168, 2, 4, False) == 4096 * (3 * 7168 + 4)


def test_traffic_tag_ignores_comments_only(tmp_path, monkeypatch):
    csrc = tmp_path / "fp8_group_quant_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "fp8q_internal.h").write_text("struct P { int a; };\n")
    (csrc / "k.hip").write_text("int f() { return 1; }  // one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    t0 = bench._kernel_source_tag("k.hip")
    (csrc / "k.hip").write_text("// header comment\n\nint f() { return 1; }  // changed comment\n")
    assert bench._kernel_source_tag("k.hip") == t0
    (csrc / "k.hip").write_text("int f() { return 2; }\n")
    assert bench._kernel_source_tag("k.hip") != t0
    (csrc / "k.hip").write_text("int f() { return 1; }\n")
    (csrc / "fp8q_internal.h").write_text("struct P { int a; int b; };\n")
    assert bench._kernel_source_tag("k.hip") != t0


def test_committed_traffic_matches_the_current_kernels():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    for src in ("quant.hip", "gemm.hip"):
        ent = rec["dense_m4096"][src]
        assert abs(ent["bytes_per_launch"] - (ent["fetch_bytes"] + ent["write_bytes"])) <= 1
    # reported only while the code is the one the counters were taken on
    for src in ("quant.hip", "gemm.hip"):
        tag = bench._kernel_source_tag(src)
        assert (bench._measured_traffic(src, "dense_m4096") is not None) == (tag == rec["dense_m4096"][src]["source_sha256_16"])

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
    # headers included from csrc/ count too, transitively
    (csrc / "fp8q_internal.h").write_text('#include "more.h"\nstruct P { int a; };\n')
    (csrc / "more.h").write_text("int g();\n")
    t1 = bench._kernel_source_tag("k.hip")
    (csrc / "more.h").write_text("int g(int);\n")
    assert bench._kernel_source_tag("k.hip") != t1


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


def _counter_db(path, rows):
    import sqlite3
    path.parent.mkdir(parents=True, exist_ok=True)
    con = sqlite3.connect(str(path))
    con.execute("create table counters_collection (kernel_name text, dispatch_id int, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_record_traffic_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    """Counters of a run are scaled so that the reference copy reads 2n and writes n bytes;
    a call's kernels (split GEMM + reduction) are summed; values of one dispatch's hardware
    instances are summed first."""
    n = bench.CALIBRATION_ELEMS
    fetch, write = [], []
    d = 0
    for _ in range(4):  # copy: FETCH reads half the truth (scale 2), WRITE exact
        d += 1
        fetch += [("copy_hi_bytes(...)", d, "FETCH_SIZE", n / 1024)]
        write += [("copy_hi_bytes(...)", d, "WRITE_SIZE", n / 2048), ("copy_hi_bytes(...)", d, "WRITE_SIZE", n / 2048)]
    for _ in range(3):
        d += 1
        fetch += [("group_quant_rows4_kernel<0, 128, false>", d, "FETCH_SIZE", 100.0)]
        write += [("group_quant_rows4_kernel<0, 128, false>", d, "WRITE_SIZE", 50.0)]
        d += 1
        fetch += [("gemm_splitk_kernel<8, 1, 0>", d, "FETCH_SIZE", 1000.0)]
        write += [("gemm_splitk_kernel<8, 1, 0>", d, "WRITE_SIZE", 400.0)]
        d += 1
        fetch += [("splitk_reduce_kernel(...)", d, "FETCH_SIZE", 300.0)]
        write += [("splitk_reduce_kernel(...)", d, "WRITE_SIZE", 30.0)]
    _counter_db(tmp_path / "f" / "host" / "run_results.db", fetch)
    _counter_db(tmp_path / "w" / "host" / "run_results.db", write)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    ent = bench.record_traffic("dense_m128", str(tmp_path / "f"), str(tmp_path / "w"))
    assert ent["fetch_scale"] == 2.0 and ent["write_scale"] == 1.0
    q, g = ent["quant.hip"], ent["gemm.hip"]
    assert q["fetch_bytes"] == 100 * 1024 * 2 and q["write_bytes"] == 50 * 1024
    assert g["fetch_bytes"] == 1300 * 1024 * 2 and g["write_bytes"] == 430 * 1024
    assert g["bytes_per_launch"] == g["fetch_bytes"] + g["write_bytes"] and g["launches"] == 3
    assert g["source_sha256_16"] == bench._kernel_source_tag("gemm.hip")
    with open(tmp_path / "traffic.json") as f:
        assert json.load(f)["dense_m128"]["gemm.hip"]["bytes_per_launch"] == g["bytes_per_launch"]

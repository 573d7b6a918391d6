"""Benchmark of the FP8 group-quant -> block-scaled FP8 GEMM path on one MI355X.

One step = the whole hot path over one batch of synthetic input resident in HBM:
per-token-group quantization of bf16 activations (UE8M0 column-major scales) followed by
the 1x128 x 128x128 block-scaled FP8 GEMM against e4m3 weights, bf16 output. The default
workload is the dense DeepSeek-V3-like projection at M = 4096 (X [4096, 7168], W [4096,
7168]); --workload picks another named shape for the step line.

Timing: W untimed warm-up steps, then exactly K steps between two synchronizations,
measured with HIP events on the stream the kernels run on. The per-kernel roofline figures
come from two more event-timed loops of K launches of each kernel alone. To defeat the 256 MB
Infinity Cache and the L2s, the steps rotate over enough independent input/output buffer
sets that the working set exceeds 1 GB.

Besides the step line's headline figures, the same JSON line carries:
  configs      every named workload (tiny; dense M = 1, 16, 128, 4096; the fused silu
               down-projection; the masked MoE; MXFP8 8192^3): each kernel's duration,
               rate and fraction of the roofline that binds it, timed as a captured HIP graph
               of back-to-back launches (so microsecond kernels are not timed against the
               host's launch rate) over >= 1 GB of rotating buffers where memory allows
  ceilings     reference kernels moving the same bytes with no arithmetic: a bf16 -> byte
               copy of the quant's traffic, and a read of the small-M GEMM's weights
  parity       a gate in the same run: the dense M = 4096 quant output compared byte for
               byte with the CPU oracle, and sampled GEMM outputs (>= 4096 and one whole
               256 x 256 tile) checked with the parity tests' tolerance rule
  cpu_baseline the plain CPU oracle timed on the host's cores (all of them, and one),
               on bounded samples of the same workload, scaled to the metric's unit
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-FP8 GEMM TFLOP/s & % MFMA peak; group-quant GB/s & % HBM peak"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
BENCH_LIB = os.path.join(ROOT, "fp8_group_quant_amd", "libfp8q_bench.so")


def _kernel_source_tag(name: str) -> str:
    """Hash of a kernel source, the shared internal header and every header of csrc/ that
    they include (transitively), with // comments and blank lines removed: a comment edit
    keeps the tag, any code change breaks it."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "fp8_group_quant_amd", "csrc")
    h = hashlib.sha256()
    todo, seen = [name, "fp8q_internal.h"], set()
    while todo:
        fn = todo.pop(0)
        if fn in seen or not os.path.exists(os.path.join(csrc, fn)):
            continue
        seen.add(fn)
        with open(os.path.join(csrc, fn), encoding="utf-8") as f:
            for line in f:
                line = re.sub(r"//.*$", "", line).rstrip()
                if line.strip():
                    h.update(line.encode() + b"\n")
                m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
                if m:
                    todo.append(m.group(1))
    return h.hexdigest()[:16]


def _measured_traffic(kernel_file: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on the
    current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        ent = rec[workload][kernel_file]
        if ent["source_sha256_16"] != _kernel_source_tag(kernel_file):
            return None
        return ent["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def _counter_dispatches(run_dir: str, counter: str) -> list:
    """[(dispatch_id, kernel_name, value)] of one counter from the rocpd databases under
    run_dir (a rocprofv3 --pmc run), values summed over the counter's hardware instances,
    in dispatch order."""
    import glob
    import sqlite3
    vals, names = {}, {}
    dbs = sorted(glob.glob(os.path.join(run_dir, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocpd database under {run_dir}")
    for i, db in enumerate(dbs):
        con = sqlite3.connect(db)
        for name, did, cn, v in con.execute(
                "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
            if cn == counter:
                vals[(i, did)] = vals.get((i, did), 0.0) + (v or 0.0)
                names[(i, did)] = name
        con.close()
    return [(k, names[k], vals[k]) for k in sorted(vals)]


CALIBRATION_ELEMS = 1 << 24  # bf16 values the calibration copies move (32 MiB in, 16 MiB out)

# kernels of each source file, by name
_KERNEL_FILES = {"quant.hip": ("group_quant_", "token_quant_"),
                 "gemm.hip": ("gemm_", "splitk_reduce_kernel")}


def record_traffic(workload: str, fetch_dir: str, write_dir: str) -> dict:
    """HBM bytes per quant and per GEMM call of `workload` from two rocprofv3 runs of this
    script's step loop (the first with --pmc FETCH_SIZE, the second with --pmc WRITE_SIZE;
    both KiB per dispatch). Each counter is scaled by what it reads for the reference copy
    kernel (copy_hi_bytes, run --calibration-copies times on CALIBRATION_ELEMS bf16 values:
    exactly 2n bytes read and n written); the result is merged into profiles/traffic.json
    with the source tag of each kernel file."""
    import numpy as np
    n = CALIBRATION_ELEMS
    truth = {"FETCH_SIZE": 2 * n, "WRITE_SIZE": n}
    runs = {"FETCH_SIZE": _counter_dispatches(fetch_dir, "FETCH_SIZE"),
            "WRITE_SIZE": _counter_dispatches(write_dir, "WRITE_SIZE")}
    scale, per_file = {}, {}
    for cn, disp in runs.items():
        copies = [v for _, name, v in disp if "copy_hi_bytes" in name and v > 0]
        if not copies:
            raise SystemExit(f"{cn}: no calibration copies (run the step loop with --calibration-copies)")
        scale[cn] = truth[cn] / (float(np.median(copies)) * 1024.0)
        for fname, pats in _KERNEL_FILES.items():
            ks = [(n, v) for _, n, v in disp if any(p in n for p in pats)]
            if ks:
                per_file.setdefault(fname, {})[cn] = ks
    out = {}
    for fname, d in per_file.items():
        if "FETCH_SIZE" not in d or "WRITE_SIZE" not in d:
            continue
        ent = {"source_sha256_16": _kernel_source_tag(fname)}
        total = 0.0
        kinds = sorted({n for n, _ in d["FETCH_SIZE"]})
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            kib = sum(float(np.median([v for n, v in d[cn] if n == k])) for k in kinds)
            ent[cn.split("_")[0].lower() + "_kib"] = round(kib, 1)
            ent[cn.split("_")[0].lower() + "_bytes"] = int(kib * 1024 * scale[cn])
            total += kib * 1024 * scale[cn]
        ent["kernels"] = [k[:120] for k in kinds]
        ent["bytes_per_launch"] = int(total)
        ent["launches"] = min(sum(1 for n, _ in d["FETCH_SIZE"] if n == k) for k in kinds)
        out[fname] = ent
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec["_note"] = ("HBM bytes per call from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed "
                    "over a call's kernels), each scaled by what it reads for a reference copy of known size "
                    "(bench.py --calibration-copies); fetch_scale and write_scale are per workload")
    rec[workload] = dict(out, fetch_scale=round(scale["FETCH_SIZE"], 4), write_scale=round(scale["WRITE_SIZE"], 4))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec[workload]


def quant_bytes(rows: int, K: int, G: int, in_bytes: int, scale_bytes: int, silu: bool) -> int:
    """Algorithmic bytes of one group-quant launch: read the input once, write codes + scales."""
    width = 2 * K if silu else K
    return rows * (width * in_bytes + K + (K // G) * scale_bytes)


def gemm_bytes(M: int, N: int, K: int, sa_bytes: int, sb_bytes: int) -> int:
    """Algorithmic bytes of one block-scaled GEMM: A, B and their scales once, Y (bf16) once."""
    return M * K + N * K + M * (K // 128) * sa_bytes + (-(-N // 128)) * (K // 128) * sb_bytes + M * N * 2


def build_workload(name: str):
    import synth
    if name.startswith("dense"):
        M = int(name.split("_m")[1]) if "_m" in name else 4096
        return synth.dense(M)
    if name == "silu_down":
        return synth.SILU
    if name == "tiny":
        return synth.TINY
    raise SystemExit(f"unknown workload {name!r}")


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def graph_time_ms(fn, n: int) -> float:
    """Average ms per launch of fn(0..n-1) captured into one HIP graph and replayed (after an
    untimed replay): the launches run back to back on the GPU."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(n, 3)):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    del g
    return ms


# buffer sets the masked quants rotate over: their per-launch bytes (82-169 MB) fit in the
# 256 MB Infinity Cache, so one set would be timed warm
MASKED_QUANT_SETS = 4


def _nsets(set_bytes: int, cap: int = 8) -> int:
    return max(1, min(cap, -(-(1 << 30) // max(set_bytes, 1))))


# --------------------------------------------------------------------------- ceilings
def _progress(msg: str) -> None:
    """One line per finished phase on stderr (the JSON line alone goes to stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _bench_lib():
    lib = ctypes.CDLL(BENCH_LIB)
    for name in ("fp8q_bench_copy", "fp8q_bench_stream"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
    lib.fp8q_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.fp8q_bench_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    lib.fp8q_bench_mfma.restype = ctypes.c_int
    lib.fp8q_bench_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    return lib


def ceilings(launches: int) -> dict:
    """The copy and stream reference kernels at the sizes of the dense workload, and the
    GEMM's MFMA instruction mix run from registers."""
    import torch
    lib = _bench_lib()
    dev = torch.device("cuda", 0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M, K, N = 4096, 7168, 4096
    out = {}
    ns = _nsets(3 * M * K)
    xs = [torch.zeros((M, K), dtype=torch.int16, device=dev) for _ in range(ns)]
    qs = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(ns)]
    stream = lambda: torch.cuda.current_stream().cuda_stream
    best = None
    for grid in (2048, 4096, 8192):
        def cp(i, grid=grid):
            rc = lib.fp8q_bench_copy(xs[i % ns].data_ptr(), qs[i % ns].data_ptr(), M * K, grid, stream())
            assert rc == 0, rc
        ms = graph_time_ms(cp, launches)
        if best is None or ms < best[0]:
            best = (ms, grid)
    nbytes = 3 * M * K
    out["copy"] = {"what": "bf16 -> byte copy, the dense M=4096 quant's traffic without scales",
                   "bytes": nbytes, "us": round(best[0] * 1e3, 2),
                   "GB/s": round(nbytes / (best[0] * 1e-3) / 1e9, 1),
                   "frac_hbm": round(nbytes / (best[0] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "grid": best[1]}
    del xs, qs
    ns = _nsets(N * K, 40)
    ws = [torch.zeros((N, K), dtype=torch.uint8, device=dev) for _ in range(ns)]
    sink = torch.empty(cus * 256, dtype=torch.int32, device=dev)

    def rd(i):
        rc = lib.fp8q_bench_stream(ws[i % ns].data_ptr(), N * K, sink.data_ptr(), cus, stream())
        assert rc == 0, rc
    ms = graph_time_ms(rd, launches)
    out["weight_stream"] = {"what": "read of the dense weights W [4096, 7168] once, one slice per CU",
                            "bytes": N * K, "us": round(ms * 1e3, 2), "GB/s": round(N * K / (ms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(N * K / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del ws
    # the GEMM's per-step instruction mix from registers (32 scaled FP8 MFMAs per wave and
    # step on real e4m3 codes, with or without the BLOCK128 fold), eight waves on every CU
    import synth
    codes = torch.from_numpy(synth.weight_codes(7, cus * 512, 192)).to(dev)
    sink = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    iters = 400
    flops = float(cus) * 8 * iters * 32 * 2 * 16 * 16 * 128
    for key, fold in (("mfma_stream", 0), ("mfma_fold_stream", 1)):
        def mx(i, fold=fold):
            rc = lib.fp8q_bench_mfma(codes.data_ptr(), iters, fold, sink.data_ptr(), cus, stream())
            assert rc == 0, rc
        ms = graph_time_ms(mx, max(4, launches // 8))
        out[key] = {"what": "32 scaled 16x16x128 FP8 MFMAs per wave and step from registers on e4m3 codes, "
                            + ("each product folded into fp32 by fma (BLOCK128)" if fold else
                               "accumulated in the matrix core (MXFP8)") + "; 8 waves per CU",
                    "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
                    "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
    del codes, sink
    # context: the vendor library's FP8 GEMM (torch._scaled_mm, hipBLASLt) on the dense shape,
    # with the simpler per-row x per-column fp32 scaling (no block-128 fold)
    try:
        xa = torch.from_numpy(synth.weight_codes(8, M, K)).to(dev).view(torch.float8_e4m3fn)
        wb = torch.from_numpy(synth.weight_codes(9, N, K)).to(dev).view(torch.float8_e4m3fn)
        sa = torch.ones((M, 1), dtype=torch.float32, device=dev)
        sbt = torch.ones((1, N), dtype=torch.float32, device=dev)
        # rotating operand sets, like the GEMM's own timing (one set would stay in the
        # Infinity Cache)
        nv = _nsets(2 * M * K + 2 * M * N)
        vsets = [(xa.clone(), wb.clone().t()) for _ in range(nv)]

        def mm(i):
            a, bt = vsets[i % nv]
            torch._scaled_mm(a, bt, scale_a=sa, scale_b=sbt, out_dtype=torch.bfloat16)
        ms = graph_time_ms(mm, max(4, launches // 4))
        out["vendor_fp8_gemm"] = {"what": "torch._scaled_mm (hipBLASLt) FP8 [4096, 7168] x [7168, 4096], row x column "
                                          "fp32 scales, bf16 out (no 128-block fold)",
                                  "us": round(ms * 1e3, 2), "buffer_sets": nv,
                                  "TFLOP/s": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        del xa, wb, vsets
    except Exception as ex:  # the backend may lack this form: recorded, not fatal
        out["vendor_fp8_gemm"] = {"error": repr(ex)[:200]}
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- configs
def _rec(cfg, workload, kernel, ms, bound, flops=None, nbytes=None, extra=None):
    rec = {"config": cfg, "workload": workload, "kernel": kernel, "us": round(ms * 1e3, 2), "bound": bound}
    if flops:
        t = flops / (ms * 1e-3) / 1e12
        rec["TFLOP/s"] = round(t, 1)
    if nbytes:
        rec["GB/s"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        rec["algorithmic_bytes"] = int(nbytes)
    if bound == "mfma":
        rec["frac"] = round(flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)
    elif bound == "hbm":
        rec["frac"] = round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    if extra:
        rec.update(extra)
    return rec


def configs(launches: int, ceil: dict | None) -> list:
    """One record per kernel of every named workload (graph-replayed launch loops)."""
    import torch
    import fp8_group_quant_amd as fq
    import synth
    dev = torch.device("cuda", 0)
    recs = []
    copy_gbs = ceil["copy"]["GB/s"] if ceil else None
    stream_gbs = ceil["weight_stream"]["GB/s"] if ceil else None
    fold_tf = ceil["mfma_fold_stream"]["TFLOP/s"] if ceil else None
    mix_tf = ceil["mfma_stream"]["TFLOP/s"] if ceil else None

    def note(r):
        recs.append(r)
        print(json.dumps(r), file=sys.stderr, flush=True)

    # c1 tiny, c2 dense (M = 1, 16, 128, 4096) and c3 (fused silu): quant then GEMM, rotating
    # buffer sets. Binding roofline: the quant streams HBM at M = 4096 and 8192 (smaller M is
    # latency-bound); the GEMM is bound by HBM (reading W) for M <= 128 and by the matrix
    # cores at M = 4096 and 8192; the tiny workload is latency-bound throughout.
    weights = {}
    for cfg, w in (("c1", synth.TINY), ("c2", synth.dense(1)), ("c2", synth.dense(16)), ("c2", synth.dense(128)),
                   ("c2", synth.dense(4096)), ("c3", synth.SILU)):
        M, K, N, G = w.M, w.K, w.N, w.G
        x = torch.from_numpy(synth.quant_input(w)).to(dev).view(torch.bfloat16)
        key = (w.seed, N, K)
        if key not in weights:
            wq, wsc = synth.weights(w)
            weights = {key: (torch.from_numpy(wq).to(dev), torch.from_numpy(wsc).to(dev))}
        wd, wsd = weights[key]
        set_bytes = x.numel() * 2 + M * K + wd.numel() + M * N * 2
        ns = _nsets(set_bytes, 40)
        sets = [dict(x=x.clone(), q=torch.empty((M, K), dtype=torch.uint8, device=dev),
                     s=fq.alloc_scales(None, M, K // G, w.scale_fmt, w.layout, dev), w=wd.clone(), sw=wsd.clone(),
                     y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for _ in range(ns)]
        qf = fq.fp8q_silu_mul_group_quant if w.silu else fq.fp8q_group_quant
        sb = 1 if w.scale_fmt == "ue8m0" else 4
        big = M >= 4096
        ms = graph_time_ms(lambda i: qf(sets[i % ns]["x"], sets[i % ns]["q"], sets[i % ns]["s"], G), launches)
        qb = quant_bytes(M, K, G, 2, sb, w.silu)
        extra = {"frac_copy": round(qb / (ms * 1e-3) / 1e9 / copy_gbs, 4)} if copy_gbs and big else None
        note(_rec(cfg, w.name, "silu_mul_group_quant" if w.silu else "group_quant", ms, "hbm" if big else "latency",
                  nbytes=qb, extra=extra))
        ms = graph_time_ms(lambda i: fq.fp8q_gemm_blockscaled(sets[i % ns]["q"], sets[i % ns]["s"], sets[i % ns]["w"],
                                                             sets[i % ns]["sw"], sets[i % ns]["y"]), launches)
        gb = gemm_bytes(M, N, K, sb, 4)
        bound = "latency" if w.name == "tiny" else ("mfma" if big else "hbm")
        extra = None
        if bound == "hbm" and stream_gbs:
            extra = {"frac_weight_stream": round(gb / (ms * 1e-3) / 1e9 / stream_gbs, 4)}
        elif bound == "mfma" and fold_tf:
            extra = {"frac_mfma_mix": round(2.0 * M * N * K / (ms * 1e-3) / 1e12 / fold_tf, 4)}
        note(_rec(cfg, w.name, "gemm_blockscaled", ms, bound, flops=2.0 * M * N * K, nbytes=gb, extra=extra))
        del sets, x
        torch.cuda.empty_cache()
    del weights
    torch.cuda.empty_cache()

    # c4 masked MoE: masked quant and the masked grouped GEMM over the 32 experts
    w = synth.MASKED
    E, cap, K, N, G = w.E, w.M, w.K, w.N, w.G
    mm = synth.masked_rows(w.seed, E, cap)
    rows = int(mm.sum())
    x = torch.from_numpy(np.stack([synth.quant_input(w, e) for e in range(E)])).to(dev).view(torch.bfloat16)
    mmd = torch.from_numpy(mm).to(dev)
    # rotating buffer sets: one set's valid rows (168 MB moved) would otherwise stay in the
    # 256 MB Infinity Cache between launches
    qsets = [dict(x=x.clone(), q=torch.empty((E, cap, K), dtype=torch.uint8, device=dev),
                  s=fq.alloc_scales(E, cap, K // G, "ue8m0", "col", dev)) for _ in range(MASKED_QUANT_SETS)]
    del x
    ms = graph_time_ms(lambda i: fq.fp8q_group_quant(qsets[i % MASKED_QUANT_SETS]["x"], qsets[i % MASKED_QUANT_SETS]["q"],
                                                     qsets[i % MASKED_QUANT_SETS]["s"], G, masked_m=mmd,
                                                     expected_m=cap // 2), launches)
    note(_rec("c4", w.name, "group_quant_masked", ms, "hbm", nbytes=quant_bytes(rows, K, G, 2, 1, False),
              extra={"sum_masked_m": rows, "buffer_sets": MASKED_QUANT_SETS}))
    q, sq = qsets[0]["q"], qsets[0]["s"]
    del qsets
    wq = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
    for e in range(E):
        a, b = synth.weights(w, e)
        wq[e].copy_(torch.from_numpy(a))
        ws[e].copy_(torch.from_numpy(b))
    y = torch.empty((E, cap, N), dtype=torch.bfloat16, device=dev)
    ms = graph_time_ms(lambda i: fq.fp8q_grouped_gemm_masked(q, sq, wq, ws, y, mmd, cap // 2), max(4, launches // 4))
    active = int((mm > 0).sum())
    gb = rows * K + active * N * K + rows * (K // 128) + active * (N // 128) * (K // 128) * 4 + rows * N * 2
    note(_rec("c4", w.name, "grouped_gemm_masked", ms, "hbm", flops=2.0 * rows * N * K, nbytes=gb,
              extra={"sum_masked_m": rows}))
    del wq, ws, q, y
    torch.cuda.empty_cache()

    # c5 MXFP8 8192^3, E8M0 row-major bytes [rows, K/32]
    w = synth.MX
    a, b, ea, eb = synth.mx_operands(w)
    ad, bd, ead, ebd = (torch.from_numpy(t).to(dev) for t in (a, b, ea, eb))
    ns = _nsets(a.nbytes + b.nbytes + w.M * w.N * 2, 4)
    sets = [dict(a=ad.clone(), b=bd.clone(), ea=ead.clone(), eb=ebd.clone(),
                 y=torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)) for _ in range(ns)]
    ms = graph_time_ms(lambda i: fq.fp8q_gemm_blockscaled(sets[i % ns]["a"], sets[i % ns]["ea"], sets[i % ns]["b"],
                                                         sets[i % ns]["eb"], sets[i % ns]["y"], fq.GEMM_MX32),
                       max(4, launches // 4))
    note(_rec("c5", w.name, "gemm_mx32", ms, "mfma", flops=2.0 * w.M * w.N * w.K,
              nbytes=a.nbytes + b.nbytes + ea.nbytes + eb.nbytes + w.M * w.N * 2,
              extra={"scales": "E8M0 bytes, row-major [rows, K/32]",
                     **({"frac_mfma_mix": round(2.0 * w.M * w.N * w.K / (ms * 1e-3) / 1e12 / mix_tf, 4)} if mix_tf else {})}))
    # the same operands with both scale tensors as column-major packed words [K/128, rows]
    # (the layout the G=32 quant writes with packed column-major UE8M0 scales)
    def col_words(e):
        return torch.from_numpy(np.ascontiguousarray(np.ascontiguousarray(e).view(np.uint32).T).view(np.int32)).to(dev).t()
    for st in sets:
        st["ea"], st["eb"] = col_words(ea), col_words(eb)
    ms = graph_time_ms(lambda i: fq.fp8q_gemm_blockscaled(sets[i % ns]["a"], sets[i % ns]["ea"], sets[i % ns]["b"],
                                                         sets[i % ns]["eb"], sets[i % ns]["y"], fq.GEMM_MX32),
                       max(4, launches // 4))
    note(_rec("c5", w.name, "gemm_mx32", ms, "mfma", flops=2.0 * w.M * w.N * w.K,
              nbytes=a.nbytes + b.nbytes + ea.nbytes + eb.nbytes + w.M * w.N * 2,
              extra={"scales": "E8M0 packed words, column-major [K/128, rows]",
                     **({"frac_mfma_mix": round(2.0 * w.M * w.N * w.K / (ms * 1e-3) / 1e12 / mix_tf, 4)} if mix_tf else {})}))
    del sets
    torch.cuda.empty_cache()
    return recs


# --------------------------------------------------------------------------- parity gate
def parity_gate(w, x_host, w_host, sw_host, q_dev, s_dev, y_dev) -> dict:
    """The step's own outputs (set 0) against the CPU oracle: every quant byte, and sampled
    GEMM outputs under the parity tests' rule (tests/gemm_check.py)."""
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gemm_check import check
    t0 = time.perf_counter()
    fmt = oracle.SCALE_UE8M0 if w.scale_fmt == "ue8m0" else oracle.SCALE_F32
    qo, so = oracle.group_quant(x_host, w.G, fmt, w.layout, silu=w.silu)
    qg = q_dev.cpu().numpy()
    sg = s_dev.cpu().numpy() if w.layout == "row" else s_dev.t().cpu().numpy()
    q_diff = int(np.count_nonzero(qg != qo))
    s_diff = int(np.count_nonzero(sg.view(np.uint8) != np.ascontiguousarray(so).view(np.uint8)))
    g = np.random.default_rng(2024)
    M, N = w.M, w.N
    ms = g.integers(0, M, 5000)
    ns = g.integers(0, N, 5000)
    m0 = int(g.integers(0, -(-M // 256))) * 256
    n0 = int(g.integers(0, -(-N // 256))) * 256
    tm, tn = np.meshgrid(np.arange(m0, min(M, m0 + 256)), np.arange(n0, min(N, n0 + 256)), indexing="ij")
    ms = np.concatenate([ms, tm.ravel()])
    ns = np.concatenate([ns, tn.ravel()])
    ys, ss = oracle.gemm_block128(qo, so, w_host, sw_host, fmt, w.layout, at=(ms, ns))
    yg = y_dev.view(__import__("torch").int16).cpu().numpy().view(np.uint16)[ms, ns]
    gate = {"quant_rows": M, "quant_codes_differing": q_diff, "quant_scale_bytes_differing": s_diff}
    try:
        st = check(yg, ys, ss, w.K, "bench parity gate", cls="quant")
        gate["gemm"] = {k: st[k] for k in ("n", "n_cancel", "max_excess_over_S", "gamma", "n_beyond_gamma", "frob",
                                            "frob_bf16_floor")}
        gemm_ok = True
    except AssertionError as err:
        gate["gemm"] = {"n": int(ms.size), "failure": str(err)[:300]}
        gemm_ok = False
    gate["pass"] = bool(q_diff == 0 and s_diff == 0 and gemm_ok)
    gate["seconds"] = round(time.perf_counter() - t0, 1)
    return gate


# --------------------------------------------------------------------------- CPU baseline
def _oracle_step_time(w, x_host, w_host, sw_host, rows: int, cols: int) -> tuple[float, float]:
    """Seconds the oracle takes for `rows` quantized rows and rows x cols GEMM outputs, and the
    full step time extrapolated per row and per output."""
    import oracle
    M, N = w.M, w.N
    fmt = oracle.SCALE_UE8M0 if w.scale_fmt == "ue8m0" else oracle.SCALE_F32
    t0 = time.perf_counter()
    q, s = oracle.group_quant(x_host[:rows], w.G, fmt, w.layout, silu=w.silu)
    t1 = time.perf_counter()
    ms = np.repeat(np.arange(rows), cols)
    ns = np.tile(np.arange(cols), rows)
    oracle.gemm_block128(q, s, w_host, sw_host, fmt, w.layout, at=(ms, ns))
    t2 = time.perf_counter()
    return t2 - t0, (t1 - t0) / rows * M + (t2 - t1) / (rows * cols) * (M * N)


def cpu_baseline(w, x_host, w_host, sw_host, rows: int) -> dict:
    """The plain oracle on the host's cores (its OpenMP loops over rows and outputs; each
    row or output is computed whole by one thread), on a bounded sample of the same
    workload, scaled to the step: all cores, and one core."""
    import oracle
    flops = 2.0 * w.M * w.N * w.K
    nproc = os.cpu_count()
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    threads = oracle.max_threads()
    rows_all = min(w.M, 4 * rows)
    t_all, step_all = _oracle_step_time(w, x_host, w_host, sw_host, rows_all, 1024)
    with oracle.threads(1):
        t_one, step_one = _oracle_step_time(w, x_host, w_host, sw_host, rows // 2, 512)
    return {"value": round(flops / step_all / 1e12, 8), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_all} rows quantized + {rows_all}x1024 GEMM outputs of the same workload on {threads} "
                      f"threads ({t_all:.1f} s); step time extrapolated per row / per output = {step_all:.1f} s",
            "nproc": nproc, "cpus_available": avail,
            "single_core": {"value": round(flops / step_one / 1e12, 8), "unit": "TFLOP/s", "cores": 1,
                            "sample": f"{rows // 2} rows + {rows // 2}x512 outputs ({t_one:.1f} s); "
                                      f"extrapolated step = {step_one:.0f} s"}}


# --------------------------------------------------------------------------- the step line
def run(args) -> dict:
    import torch
    import fp8_group_quant_amd as fq
    import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    fq.load_library()
    if fq.fp8q_device_check(0) != fq.OK:
        raise SystemExit("device 0 is not a gfx950: " + fq.fp8q_last_error())
    w = build_workload(args.workload)
    M, K, N, G = w.M, w.K, w.N, w.G
    dev = torch.device("cuda", 0)

    # ---- synthetic inputs, resident in HBM
    x_host = synth.quant_input(w)
    w_host, sw_host = synth.weights(w)
    ue8m0 = w.scale_fmt == "ue8m0"
    x0 = torch.from_numpy(x_host).to(dev).view(torch.bfloat16)
    w0 = torch.from_numpy(w_host).to(dev)
    sw0 = torch.from_numpy(sw_host).to(dev)
    set_bytes = x0.numel() * 2 + M * K + w0.numel() + M * N * 2
    nsets = max(2, min(16, -(-(1 << 30) // set_bytes)))  # >= 1 GiB working set
    sets = []
    for _ in range(nsets):
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        s = fq.alloc_scales(None, M, K // G, w.scale_fmt, w.layout, dev)
        sets.append(dict(x=x0.clone(), q=q, s=s, w=w0.clone(), sw=sw0.clone(),
                         y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    if args.calibration_copies:
        # reference copies of known size for counter runs (record_traffic)
        src = torch.zeros(CALIBRATION_ELEMS, dtype=torch.int16, device=dev)
        dst = torch.empty(CALIBRATION_ELEMS, dtype=torch.uint8, device=dev)
        blib = _bench_lib()
        for _ in range(args.calibration_copies):
            rc = blib.fp8q_bench_copy(src.data_ptr(), dst.data_ptr(), CALIBRATION_ELEMS, 4096,
                                      torch.cuda.current_stream().cuda_stream)
            assert rc == 0, rc
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        """one pass of the path; ev = (before quant, before GEMM, after GEMM) events to record"""
        st = sets[i % nsets]
        if ev:
            ev[0].record(stream)
        if w.silu:
            fq.fp8q_silu_mul_group_quant(st["x"], st["q"], st["s"], G)
        else:
            fq.fp8q_group_quant(st["x"], st["q"], st["s"], G)
        if ev:
            ev[1].record(stream)
        fq.fp8q_gemm_blockscaled(st["q"], st["s"], st["w"], st["sw"], st["y"], fq.GEMM_BLOCK128)
        if ev:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(fn, n, warm=0):
        """average ms of n back-to-back launches between two events on the kernels' stream,
        after `warm` untimed launches queued right before them (the GPU is busy, not idle
        after a synchronize, when the first timed launch starts)"""
        e0, e1 = _events()
        torch.cuda.synchronize()
        for i in range(warm):
            fn(n + i)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def quant_only(i):
        st = sets[i % nsets]
        if w.silu:
            fq.fp8q_silu_mul_group_quant(st["x"], st["q"], st["s"], G)
        else:
            fq.fp8q_group_quant(st["x"], st["q"], st["s"], G)

    def gemm_only(i):
        st = sets[i % nsets]
        fq.fp8q_gemm_blockscaled(st["q"], st["s"], st["w"], st["sw"], st["y"], fq.GEMM_BLOCK128)

    # the timed steps: exactly args.steps passes of the whole path
    ms_step = timed(lambda i: step(args.warmup + i), args.steps)
    # the same passes again, right after, with events on the kernels' stream around each
    # launch: each kernel's launch duration under the step loop's conditions (the events
    # add a few microseconds per step, so they stay out of the timed steps above)
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    quant_in_step = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    gemm_in_step = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    # per-kernel averages (each kernel alone, same buffer rotation, warmed like the steps)
    kwarm = max(args.warmup, 10)
    quant_ms = timed(quant_only, args.steps, kwarm)
    gemm_ms = timed(gemm_only, args.steps, kwarm)

    flops = 2.0 * M * N * K
    qbytes = quant_bytes(M, K, G, 2, 1 if ue8m0 else 4, w.silu)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    quant_gbs = qbytes / (quant_ms * 1e-3) / 1e9
    gemm_step_tflops = flops / (gemm_in_step * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12

    # the outputs of set 0, for the parity gate (the last step that used set 0 wrote them)
    step(0)
    torch.cuda.synchronize()
    out_set = sets[0]

    traffic = _measured_traffic("gemm.hip", w.name)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp8e4m3 -> fp32 acc -> bf16 (quant: bf16 -> e4m3, fp32 arithmetic)",
        "data": "synthetic (seeded Philox; shapes and distributions of the named workload, no weights)",
        "config": {"workload": w.name, "M": M, "K": K, "N": N, "group_size": G,
                   "act_scale": f"{w.scale_fmt} {w.layout}-major", "weight_scale": "fp32 128x128",
                   "buffer_sets": nsets, "silu": w.silu},
        # the GEMM's average launch duration in its own loop of K back-to-back launches (no
        # events between launches; this is the figure that matches the kernel trace)
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic},
        "kernels": {
            "group_quant": {"avg_ms_in_steps": round(quant_in_step, 5), "avg_ms": round(quant_ms, 5),
                            "algorithmic_bytes": qbytes,
                            "GB/s": round(quant_gbs, 1), "frac_hbm": round(quant_gbs / PEAK_HBM_GBS, 4),
                            "traffic": _measured_traffic("quant.hip", w.name)},
            "gemm_blockscaled": {"avg_ms_in_steps": round(gemm_in_step, 5), "avg_ms": round(gemm_ms, 5),
                                 "flops": flops, "TFLOP/s": round(gemm_tflops, 2),
                                 "TFLOP/s_in_steps": round(gemm_step_tflops, 2),
                                 "frac_mfma": round(gemm_tflops / PEAK_FP8_TFLOPS, 4)},
        },
    }
    del sets[1:]
    torch.cuda.empty_cache()
    _progress(f"steps timed: {out['ms_per_step']} ms per step")
    if not args.no_configs:
        ceil = ceilings(args.config_launches)
        out["ceilings"] = ceil
        out["kernels"]["group_quant"]["frac_copy"] = round(quant_gbs / ceil["copy"]["GB/s"], 4)
        # the GEMM against what its own MFMA-and-fold instruction mix sustains from registers
        out["kernels"]["gemm_blockscaled"]["frac_mfma_mix"] = round(
            gemm_tflops / ceil["mfma_fold_stream"]["TFLOP/s"], 4)
        _progress("ceilings done")
        out["configs"] = configs(args.config_launches, ceil)
    if not args.no_parity:
        out["parity"] = parity_gate(w, x_host, w_host, sw_host, out_set["q"], out_set["s"], out_set["y"])
        _progress("parity gate done")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x_host, w_host, sw_host, args.cpu_rows)
        _progress("cpu baseline done")
    return out


def _timed(fn, n, warm=0):
    """average ms of n back-to-back launches, after `warm` untimed ones queued right before"""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for i in range(warm):
        fn(n + i)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


SUITE_SECTIONS = ("flat", "variants", "masked", "moe_down", "mxfp8")


def suite(steps: int, warmup: int, only=None) -> list:
    """Per-kernel figures for every named workload (quant GB/s, GEMM TFLOP/s and HBM GB/s),
    each timed over `steps` launches rotating over >= 1 GiB of buffers where memory allows.
    `only`: a subset of SUITE_SECTIONS to run (all when None)."""
    import torch
    import fp8_group_quant_amd as fq
    import synth
    dev = torch.device("cuda", 0)
    fq.load_library()
    lines = []

    def report(name, kind, ms, flops=None, nbytes=None, extra=None):
        rec = {"workload": name, "kernel": kind, "us": round(ms * 1e3, 2)}
        if flops:
            t = flops / (ms * 1e-3) / 1e12
            rec.update({"TFLOP/s": round(t, 1), "frac_mfma": round(t / PEAK_FP8_TFLOPS, 4)})
        if nbytes:
            g = nbytes / (ms * 1e-3) / 1e9
            rec.update({"GB/s": round(g, 1), "frac_hbm": round(g / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes})
        if extra:
            rec.update(extra)
        lines.append(rec)
        print(json.dumps(rec), flush=True)

    def run(fn, n_sets):
        return _timed(fn, steps, max(warmup, 10))

    def want(section):
        return only is None or section in only

    if want("flat"):
        # flat workloads: quant then block-scaled GEMM
        for w in (synth.TINY, synth.dense(1), synth.dense(16), synth.dense(128), synth.dense(4096), synth.SILU):
            M, K, N, G = w.M, w.K, w.N, w.G
            x = torch.from_numpy(synth.quant_input(w)).to(dev).view(torch.bfloat16)
            wq, ws = synth.weights(w)
            wd, wsd = torch.from_numpy(wq).to(dev), torch.from_numpy(ws).to(dev)
            set_bytes = x.numel() * 2 + M * K + wd.numel() + M * N * 2
            ns = _nsets(set_bytes)
            sets = [dict(x=x.clone(), q=torch.empty((M, K), dtype=torch.uint8, device=dev),
                         s=fq.alloc_scales(None, M, K // G, w.scale_fmt, w.layout, dev), w=wd.clone(), sw=wsd.clone(),
                         y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for _ in range(ns)]
            qf = fq.fp8q_silu_mul_group_quant if w.silu else fq.fp8q_group_quant
            ms = run(lambda i: qf(sets[i % ns]["x"], sets[i % ns]["q"], sets[i % ns]["s"], G), ns)
            report(w.name, "silu_mul_group_quant" if w.silu else "group_quant", ms,
                   nbytes=quant_bytes(M, K, G, 2, 1 if w.scale_fmt == "ue8m0" else 4, w.silu))
            ms = run(lambda i: fq.fp8q_gemm_blockscaled(sets[i % ns]["q"], sets[i % ns]["s"], sets[i % ns]["w"],
                                                        sets[i % ns]["sw"], sets[i % ns]["y"]), ns)
            sbytes = M * (K // 128) * (1 if w.scale_fmt == "ue8m0" else 4) + ws.nbytes
            report(w.name, "gemm_blockscaled", ms, flops=2.0 * M * N * K, nbytes=M * K + N * K + sbytes + M * N * 2)
            del sets
            torch.cuda.empty_cache()

    if want("variants"):
        # quant variants on the dense M=4096 activations: per-token (G = K, one fp32 scale per
        # row) and int8 output (G = 128, fp32 row-major scales)
        w = synth.dense(4096)
        M, K = w.M, w.K
        x = torch.from_numpy(synth.quant_input(w)).to(dev).view(torch.bfloat16)
        ns = _nsets(x.numel() * 3)
        sets = [dict(x=x.clone(), q=torch.empty((M, K), dtype=torch.uint8, device=dev),
                     s=torch.empty((M, 1), dtype=torch.float32, device=dev),
                     s8=torch.empty((M, K // 128), dtype=torch.float32, device=dev)) for _ in range(ns)]
        ms = run(lambda i: fq.fp8q_group_quant(sets[i % ns]["x"], sets[i % ns]["q"], sets[i % ns]["s"], K), ns)
        report("dense_m4096_per_token", "token_quant", ms, nbytes=quant_bytes(M, K, K, 2, 4, False),
               extra={"scales": "f32 [M, 1]"})
        ms = run(lambda i: fq.fp8q_group_quant_int8(sets[i % ns]["x"], sets[i % ns]["q"].view(torch.int8),
                                                    sets[i % ns]["s8"], 128), ns)
        report("dense_m4096_int8", "group_quant_int8", ms, nbytes=quant_bytes(M, K, 128, 2, 4, False),
               extra={"scales": "f32 row-major"})
        # the dense GEMM with UE8M0 weight-block scales (powers of two on both sides: applied by
        # the matrix core, no fold)
        N = w.N
        wq, ws = synth.weights(w)
        ws8 = synth.e8m0_exponents(w.seed, ws.shape[0], ws.shape[1], lo=-4, hi=4, tensor_id=synth.T_SW + 1)
        for st in sets:
            qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
            sa_col = fq.alloc_scales(None, M, K // 128, "ue8m0", "col", dev)
            fq.fp8q_group_quant(st["x"], qa, sa_col, 128)
            st.update(qa=qa, sa_col=sa_col, w=torch.from_numpy(wq).to(dev), sw8=torch.from_numpy(ws8).to(dev),
                      y=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
        ms = run(lambda i: fq.fp8q_gemm_blockscaled(sets[i % ns]["qa"], sets[i % ns]["sa_col"], sets[i % ns]["w"],
                                                    sets[i % ns]["sw8"], sets[i % ns]["y"]), ns)
        report("dense_m4096_ue8m0_weights", "gemm_blockscaled", ms, flops=2.0 * M * N * K,
               nbytes=M * K + N * K + M * (K // 128) + ws8.nbytes + M * N * 2,
               extra={"weight_scale": "ue8m0 128x128"})
        del sets, x
        torch.cuda.empty_cache()

    if want("masked"):
        # masked MoE: masked quant then masked grouped GEMM
        w = synth.MASKED
        E, cap, K, N, G = w.E, w.M, w.K, w.N, w.G
        mm = synth.masked_rows(w.seed, E, cap)
        rows = int(mm.sum())
        x = torch.from_numpy(np.stack([synth.quant_input(w, e) for e in range(E)])).to(dev).view(torch.bfloat16)
        mmd = torch.from_numpy(mm).to(dev)
        ns = MASKED_QUANT_SETS
        qsets = [dict(x=x.clone(), q=torch.empty((E, cap, K), dtype=torch.uint8, device=dev),
                      s=fq.alloc_scales(E, cap, K // G, "ue8m0", "col", dev)) for _ in range(ns)]
        del x
        ms = run(lambda i: fq.fp8q_group_quant(qsets[i % ns]["x"], qsets[i % ns]["q"], qsets[i % ns]["s"], G,
                                               masked_m=mmd, expected_m=cap // 2), ns)
        report(w.name, "group_quant_masked", ms, nbytes=quant_bytes(rows, K, G, 2, 1, False),
               extra={"sum_masked_m": rows, "buffer_sets": ns})
        q, sq = qsets[0]["q"], qsets[0]["s"]
        del qsets
        wq = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        ws = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            a, b = synth.weights(w, e)
            wq[e].copy_(torch.from_numpy(a))
            ws[e].copy_(torch.from_numpy(b))
        y = torch.empty((E, cap, N), dtype=torch.bfloat16, device=dev)
        ms = run(lambda i: fq.fp8q_grouped_gemm_masked(q, sq, wq, ws, y, mmd, cap // 2), 1)
        active = int((mm > 0).sum())
        gemm_bytes = rows * K + active * N * K + rows * (K // 128) + active * ws[0].numel() * 4 + rows * N * 2
        report(w.name, "grouped_gemm_masked", ms, flops=2.0 * rows * N * K, nbytes=gemm_bytes,
               extra={"sum_masked_m": rows})
        del y
        # the same experts' rows packed one after another: the contiguous layout (each expert at a
        # 128-aligned offset, padded with m_indices = -1; UE8M0 column-major scales) and segments
        # (no padding; packed UE8M0 words, which are the row-major bytes read as int32)
        sq_store = sq.transpose(1, 2)  # [E, K/128, cap] storage
        blocks = (mm.astype(np.int64) + 127) // 128
        offs = np.concatenate([[0], np.cumsum(blocks * 128)])
        Tc = int(offs[-1])
        ac = torch.zeros((Tc, K), dtype=torch.uint8, device=dev)
        sc = torch.zeros((K // G, Tc), dtype=torch.uint8, device=dev)
        mi = torch.full((Tc,), -1, dtype=torch.int32, device=dev)
        seg = np.concatenate([[0], np.cumsum(mm.astype(np.int64))])
        asg = torch.empty((rows, K), dtype=torch.uint8, device=dev)
        ssg = torch.empty((rows, K // G), dtype=torch.uint8, device=dev)
        for e in range(E):
            m, o, so = int(mm[e]), int(offs[e]), int(seg[e])
            ac[o:o + m] = q[e, :m]
            sc[:, o:o + m] = sq_store[e, :, :m]
            mi[o:o + m] = e
            asg[so:so + m] = q[e, :m]
            ssg[so:so + m] = sq_store[e, :, :m].t()
        yc = torch.empty((Tc, N), dtype=torch.bfloat16, device=dev)
        ms = run(lambda i: fq.fp8q_grouped_gemm_contiguous(ac, sc.t(), wq, ws, yc, mi), 1)
        report("contiguous_moe", "grouped_gemm_contiguous", ms, flops=2.0 * rows * N * K, nbytes=gemm_bytes,
               extra={"rows": rows, "padded_rows": Tc, "layout": "masked_moe experts, 128-aligned, m_indices"})
        del yc, ac, sc, mi
        ys = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
        sid = torch.from_numpy(seg.astype(np.int32)).to(dev)
        ms = run(lambda i: fq.fp8q_grouped_gemm_segments(asg, ssg.view(torch.int32), wq, ws, ys, sid,
                                                         expected_rows=rows), 1)
        report("segments_moe", "grouped_gemm_segments", ms, flops=2.0 * rows * N * K, nbytes=gemm_bytes,
               extra={"rows": rows, "layout": "masked_moe experts, seg_indptr, packed UE8M0 words"})
        del ys, asg, ssg, wq, q
        torch.cuda.empty_cache()

    if want("moe_down"):
        # MoE second stage: masked silu_and_mul + quant into packed UE8M0 words (column-major,
        # four groups per word), then the masked grouped down-projection GEMM
        w = synth.MASKED_DOWN
        E, cap, K, N, G = w.E, w.M, w.K, w.N, w.G
        mm = synth.masked_rows(w.seed, E, cap)
        rows = int(mm.sum())
        h = torch.from_numpy(np.stack([synth.quant_input(w, e) for e in range(E)])).to(dev).view(torch.bfloat16)
        mmd = torch.from_numpy(mm).to(dev)
        ns = MASKED_QUANT_SETS
        qsets = [dict(h=h.clone(), q=torch.empty((E, cap, K), dtype=torch.uint8, device=dev),
                      s=fq.alloc_scales(E, cap, K // G, "ue8m0_packed", "col", dev)) for _ in range(ns)]
        del h
        ms = run(lambda i: fq.fp8q_silu_mul_group_quant(qsets[i % ns]["h"], qsets[i % ns]["q"], qsets[i % ns]["s"], G,
                                                        masked_m=mmd, expected_m=cap // 2), ns)
        report(w.name, "silu_mul_group_quant_masked", ms, nbytes=quant_bytes(rows, K, G, 2, 1, True),
               extra={"sum_masked_m": rows, "scales": "ue8m0 packed, column-major words", "buffer_sets": ns})
        q, sq = qsets[0]["q"], qsets[0]["s"]
        del qsets
        wq = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        ws = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            a, b = synth.weights(w, e)
            wq[e].copy_(torch.from_numpy(a))
            ws[e].copy_(torch.from_numpy(b))
        y = torch.empty((E, cap, N), dtype=torch.bfloat16, device=dev)
        ms = run(lambda i: fq.fp8q_grouped_gemm_masked(q, sq, wq, ws, y, mmd, cap // 2), 1)
        active = int((mm > 0).sum())
        report(w.name, "grouped_gemm_masked", ms, flops=2.0 * rows * N * K,
               nbytes=rows * K + active * N * K + rows * (K // 128) + active * ws[0].numel() * 4 + rows * N * 2,
               extra={"sum_masked_m": rows})
        del wq, q, y
        torch.cuda.empty_cache()

    if want("mxfp8"):
        # MXFP8
        w = synth.MX
        a, b, ea, eb = synth.mx_operands(w)
        ad, bd, ead, ebd = (torch.from_numpy(t).to(dev) for t in (a, b, ea, eb))
        ns = _nsets(a.nbytes + b.nbytes + w.M * w.N * 2, 4)
        sets = [dict(a=ad.clone(), b=bd.clone(), ea=ead.clone(), eb=ebd.clone(),
                     y=torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)) for _ in range(ns)]
        ms = run(lambda i: fq.fp8q_gemm_blockscaled(sets[i % ns]["a"], sets[i % ns]["ea"], sets[i % ns]["b"],
                                                    sets[i % ns]["eb"], sets[i % ns]["y"], fq.GEMM_MX32), ns)
        report(w.name, "gemm_mx32", ms, flops=2.0 * w.M * w.N * w.K,
               nbytes=a.nbytes + b.nbytes + ea.nbytes + eb.nbytes + w.M * w.N * 2,
               extra={"scales": "E8M0 bytes, row-major [rows, K/32]"})
        # the same operands with both scale tensors as column-major packed words [K/128, rows]
        # (four E8M0 bytes of one 128-wide K step per 32-bit word)
        def col_words(e):
            wd = e.view(np.uint32) if e.flags.c_contiguous else np.ascontiguousarray(e).view(np.uint32)
            return torch.from_numpy(np.ascontiguousarray(wd.T).view(np.int32)).to(dev).t()
        for st in sets:
            st["ea"], st["eb"] = col_words(ea), col_words(eb)
        ms = run(lambda i: fq.fp8q_gemm_blockscaled(sets[i % ns]["a"], sets[i % ns]["ea"], sets[i % ns]["b"],
                                                    sets[i % ns]["eb"], sets[i % ns]["y"], fq.GEMM_MX32), ns)
        report(w.name, "gemm_mx32", ms, flops=2.0 * w.M * w.N * w.K,
               nbytes=a.nbytes + b.nbytes + ea.nbytes + eb.nbytes + w.M * w.N * 2,
               extra={"scales": "E8M0 packed words, column-major [K/128, rows]"})
    return lines


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_m4096")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--config-launches", type=int, default=40,
                    help="launches per graph-replayed loop in the configs and ceilings records")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the configs and ceilings records")
    ap.add_argument("--no-parity", action="store_true", help="skip the in-run parity gate")
    ap.add_argument("--only", default=None,
                    help="with --suite: comma-separated sections to run (" + ",".join(SUITE_SECTIONS) + ")")
    ap.add_argument("--suite", action="store_true",
                    help="print per-kernel lines for every named workload instead of the step line")
    ap.add_argument("--calibration-copies", type=int, default=0,
                    help="launch this many reference copies of known size before the steps (counter runs)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="(no GPU) merge the --workload's HBM bytes per call from two rocprofv3 counter runs "
                         "of the step loop into profiles/traffic.json")
    args = ap.parse_args(argv)
    if args.record_traffic:
        print(json.dumps(record_traffic(args.workload, *args.record_traffic)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              f"multi-GPU path", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")
    if args.suite:
        only = None
        if args.only:
            only = set(args.only.split(","))
            bad = only - set(SUITE_SECTIONS)
            if bad:
                raise SystemExit(f"unknown suite sections: {sorted(bad)}")
        suite(args.steps, args.warmup, only)
        return 0
    print(json.dumps(run(args)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

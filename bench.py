"""Benchmark of the FP8 group-quant -> block-scaled FP8 GEMM path on one MI355X.

One step = the whole hot path over one batch of synthetic input resident in HBM:
per-token-group quantization of bf16 activations (UE8M0 column-major scales) followed by
the 1x128 x 128x128 block-scaled FP8 GEMM against e4m3 weights, bf16 output. The default
workload is the dense DeepSeek-V3-like projection at M = 4096 (X [4096, 7168], W [4096,
7168]); --workload picks another named shape for reporting (extra lines are only printed
when asked for).

Timing: W untimed warm-up steps, then exactly K steps between two synchronizations,
measured with HIP events on the stream the kernels run on. The per-kernel roofline figures
come from two more event-timed loops of K launches of each kernel alone. To defeat the 256 MB
Infinity Cache and the L2s, the steps rotate over enough independent input/output buffer
sets that the working set exceeds 1 GB.

The CPU baseline is the plain oracle (single-threaded C), timed on a bounded sample of the
same workload in the same run and scaled to the metric's unit.
"""
from __future__ import annotations

import argparse
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


def _kernel_source_tag(name: str) -> str:
    """Hash of a kernel source and the shared internal header, with // comments and blank
    lines removed: a comment edit keeps the tag, any code change breaks it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for fn in (name, "fp8q_internal.h"):
        with open(os.path.join(ROOT, "fp8_group_quant_amd", "csrc", fn), encoding="utf-8") as f:
            for line in f:
                line = re.sub(r"//.*$", "", line).rstrip()
                if line.strip():
                    h.update(line.encode() + b"\n")
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


def quant_bytes(rows: int, K: int, G: int, in_bytes: int, scale_bytes: int, silu: bool) -> int:
    """Algorithmic bytes of one group-quant launch: read the input once, write codes + scales."""
    width = 2 * K if silu else K
    return rows * (width * in_bytes + K + (K // G) * scale_bytes)


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
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
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
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x_host, w_host, sw_host, args.cpu_rows)
    return out


def cpu_baseline(w, x_host, w_host, sw_host, rows: int) -> dict:
    """Times the plain oracle on a bounded sample of the same workload: quantization of
    `rows` activation rows, then the GEMM outputs of those rows against 512 weight rows.
    The per-row and per-output costs are scaled up to the full step and reported in the
    metric's unit."""
    import oracle
    M, K, N, G = w.M, w.K, w.N, w.G
    fmt = oracle.SCALE_UE8M0 if w.scale_fmt == "ue8m0" else oracle.SCALE_F32
    t0 = time.perf_counter()
    q, s = oracle.group_quant(x_host[:rows], G, fmt, w.layout, silu=w.silu)
    t1 = time.perf_counter()
    cols = min(N, 512)
    ms = np.repeat(np.arange(rows), cols)
    ns = np.tile(np.arange(cols), rows)
    oracle.gemm_block128(q, s, w_host, sw_host, fmt, w.layout, at=(ms, ns))
    t2 = time.perf_counter()
    t_step = (t1 - t0) / rows * M + (t2 - t1) / (rows * cols) * (M * N)
    return {"value": round(2.0 * M * N * K / t_step / 1e12, 8), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{rows} rows quantized + {rows}x{cols} GEMM outputs of the same workload "
                      f"({t2 - t0:.1f} s); step time extrapolated per row / per output = {t_step:.0f} s"}


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


def _nsets(set_bytes: int, cap: int = 8) -> int:
    return max(1, min(cap, -(-(1 << 30) // max(set_bytes, 1))))


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
        q = torch.empty((E, cap, K), dtype=torch.uint8, device=dev)
        sq = fq.alloc_scales(E, cap, K // G, "ue8m0", "col", dev)
        ms = run(lambda i: fq.fp8q_group_quant(x, q, sq, G, masked_m=mmd, expected_m=cap // 2), 1)
        report(w.name, "group_quant_masked", ms, nbytes=quant_bytes(rows, K, G, 2, 1, False), extra={"sum_masked_m": rows})
        del x
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
        q = torch.empty((E, cap, K), dtype=torch.uint8, device=dev)
        sq = fq.alloc_scales(E, cap, K // G, "ue8m0_packed", "col", dev)
        ms = run(lambda i: fq.fp8q_silu_mul_group_quant(h, q, sq, G, masked_m=mmd, expected_m=cap // 2), 1)
        report(w.name, "silu_mul_group_quant_masked", ms, nbytes=quant_bytes(rows, K, G, 2, 1, True),
               extra={"sum_masked_m": rows, "scales": "ue8m0 packed, column-major words"})
        del h
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="with --suite: comma-separated sections to run (" + ",".join(SUITE_SECTIONS) + ")")
    ap.add_argument("--suite", action="store_true",
                    help="print per-kernel lines for every named workload instead of the step line")
    args = ap.parse_args(argv)
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

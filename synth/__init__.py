"""Seeded synthetic inputs for the FP8 group-quant + block-scaled GEMM workloads.

This module serves both the HIP path and the CPU oracle, so it holds none of the
method's arithmetic: no amax, no scale computation, no quantization of activations
and no GEMM. It only draws random numbers and rounds them to the storage types the
workloads name (bf16 activations, e4m3 weight bytes, fp32 block scales, E8M0 bytes).

Random numbers come from numpy's Philox counter-based generator (Philox4x64-10,
Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11).
Every tensor is keyed by (workload seed, tensor id, chunk index), so the values do
not depend on thread counts or on how a caller batches its requests. Large tensors
are drawn one chunk (one expert, or one block of rows) at a time under their own
key; the chunking is part of the recipe.

Storage rounding uses library routines (torch's CPU casts): fp64 -> fp32 -> bf16
round-to-nearest-even for activations, and fp32 -> float8_e4m3fn for weight codes
(values are clamped to +-448 first, because that cast maps larger values to NaN).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

# tensor ids (second key word of each Philox stream)
T_X = 1
T_OUTLIER = 2
T_W = 3
T_SW = 4
T_MASK = 5
T_A = 6
T_B = 7
T_EA = 8
T_EB = 9

_CHUNK_ROWS = 4096  # rows per Philox stream for row-chunked tensors


def rng(seed: int, tensor_id: int, chunk: int = 0) -> np.random.Generator:
    """Philox4x64-10 stream keyed by (seed, tensor_id, chunk)."""
    key = np.array([seed & 0xFFFFFFFFFFFFFFFF, ((tensor_id & 0xFFFFFFFF) << 32) | (chunk & 0xFFFFFFFF)],
                   dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (both round-to-nearest-even), returned as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """fp32 values (clamped to +-448 first) -> float8_e4m3fn bytes via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _rows_chunked(seed: int, tensor_id: int, rows: int, cols: int, fn) -> np.ndarray:
    out = []
    for c, r0 in enumerate(range(0, rows, _CHUNK_ROWS)):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        out.append(fn(rng(seed, tensor_id, c), (r1 - r0, cols)))
    if not out:
        return fn(rng(seed, tensor_id, 0), (0, cols))
    return np.concatenate(out, axis=0)


def activations_bf16(seed: int, rows: int, cols: int, outlier_p: float = 0.0,
                     outlier_mul: float = 50.0, tensor_id: int = T_X) -> np.ndarray:
    """bf16 bits [rows, cols]: N(0,1); with outlier_p > 0 each entry independently is
    multiplied by outlier_mul with probability outlier_p (before rounding to bf16)."""
    def draw(g, shape):
        v = g.standard_normal(shape)
        if outlier_p > 0.0:
            hit = g.random(shape) < outlier_p
            v = np.where(hit, v * outlier_mul, v)
        return v
    return f64_to_bf16_bits(_rows_chunked(seed, tensor_id, rows, cols, draw))


def weight_codes(seed: int, rows: int, cols: int, tensor_id: int = T_W, sigma: float = 1.0) -> np.ndarray:
    """e4m3 bytes [rows, cols] of N(0, sigma^2) samples (values directly, no per-block
    scaling). sigma = 100 spreads the codes over the e4m3 range the way group-quantized
    activations do (their group maximum maps to about 448)."""
    return f32_to_e4m3_bytes(_rows_chunked(seed, tensor_id, rows, cols,
                                           lambda g, s: sigma * g.standard_normal(s)))


def block_scales(seed: int, rows: int, cols: int, sigma: float = 0.5,
                 tensor_id: int = T_SW) -> np.ndarray:
    """fp32 [rows, cols] ~ lognormal(0, sigma)."""
    g = rng(seed, tensor_id)
    return np.exp(sigma * g.standard_normal((rows, cols))).astype(np.float32)


def masked_rows(seed: int, experts: int, cap: int, tensor_id: int = T_MASK) -> np.ndarray:
    """int32 [experts] ~ Uniform{0..cap} (inclusive, unbiased integer draw)."""
    g = rng(seed, tensor_id)
    return g.integers(0, cap + 1, size=experts, dtype=np.int64).astype(np.int32)


def e8m0_exponents(seed: int, rows: int, cols: int, lo: int = -4, hi: int = 4,
                   tensor_id: int = T_EA) -> np.ndarray:
    """uint8 [rows, cols] = 127 + Uniform{lo..hi} (E8M0 bytes of 2^lo .. 2^hi)."""
    return _rows_chunked(seed, tensor_id, rows, cols,
                         lambda g, s: (127 + g.integers(lo, hi + 1, size=s)).astype(np.uint8))


# ------------------------------------------------------------------------------------
# workload recipes (sizes and distributions of the five named configurations)
# ------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    M: int = 0          # activation rows (flat), or capacity per expert (masked)
    K: int = 0          # quantized width (reduction dim of the GEMM)
    N: int = 0          # GEMM output columns (weight rows)
    E: int = 1          # experts (masked)
    G: int = 128        # group size
    scale_fmt: str = "f32"     # "f32" | "ue8m0"
    layout: str = "row"        # activation-scale layout: "row" | "col"
    silu: bool = False
    masked: bool = False
    mx: bool = False
    outlier_p: float = 0.0


TINY = Workload("tiny", seed=0, M=64, K=512, N=256, scale_fmt="f32", layout="row", outlier_p=0.01)


def dense(M: int = 4096) -> Workload:
    return Workload(f"dense_m{M}", seed=1, M=M, K=7168, N=4096, scale_fmt="ue8m0", layout="col")


SILU = Workload("silu_down", seed=2, M=8192, K=2048, N=7168, scale_fmt="f32", layout="row", silu=True)
MASKED = Workload("masked_moe", seed=3, M=512, K=7168, N=4096, E=32, scale_fmt="ue8m0", layout="col",
                  masked=True)
MX = Workload("mxfp8", seed=4, M=8192, K=8192, N=8192, mx=True)
# MoE second stage: the masked expert buffer's gate|up halves (intermediate width 2048) go
# through silu_and_mul + quant into the down projection back to the 7168-wide hidden size
MASKED_DOWN = Workload("masked_moe_down", seed=5, M=512, K=2048, N=7168, E=32, scale_fmt="ue8m0",
                       layout="col", masked=True, silu=True)


def quant_input(w: Workload, expert: int | None = None) -> np.ndarray:
    """bf16 bits of the quant input: [M, K] (flat), [M, 2K] (silu: gate | up) or, for the
    masked workload, expert `expert`'s [M, K] slab (each expert is its own stream)."""
    cols = 2 * w.K if w.silu else w.K
    if w.masked:
        assert expert is not None
        return activations_bf16(w.seed, w.M, cols, w.outlier_p, tensor_id=(T_X << 12) | expert)
    return activations_bf16(w.seed, w.M, cols, w.outlier_p)


def weights(w: Workload, expert: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """(e4m3 bytes [N, K], fp32 block scales [ceil(N/128), K/128]) for one (expert) GEMM."""
    tid_w = T_W if expert is None else (T_W << 12) | expert
    tid_s = T_SW if expert is None else (T_SW << 12) | expert
    return (weight_codes(w.seed, w.N, w.K, tensor_id=tid_w),
            block_scales(w.seed, (w.N + 127) // 128, w.K // 128, tensor_id=tid_s))


def mx_operands(w: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(A bytes [M, K], B bytes [N, K], ea [M, K/32], eb [N, K/32]) for the MXFP8 GEMM."""
    a = weight_codes(w.seed, w.M, w.K, tensor_id=T_A)
    b = weight_codes(w.seed, w.N, w.K, tensor_id=T_B)
    ea = e8m0_exponents(w.seed, w.M, w.K // 32, tensor_id=T_EA)
    eb = e8m0_exponents(w.seed, w.N, w.K // 32, tensor_id=T_EB)
    return a, b, ea, eb


def gemm_activation(w: Workload, expert: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """GEMM activation operand shaped like the group quantizer's output for workload w:
    (e4m3 bytes [M, K] of N(0, 100^2) samples, scales [M, K/128] row-major storage). The
    scales are UE8M0 bytes in 118..122 (2^-9 .. 2^-5) or fp32 2^-7 * lognormal(0, 0.3)."""
    tid = T_A if expert is None else (T_A << 12) | expert
    a = weight_codes(w.seed, w.M, w.K, tensor_id=tid, sigma=100.0)
    if w.scale_fmt == "ue8m0":
        s = e8m0_exponents(w.seed, w.M, w.K // 128, lo=-9, hi=-5, tensor_id=tid + 1)
    else:
        s = (2.0 ** -7 * block_scales(w.seed, w.M, w.K // 128, sigma=0.3, tensor_id=tid + 1)).astype(np.float32)
    return a, s

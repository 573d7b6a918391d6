"""Accumulation error of the GEMMs, measured through the library on outputs whose exact value
is zero.

The GEMM tolerance (tests/gemm_check.py) allows an element that misses 2 bf16 ulp of the
fp64 result to be off by at most (eta + gamma(K)) * S, S = sum_k |term_k|, where the exact
result nearly cancels. eta is the error of the gfx950 matrix core's 128-term FP8 dot
product, relative to the block's S, per operand class; gamma(K) = (4 ceil(K/128) + 2) 2^-24
bounds the fp32 accumulation across K blocks. Both are measured here and the bounds that
gemm_check uses are asserted.

Construction: the operands are built so that every exact output is 0, so any non-zero
output is accumulation error, and rounding the output to bf16 hides none of it (relative
precision 2^-9 of the error itself). Positions are paired (k, k'): row m of A holds the same
code at k and k', row n of B opposite codes (sign bit flipped), and the scales of k and k'
are equal.
  - one block (K = 128), pairs inside the block: the matrix core's own error (fold factor
    1.0 exactly).
  - block pairs: whole blocks (j, j') with j' the negation of j. The matrix core's result for
    j' is exactly the negation of j's (its rounding is sign-symmetric), so the block errors
    cancel and what remains is the accumulation across blocks (fp32 fold, or the matrix
    core's own accumulation when the scales go to it): asserted against gamma(K).
  - global pairs over all of K (scales constant along K): every block sums unrelated
    products, so the block errors are independent and add up with the accumulation error:
    the whole error of a real GEMM, asserted against eta + gamma(K).
The oracle confirms Y* = 0 (to its fp64 rounding) and S on sampled outputs; S over all
outputs is a float64 matmul of the magnitudes per K block.

Operand classes (those the parity tests and workloads use):
  act:     activation codes of N(0, 100^2) (group maxima near 448) x weight codes of N(0, 1)
  quant:   the oracle's G=128 UE8M0 quantization of N(0, 1) bf16 rows x N(0, 1) weight codes
  outlier: the same with 1% of the inputs x50 (most groups then hold one outlier)
  silu:    the oracle's G=128 quantization of silu(g) * u, g and u N(0, 1) bf16, x N(0, 1) weights
  wide:    N(0, 1) codes on both sides (the MXFP8 workload; products span ~2^-18 .. 2^4)
  full:    codes drawn uniformly over every finite e4m3 value (products 2^-18 .. 2^17.6)
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gemm_check import ETA, gamma, record

pytestmark = pytest.mark.gpu

KB = 128


def fq():
    import fp8_group_quant_amd
    return fp8_group_quant_amd


def _codes(cls_side: str, seed: int, rows: int, cols: int, tid: int) -> np.ndarray:
    if cls_side == "act":
        return synth.weight_codes(seed, rows, cols, tensor_id=tid, sigma=100.0)
    if cls_side == "w":
        return synth.weight_codes(seed, rows, cols, tensor_id=tid, sigma=1.0)
    if cls_side in ("quant", "outlier", "silu"):
        # quantized rows of 2 cols (G = 128), the first cols codes of each
        width = 2 * cols * (2 if cls_side == "silu" else 1)
        x = synth.activations_bf16(seed, rows, width, outlier_p=0.01 if cls_side == "outlier" else 0.0,
                                   tensor_id=tid)
        q, _ = oracle.group_quant(x, 128, oracle.SCALE_UE8M0, "row", silu=cls_side == "silu")
        return np.ascontiguousarray(q[:, :cols])
    # every finite code (0x7F and 0xFF are NaN)
    g = synth.rng(seed, tid)
    c = g.integers(0, 254, size=(rows, cols)).astype(np.uint8)
    return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)


def _sides(cls: str):
    return {"act": ("act", "w"), "quant": ("quant", "w"), "outlier": ("outlier", "w"), "silu": ("silu", "w"),
            "wide": ("w", "w"), "full": ("full", "full")}[cls]


def _pair_positions(a_half, b_half, seed):
    """[rows, K/2] halves -> [rows, K] operands whose row dot products are exactly 0: the K
    positions are split into random pairs (k, k'), same A code, opposite B codes."""
    h = a_half.shape[1]
    g = np.random.default_rng(seed)
    p = g.permutation(2 * h)
    a = np.empty((a_half.shape[0], 2 * h), np.uint8)
    b = np.empty((b_half.shape[0], 2 * h), np.uint8)
    a[:, p[:h]] = a_half
    a[:, p[h:]] = a_half
    b[:, p[:h]] = b_half
    b[:, p[h:]] = b_half ^ 0x80
    return a, b


def _pair_blocks(a_half, b_half, sa_half, sb_half, seed, sw=1):
    """halves of nkb/2 blocks -> nkb blocks (random pairing, second of each pair negated).
    Scales hold sw columns per 128-wide block (BLOCK128: 1; MX32: 4) and move with it."""
    nh = a_half.shape[1] // KB
    g = np.random.default_rng(seed)
    order = g.permutation(2 * nh)  # block order[i] <- half block i % nh (negated B for i >= nh)
    a = np.empty((a_half.shape[0], 2 * nh * KB), np.uint8)
    b = np.empty((b_half.shape[0], 2 * nh * KB), np.uint8)
    sa = np.empty((sa_half.shape[0], 2 * nh * sw), sa_half.dtype)
    sb = np.empty((sb_half.shape[0], 2 * nh * sw), sb_half.dtype)
    for i in range(2 * nh):
        src, neg, j = i % nh, i >= nh, order[i]
        a[:, j * KB:(j + 1) * KB] = a_half[:, src * KB:(src + 1) * KB]
        bb = b_half[:, src * KB:(src + 1) * KB]
        b[:, j * KB:(j + 1) * KB] = bb ^ 0x80 if neg else bb
        sa[:, j * sw:(j + 1) * sw] = sa_half[:, src * sw:(src + 1) * sw]
        sb[:, j * sw:(j + 1) * sw] = sb_half[:, src * sw:(src + 1) * sw]
    return a, b, sa, sb


def _scale_f64(s, fmt):
    return np.ldexp(1.0, s.astype(np.int64) - 127) if fmt == oracle.SCALE_UE8M0 else s.astype(np.float64)


def _s_all(a, b, sa, sb, sa_fmt, sb_fmt, mx=False):
    """S[m, n] = sum_k |term| over all outputs (float64 matmul of magnitudes per block)."""
    da = np.abs(oracle.e4m3_decode(a))
    db = np.abs(oracle.e4m3_decode(b))
    bs = 32 if mx else KB
    fa, fb = _scale_f64(sa, sa_fmt), _scale_f64(sb, sb_fmt)
    S = np.zeros((a.shape[0], b.shape[0]))
    for j in range(a.shape[1] // bs):
        blk = da[:, j * bs:(j + 1) * bs] @ db[:, j * bs:(j + 1) * bs].T
        if mx:
            S += blk * np.outer(fa[:, j], fb[:, j])
        else:
            col = np.repeat(fb[:, j], KB)[: b.shape[0]]
            S += blk * np.outer(fa[:, j], col)
    return S


def _run_block(a, sa_store, b, sb, sa_layout):
    f = fq()
    M, N = a.shape[0], b.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sa_d = torch.from_numpy(np.ascontiguousarray(sa_store)).cuda()
    if sa_layout == "col":
        sa_d = sa_d.t()
    f.fp8q_gemm_blockscaled(torch.from_numpy(a).cuda(), sa_d, torch.from_numpy(b).cuda(),
                            torch.from_numpy(np.ascontiguousarray(sb)).cuda(), y, f.GEMM_BLOCK128)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _run_mx(a, ea, b, eb):
    f = fq()
    y = torch.empty((a.shape[0], b.shape[0]), dtype=torch.bfloat16, device="cuda")
    f.fp8q_gemm_blockscaled(torch.from_numpy(a).cuda(), torch.from_numpy(ea).cuda(), torch.from_numpy(b).cuda(),
                            torch.from_numpy(eb).cuda(), y, f.GEMM_MX32)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _confirm_exact_zero(a, sa, b, sb, sa_fmt, sb_fmt, S, mx=False):
    g = np.random.default_rng(1)
    ms = g.integers(0, a.shape[0], 64)
    ns = g.integers(0, b.shape[0], 64)
    if mx:
        ys, ss = oracle.gemm_mx32(a, sa, b, sb, at=(ms, ns))
    else:
        ys, ss = oracle.gemm_block128(a, sa, b, sb, sa_fmt, "row", sb_fmt, at=(ms, ns))
    # exactly 0 mathematically; the fp64 oracle's own running sum may round (fp32 scale x
    # code products carry more than 53 bits)
    assert np.all(np.abs(ys) <= 2.0 ** -40 * ss)
    assert np.allclose(ss, S[ms, ns], rtol=1e-12)


def _measure(y, S, cls, path, K):
    r = np.abs(y) / S
    worst = float(r.max())
    stats = {"class": cls, "path": path, "K": K, "outputs": int(r.size), "max_err_over_S": worst,
             "log2_max": float(np.log2(worst)) if worst > 0 else None,
             "p99_99": float(np.quantile(r, 0.9999)), "frac_nonzero": float(np.mean(y != 0))}
    record("accumulation", stats)
    print(json.dumps(stats), flush=True)
    return stats


# One K block: the matrix core's own 128-term sum (fold factor 1.0 exactly)
@pytest.mark.parametrize("cls", ["act", "quant", "outlier", "silu", "wide", "full"])
def test_one_block_error(cls):
    M = N = 2048
    sa_side, sb_side = _sides(cls)
    ah = _codes(sa_side, 80, M, 64, 1)
    bh = _codes(sb_side, 80, N, 64, 2)
    a, b = _pair_positions(ah, bh, 3)
    sa = np.ones((M, 1), np.float32)
    sb = np.ones(((N + 127) // 128, 1), np.float32)
    S = _s_all(a, b, sa, sb, oracle.SCALE_F32, oracle.SCALE_F32)
    _confirm_exact_zero(a, sa, b, sb, oracle.SCALE_F32, oracle.SCALE_F32, S)
    y = _run_block(a, sa, b, sb, "row")
    st = _measure(y, S, cls, "one block, fp32 scales", KB)
    assert st["max_err_over_S"] <= ETA[cls], f"{cls}: {st['max_err_over_S']:.3e} * S > eta {ETA[cls]:.3e} * S"


def _block_operands(cls, path, M, N, K, seed, constant_scales):
    nkb = K // KB
    sa_side, sb_side = _sides(cls)
    ah = _codes(sa_side, seed, M, K // 2, 1)
    bh = _codes(sb_side, seed, N, K // 2, 2)
    cols = 1 if constant_scales else nkb // 2
    if path == "f32-fold":
        sah = (2.0 ** -7 * synth.block_scales(seed, M, cols, sigma=0.3, tensor_id=3)).astype(np.float32)
        sbh = synth.block_scales(seed, N // 128, cols, tensor_id=4)
        fmts = (oracle.SCALE_F32, oracle.SCALE_F32)
    else:
        sah = synth.e8m0_exponents(seed, M, cols, lo=-9, hi=-5, tensor_id=3)
        if path == "e8-act-fold":
            sbh, fmts = synth.block_scales(seed, N // 128, cols, tensor_id=4), (oracle.SCALE_UE8M0, oracle.SCALE_F32)
        else:
            sbh = synth.e8m0_exponents(seed, N // 128, cols, lo=-4, hi=4, tensor_id=4)
            fmts = (oracle.SCALE_UE8M0, oracle.SCALE_UE8M0)
    if constant_scales:  # every block of a row (weight block) has the same scale
        a, b = _pair_positions(ah, bh, seed + 1)
        sa, sb = np.repeat(sah, nkb, axis=1), np.repeat(sbh, nkb, axis=1)
    else:
        a, b, sa, sb = _pair_blocks(ah, bh, sah, sbh, seed + 1)
    return a, b, sa, sb, fmts


def _run_paths(a, b, sa, sb, path):
    if path == "f32-fold":
        return _run_block(a, sa, b, sb, "row")
    return _run_block(a, np.ascontiguousarray(sa.T), b, sb, "col")


# Block pairs: the block errors cancel, the accumulation across blocks remains -- fp32 fold
# (fp32 scales), UE8M0 activation scales applied by the matrix core with the fp32
# weight-block fold, and UE8M0 on both sides (no fold: the matrix core accumulates across K)
@pytest.mark.parametrize("cls", ["act", "wide"])
@pytest.mark.parametrize("path", ["f32-fold", "e8-act-fold", "e8-both-nofold"])
@pytest.mark.parametrize("K", [2048, 7168])
def test_accumulation_across_blocks(cls, path, K):
    a, b, sa, sb, fmts = _block_operands(cls, path, 512, 768, K, 81, constant_scales=False)
    S = _s_all(a, b, sa, sb, *fmts)
    _confirm_exact_zero(a, sa, b, sb, *fmts, S)
    st = _measure(_run_paths(a, b, sa, sb, path), S, cls, path + ", block pairs", K)
    assert st["max_err_over_S"] <= gamma(K), f"{st['max_err_over_S']:.3e} * S > gamma {gamma(K):.3e} * S"


# Global pairs: the whole error of a GEMM (independent block errors plus the accumulation)
@pytest.mark.parametrize("cls", ["act", "quant", "outlier", "silu", "wide"])
@pytest.mark.parametrize("path", ["f32-fold", "e8-act-fold", "e8-both-nofold"])
@pytest.mark.parametrize("K", [512, 2048, 7168])
def test_whole_gemm_error(cls, path, K):
    a, b, sa, sb, fmts = _block_operands(cls, path, 512, 768, K, 83, constant_scales=True)
    S = _s_all(a, b, sa, sb, *fmts)
    _confirm_exact_zero(a, sa, b, sb, *fmts, S)
    st = _measure(_run_paths(a, b, sa, sb, path), S, cls, path + ", global pairs", K)
    bound = ETA[cls] + gamma(K)
    assert st["max_err_over_S"] <= bound, f"{st['max_err_over_S']:.3e} * S > {bound:.3e} * S"


# MXFP8: E8M0 per 1x32 block on both operands, accumulation in the matrix core across K;
# block pairs (each 128-wide block carries its four scale bytes) and global pairs (scales
# constant along K)
@pytest.mark.parametrize("cls", ["wide", "act"])
@pytest.mark.parametrize("pairs", ["block", "global"])
def test_mx_error(cls, pairs):
    M, N, K = 512, 512, 8192
    sa_side, sb_side = _sides(cls)
    ah = _codes(sa_side, 82, M, K // 2, 1)
    bh = _codes(sb_side, 82, N, K // 2, 2)
    if pairs == "block":
        eah = synth.e8m0_exponents(82, M, K // 64, tensor_id=3)
        ebh = synth.e8m0_exponents(82, N, K // 64, tensor_id=4)
        a, b, ea, eb = _pair_blocks(ah, bh, eah, ebh, 6, sw=4)
    else:
        a, b = _pair_positions(ah, bh, 7)
        ea = np.repeat(synth.e8m0_exponents(82, M, 1, tensor_id=3), K // 32, axis=1)
        eb = np.repeat(synth.e8m0_exponents(82, N, 1, tensor_id=4), K // 32, axis=1)
    S = _s_all(a, b, ea, eb, oracle.SCALE_UE8M0, oracle.SCALE_UE8M0, mx=True)
    _confirm_exact_zero(a, ea, b, eb, None, None, S, mx=True)
    st = _measure(_run_mx(a, ea, b, eb), S, cls, "mx32, " + pairs + " pairs", K)
    bound = gamma(K) if pairs == "block" else ETA[cls] + gamma(K)
    assert st["max_err_over_S"] <= bound, f"{st['max_err_over_S']:.3e} * S > {bound:.3e} * S"

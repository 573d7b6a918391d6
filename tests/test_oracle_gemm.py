"""Pins of the oracle's block-scaled and MXFP8 GEMM: exact rational arithmetic (Python
Fractions over the integer structure of e4m3 values), torch float64 dequantize-then-matmul
(a library routine), one-hot operands with closed-form results, and scale-index checks
chosen so a swapped operand or a wrong block index fails."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _codes(seed, rows, cols, tid):
    return synth.weight_codes(seed, rows, cols, tensor_id=tid)


def _torch_dequant(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)


def _exact_value(code: int) -> Fraction:
    """e4m3 value as a Fraction, from the format definition (integer * 2^-9)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    mag = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -mag if s else mag


# ----------------------------------------------------------------------------- BLOCK128
def _block_case(M, N, K, seed, sa_fmt):
    a = _codes(seed, M, K, 1)
    b = _codes(seed, N, K, 2)
    kb, nb = K // 128, (N + 127) // 128
    if sa_fmt == oracle.SCALE_UE8M0:
        sa = synth.e8m0_exponents(seed, M, kb, -6, 6, tensor_id=3)
    else:
        sa = synth.block_scales(seed, M, kb, tensor_id=3)
    sb = synth.block_scales(seed, nb, kb, tensor_id=4)
    return a, b, sa, sb


def test_block128_exact_rational_tiny():
    M, N, K = 3, 130, 256   # two N blocks (the second ragged), two K blocks
    a, b, sa, sb = _block_case(M, N, K, 5, oracle.SCALE_F32)
    y, s = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32)
    for m in range(M):
        for n in range(0, N, 7):
            exact = Fraction(0)
            for kb in range(K // 128):
                part = sum(_exact_value(int(a[m, k])) * _exact_value(int(b[n, k]))
                           for k in range(kb * 128, kb * 128 + 128))
                exact += Fraction(float(sa[m, kb])) * Fraction(float(sb[n // 128, kb])) * part
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(s[m, n]) * Fraction(1, 2 ** 45), (m, n)


@pytest.mark.parametrize("sa_fmt,sa_layout", [(oracle.SCALE_F32, "row"), (oracle.SCALE_UE8M0, "col")])
def test_block128_matches_torch_float64_dequant_matmul(sa_fmt, sa_layout):
    M, N, K = 37, 300, 640
    a, b, sa, sb = _block_case(M, N, K, 6, sa_fmt)
    sa_arg = sa if sa_layout == "row" else np.ascontiguousarray(sa.T)
    y, s = oracle.gemm_block128(a, sa_arg, b, sb, sa_fmt, sa_layout)
    if sa_fmt == oracle.SCALE_UE8M0:
        sa_val = torch.from_numpy(np.ldexp(1.0, sa.astype(np.int64) - 127))
    else:
        sa_val = torch.from_numpy(sa.astype(np.float64))
    sb_val = torch.from_numpy(sb.astype(np.float64))
    A = _torch_dequant(a) * sa_val.repeat_interleave(128, dim=1)
    B = _torch_dequant(b) * sb_val.repeat_interleave(128, dim=0)[:N].repeat_interleave(128, dim=1)
    ref = (A @ B.T).numpy()
    assert np.all(np.abs(y - ref) <= 1e-12 * s)
    assert np.all(s >= np.abs(y))


def test_block128_one_hot_weights():
    # each weight row has one non-zero code: Y = dec(a[m, k_n]) * sa * dec(w) * sb exactly
    M, N, K = 5, 256, 384
    a, _, sa, sb = _block_case(M, N, K, 7, oracle.SCALE_F32)
    b = np.zeros((N, K), dtype=np.uint8)
    ks = (np.arange(N) * 37) % K
    b[np.arange(N), ks] = 0x40  # 2.0
    y, _ = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32)
    da = oracle.e4m3_decode(a)
    for n in range(N):
        k = ks[n]
        want = da[:, k] * sa[:, k // 128].astype(np.float64) * 2.0 * float(sb[n // 128, k // 128])
        assert np.array_equal(y[:, n], want)


def test_block128_scale_indices_are_not_transposed():
    # a scale change in block (nb=1, kb=0) of b must only move columns 128..255
    M, N, K = 4, 256, 256
    a, b, sa, sb = _block_case(M, N, K, 8, oracle.SCALE_F32)
    y0, _ = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32)
    sb2 = sb.copy()
    sb2[1, 0] *= 2
    y1, _ = oracle.gemm_block128(a, sa, b, sb2, oracle.SCALE_F32)
    assert np.array_equal(y0[:, :128], y1[:, :128])
    assert not np.array_equal(y0[:, 128:], y1[:, 128:])
    # a change in sa for row 2, kb=1 moves row 2 only
    sa2 = sa.copy()
    sa2[2, 1] *= 2
    y2, _ = oracle.gemm_block128(a, sa2, b, sb, oracle.SCALE_F32)
    assert np.array_equal(np.delete(y0, 2, 0), np.delete(y2, 2, 0))
    assert not np.array_equal(y0[2], y2[2])


def test_block128_sampled_elements_equal_full():
    M, N, K = 9, 200, 256
    a, b, sa, sb = _block_case(M, N, K, 9, oracle.SCALE_F32)
    y, s = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32)
    ms = np.array([0, 8, 4, 3]); ns = np.array([199, 0, 128, 77])
    ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32, at=(ms, ns))
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(ss, s[ms, ns])


# ----------------------------------------------------------------------------- MX32
def test_mx32_exact_rational_tiny():
    M, N, K = 2, 5, 128
    a = _codes(10, M, K, 1); b = _codes(10, N, K, 2)
    ea = synth.e8m0_exponents(10, M, K // 32, tensor_id=3)
    eb = synth.e8m0_exponents(10, N, K // 32, tensor_id=4)
    y, s = oracle.gemm_mx32(a, ea, b, eb)
    for m in range(M):
        for n in range(N):
            exact = sum(_exact_value(int(a[m, k])) * Fraction(2) ** (int(ea[m, k // 32]) - 127)
                        * _exact_value(int(b[n, k])) * Fraction(2) ** (int(eb[n, k // 32]) - 127)
                        for k in range(K))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(s[m, n]) * Fraction(1, 2 ** 45)


def test_mx32_matches_torch_float64():
    M, N, K = 33, 70, 512
    a = _codes(11, M, K, 1); b = _codes(11, N, K, 2)
    ea = synth.e8m0_exponents(11, M, K // 32, tensor_id=3)
    eb = synth.e8m0_exponents(11, N, K // 32, tensor_id=4)
    y, s = oracle.gemm_mx32(a, ea, b, eb)
    A = _torch_dequant(a) * torch.from_numpy(np.ldexp(1.0, ea.astype(np.int64) - 127)).repeat_interleave(32, 1)
    B = _torch_dequant(b) * torch.from_numpy(np.ldexp(1.0, eb.astype(np.int64) - 127)).repeat_interleave(32, 1)
    ref = (A @ B.T).numpy()
    assert np.all(np.abs(y - ref) <= 1e-12 * s)


def test_mx32_scale_block_is_32_wide():
    M, N, K = 1, 1, 64
    a = np.full((M, K), 0x38, dtype=np.uint8)  # 1.0
    b = np.full((N, K), 0x38, dtype=np.uint8)
    ea = np.array([[127, 128]], dtype=np.uint8)  # 1, 2
    eb = np.array([[129, 127]], dtype=np.uint8)  # 4, 1
    y, _ = oracle.gemm_mx32(a, ea, b, eb)
    assert y[0, 0] == 32 * 1 * 4 + 32 * 2 * 1


# ------------------------------------------------------------- segments / contiguous
def _seg_operands(T=20, K=256, N=40, W=3, seed=5):
    g = np.random.default_rng(seed)
    a = oracle.e4m3_encode(g.normal(0, 60, (T, K)).astype(np.float32))
    sa = (2.0 ** g.integers(-8, -5, (T, K // 128))).astype(np.float32)
    b = oracle.e4m3_encode(g.normal(0, 1, (W, N, K)).astype(np.float32))
    sb = np.exp(g.normal(0, 0.5, (W, (N + 127) // 128, K // 128))).astype(np.float32)
    return a, sa, b, sb


def test_gemm_segments_rows_and_weights():
    """Each computed row equals the whole-matrix product against its segment's weight; clamped
    ends, empty segments, out-of-range weights and gaps leave rows out."""
    a, sa, b, sb = _seg_operands()
    full = [oracle.gemm_block128(a, sa, b[w], sb[w], oracle.SCALE_F32)[0] for w in range(3)]
    indptr = [-3, 4, 4, 9, 12, 30]          # [0,4) [4,4) [4,9) [9,12) [12,20)
    weight = [2, 0, 1, 7, 0]                 # segment 3 uses a weight outside [0, 3)
    Y, _ = oracle.gemm_segments(a, sa, oracle.SCALE_F32, b, sb, indptr, weight)
    want_w = {**{t: 2 for t in range(0, 4)}, **{t: 1 for t in range(4, 9)}, **{t: 0 for t in range(12, 20)}}
    for t in range(20):
        if t in want_w:
            assert np.array_equal(Y[t], full[want_w[t]][t]), t
        else:
            assert np.all(np.isnan(Y[t])), t
    # default weights (segment s uses weight s) and column-major scale storage give the same rows
    Y2, _ = oracle.gemm_segments(a, np.ascontiguousarray(sa.T), oracle.SCALE_F32, b, sb, [0, 5, 20], None, "col")
    assert np.array_equal(Y2[:5], full[0][:5]) and np.array_equal(Y2[5:], full[1][5:])


def test_gemm_contiguous_block_rule():
    """Blocks take the weight of their first row; rows with another index (padding -1, or a
    stray index) are left out; a block starting with -1 or an index outside [0, W) is skipped."""
    a, sa, b, sb = _seg_operands(T=24)
    full = [oracle.gemm_block128(a, sa, b[w], sb[w], oracle.SCALE_F32)[0] for w in range(3)]
    mi = np.array([1] * 6 + [-1] * 2 + [0, 0, 2, 0, -1, -1, -1, -1] + [-1] * 4 + [5] * 4, dtype=np.int32)
    Y, _ = oracle.gemm_contiguous(a, sa, oracle.SCALE_F32, b, sb, mi, block=8)
    for t in range(24):
        if t < 6:
            assert np.array_equal(Y[t], full[1][t]), t
        elif t in (8, 9, 11):
            assert np.array_equal(Y[t], full[0][t]), t
        else:
            assert np.all(np.isnan(Y[t])), t

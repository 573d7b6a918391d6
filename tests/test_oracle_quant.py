"""Pins of the oracle's group quantization and fused silu_and_mul: hand-derived golden
group, the dequantization error bound, the exp accuracy against math.exp, and the
layout / dispatch invariants the C ABI promises."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(vals) -> np.ndarray:
    return torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _golden_group():
    xs, codes = [], []
    with open(os.path.join(GOLDEN, "quant_group32.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                p = line.split()
                xs.append(float(eval(p[0])))
                codes.append(int(p[1], 16))
    n0 = 32 - len(xs)
    return xs + [0.0] * n0, codes + [0] * n0


# ----------------------------------------------------------------------------- golden
@pytest.mark.parametrize("fmt", [oracle.SCALE_UE8M0, oracle.SCALE_F32])
def test_golden_group(fmt):
    xs, codes = _golden_group()
    x = _bf16(xs)
    assert np.array_equal(_bf16_to_f32(x).astype(np.float64), np.array(xs)), "inputs must be bf16-exact"
    q, s = oracle.group_quant(x[None, :], 32, fmt, "row")
    assert q[0].tolist() == codes
    if fmt == oracle.SCALE_UE8M0:
        assert s[0, 0] == 120
    else:
        assert s[0, 0] == np.float32(2.0 ** -7)


def test_all_zero_group_gives_zero_codes_and_eps_scale():
    x = np.zeros((2, 128), dtype=np.uint16)
    x[1, :] = 0x8000  # -0.0
    q, s = oracle.group_quant(x, 128, oracle.SCALE_UE8M0, "row")
    assert q[0].tolist() == [0] * 128 and q[1].tolist() == [0x80] * 128
    assert s[:, 0].tolist() == [85, 85]
    q, s = oracle.group_quant(x, 128, oracle.SCALE_F32, "row")
    assert s[0, 0] == np.float32(1e-10) / np.float32(448)


# ----------------------------------------------------------------------------- error bound
def _ulp_e4m3(v: np.ndarray) -> np.ndarray:
    """spacing of e4m3 values around |v| (2^-9 in the subnormal range)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.ldexp(1.0, (e - 3).astype(np.int64))


def _dequant_check(fmt, x_bits, G, slack_rel):
    xf = _bf16_to_f32(x_bits).astype(np.float64)
    q, s = oracle.group_quant(x_bits, G, fmt, "row")
    dq = oracle.e4m3_decode(q)
    M, K = xf.shape
    if fmt == oracle.SCALE_UE8M0:
        sc = np.ldexp(1.0, s.astype(np.int64) - 127)
    else:
        sc = s.astype(np.float64)
    scale = np.repeat(sc, G, axis=1)
    err = np.abs(dq * scale - xf)
    # |x*inv| <= 448 (plus slack) and the rounding error is at most half an e4m3 step
    bound = 0.5 * _ulp_e4m3(xf / scale) * scale + slack_rel * np.abs(xf)
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))
    return q, s


def test_dequant_error_within_half_ulp_ue8m0():
    x = synth.activations_bf16(11, 64, 1024, outlier_p=0.01)
    _, s = _dequant_check(oracle.SCALE_UE8M0, x, 128, 0.0)
    # each scale is the smallest power of two >= amax/448
    xf = _bf16_to_f32(x).astype(np.float64)
    amax = np.maximum(np.abs(xf).reshape(64, 8, 128).max(-1), np.float32(1e-10))
    sc = np.ldexp(1.0, s.astype(np.int64) - 127)
    assert np.all(sc * 448 >= amax) and np.all(sc * 224 < amax)


def test_dequant_error_within_half_ulp_fp32_scale():
    # fp32 scales: s = fl(amax/448), inv = fl(1/s); x*inv carries up to ~2 fp32 roundings
    x = synth.activations_bf16(12, 64, 1024, outlier_p=0.01)
    _dequant_check(oracle.SCALE_F32, x, 128, 2.0 ** -22)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_group_sizes(G):
    x = synth.activations_bf16(13, 8, 512)
    _dequant_check(oracle.SCALE_UE8M0, x, G, 0.0)
    _dequant_check(oracle.SCALE_F32, x, G, 2.0 ** -22)


def test_largest_element_of_each_group_lands_in_top_binade_ue8m0():
    x = synth.activations_bf16(14, 16, 1024)
    q, _ = oracle.group_quant(x, 128, oracle.SCALE_UE8M0, "row")
    mx = np.abs(oracle.e4m3_decode(q)).reshape(16, 8, 128).max(-1)
    assert np.all(mx > 224 * (1 - 2.0 ** -4)) and np.all(mx <= 448)


# ----------------------------------------------------------------------------- layouts
def test_row_and_column_layouts_hold_the_same_scales():
    x = synth.activations_bf16(15, 24, 896)
    for fmt in (oracle.SCALE_UE8M0, oracle.SCALE_F32):
        qr, sr = oracle.group_quant(x, 128, fmt, "row")
        qc, sc = oracle.group_quant(x, 128, fmt, "col")
        assert np.array_equal(qr, qc)
        assert np.array_equal(sr, sc.T)


def test_per_token_group_equals_whole_row():
    # group = the whole row (per-token quantization, as in tf_per_token_quant_fp8)
    x = synth.activations_bf16(16, 8, 128)
    q, s = oracle.group_quant(x, 128, oracle.SCALE_F32, "row")
    xf = _bf16_to_f32(x)
    amax = np.maximum(np.abs(xf).max(1), np.float32(1e-10)).astype(np.float32)
    assert np.array_equal(s[:, 0], (amax / np.float32(448)).astype(np.float32))


@pytest.mark.parametrize("K", [1024, 7168])
def test_per_token_scale_is_the_row_maximum(K):
    """G = K: one scale per row, from the maximum over the whole row (numpy's max, not
    the oracle's loop); the dequant bound holds against that one scale."""
    x = synth.activations_bf16(30, 6, K, outlier_p=0.002)
    xf = _bf16_to_f32(x)
    amax = np.abs(xf).max(1)
    qu, su = oracle.group_quant(x, K, oracle.SCALE_UE8M0, "row")
    assert su.shape == (6, 1)
    assert np.array_equal(su[:, 0], oracle.ue8m0_byte(amax))
    _dequant_check(oracle.SCALE_UE8M0, x, K, 0.0)
    qf, sf = oracle.group_quant(x, K, oracle.SCALE_F32, "col")
    assert sf.shape == (1, 6)
    assert np.array_equal(sf[0], amax / np.float32(448))
    _dequant_check(oracle.SCALE_F32, x, K, 2.0 ** -22)


def test_per_token_equals_group_quant_when_every_group_holds_the_row_max():
    """Rows whose every 128-group contains the row's largest magnitude have the same
    scale in every group, so per-token and G = 128 quantization agree code for code."""
    M, K = 8, 1024
    x = synth.activations_bf16(31, M, K)
    xf = _bf16_to_f32(x).copy()
    big = np.float32(6.5)  # larger than any N(0,1) draw here, bf16-exact
    assert np.abs(xf).max() < big
    for g in range(K // 128):
        xf[:, g * 128 + (g * 37) % 128] = np.where(np.arange(M) % 2 == 0, big, -big)
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)
    for fmt in (oracle.SCALE_UE8M0, oracle.SCALE_F32):
        qt, st = oracle.group_quant(xb, K, fmt, "row")
        qg, sg = oracle.group_quant(xb, 128, fmt, "row")
        assert np.array_equal(qt, qg)
        assert np.all(sg == st)


# ----------------------------------------------------------------------------- int8 output
def test_int8_encode_ties_to_even():
    v = np.float32([2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, -1.5, 126.5, -126.5, 127, -127, 0.49999997, 2.5000002])
    assert oracle.int8_encode(v).tolist() == [2, 4, -2, -4, 0, 0, 2, -2, 126, -126, 127, -127, 0, 3]


def test_int8_encode_matches_numpy_rint():
    v = np.linspace(-127.0, 127.0, 2_000_001, dtype=np.float64).astype(np.float32)
    halves = (np.arange(-254, 255) / 2.0).astype(np.float32)
    v = np.concatenate([v, halves, np.nextafter(halves, np.float32(0)), np.nextafter(halves, np.float32(200))])
    v = np.clip(v, -127, 127)
    assert np.array_equal(oracle.int8_encode(v), np.rint(v).astype(np.int8))


def test_int8_golden_groups():
    """Hand-derived: a group whose amax is 127 has s = 1 and multiplier 1, so each code is
    the input rounded to the nearest integer (ties to even); amax 254 gives s = 2 and
    multiplier 1/2."""
    a = [127.0, -127.0, 2.5, 3.5, -2.5, 0.5, 1.5, 99.5, -0.25, 64.0]
    b = [254.0, 5.0, 7.0, -254.0, -3.0, 0.75, 100.0, 1.0, -1.0, 2.0]
    ca = [127, -127, 2, 4, -2, 0, 2, 100, 0, 64]
    cb = [127, 2, 4, -127, -2, 0, 50, 0, 0, 1]
    pad = [0.0] * (32 - len(a))
    x = _bf16([a + pad, b + pad])
    assert np.array_equal(_bf16_to_f32(x).astype(np.float64), np.array([a + pad, b + pad]))
    q, s = oracle.group_quant(x, 32, oracle.SCALE_F32, "row", out_int8=True)
    assert q.dtype == np.int8
    assert q[0, :10].tolist() == ca and q[1, :10].tolist() == cb
    assert np.all(q[:, 10:] == 0)
    assert s[:, 0].tolist() == [1.0, 2.0]


@pytest.mark.parametrize("G", [32, 128, 1024])
def test_int8_dequant_error_within_half_step(G):
    """|q * s - x| <= s / 2 (plus a few fp32 roundings of x * (1/s)), codes within
    [-127, 127], and each group's largest magnitude maps to +-127."""
    M, K = 16, 1024
    x = synth.activations_bf16(32, M, K, outlier_p=0.01)
    xf = _bf16_to_f32(x).astype(np.float64)
    q, s = oracle.group_quant(x, G, oracle.SCALE_F32, "row", out_int8=True)
    sc = np.repeat(s.astype(np.float64), G, axis=1)
    err = np.abs(q.astype(np.float64) * sc - xf)
    assert np.all(err <= 0.5 * sc * (1 + 2.0 ** -20) + 2.0 ** -22 * np.abs(xf))
    assert q.min() >= -127 and q.max() <= 127
    amax = np.abs(xf).reshape(M, K // G, G).max(-1)
    assert np.array_equal(np.abs(q.astype(np.int64)).reshape(M, K // G, G).max(-1), np.full(amax.shape, 127))
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(127)).astype(np.float32))


def test_int8_all_zero_row_and_ue8m0_rejected():
    x = np.zeros((1, 128), dtype=np.uint16)
    q, s = oracle.group_quant(x, 128, oracle.SCALE_F32, "row", out_int8=True)
    assert np.all(q == 0) and s[0, 0] == np.float32(1e-10) / np.float32(127)
    with pytest.raises(ValueError):
        oracle.group_quant(x, 128, oracle.SCALE_UE8M0, "row", out_int8=True)


def test_int8_silu_equals_int8_of_silu_values():
    M, K = 4, 256
    h = synth.activations_bf16(33, M, 2 * K)
    q, s = oracle.group_quant(h, 64, oracle.SCALE_F32, "row", silu=True, out_int8=True)
    hf = _bf16_to_f32(h)
    y = oracle.silu_mul(hf[:, :K], hf[:, K:])
    q2, s2 = oracle.group_quant(y, 64, oracle.SCALE_F32, "row", in_dtype=oracle.F32, out_int8=True)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_masked_rows_untouched_and_flat_rows_match():
    E, M, K = 4, 16, 256
    x = np.stack([synth.activations_bf16(17, M, K, tensor_id=100 + e) for e in range(E)])
    mm = np.array([0, 1, 16, 7], dtype=np.int32)
    q, s = oracle.group_quant(x, 128, oracle.SCALE_UE8M0, "col", masked_m=mm, fill=0xA5)
    for e in range(E):
        qf, sf = oracle.group_quant(x[e], 128, oracle.SCALE_UE8M0, "col")
        r = mm[e]
        assert np.array_equal(q[e, :r], qf[:r])
        assert np.array_equal(s[e, :, :r], sf[:, :r])
        assert np.all(q[e, r:] == 0xA5) and np.all(s[e, :, r:] == 0xA5)


def test_masked_m_is_clamped():
    E, M, K = 2, 8, 128
    x = np.stack([synth.activations_bf16(18, M, K, tensor_id=200 + e) for e in range(E)])
    q, _ = oracle.group_quant(x, 128, oracle.SCALE_UE8M0, "row",
                              masked_m=np.array([-3, 99], dtype=np.int32), fill=0xA5)
    assert np.all(q[0] == 0xA5)
    qf, _ = oracle.group_quant(x[1], 128, oracle.SCALE_UE8M0, "row")
    assert np.array_equal(q[1], qf)


def test_input_dtypes_agree_on_common_values():
    x = synth.activations_bf16(19, 4, 256)
    xf = _bf16_to_f32(x)
    x16 = xf.astype(np.float16).view(np.uint16)
    qb, sb = oracle.group_quant(x, 128, oracle.SCALE_F32, "row", in_dtype=oracle.BF16)
    qf, sf = oracle.group_quant(xf, 128, oracle.SCALE_F32, "row", in_dtype=oracle.F32)
    assert np.array_equal(qb, qf) and np.array_equal(sb, sf)
    # fp16 holds every bf16 value of N(0,1) samples exactly when its exponent is in range
    exact16 = np.all(x16.view(np.float16).astype(np.float32) == xf)
    if exact16:
        qh, sh = oracle.group_quant(x16, 128, oracle.SCALE_F32, "row", in_dtype=oracle.F16)
        assert np.array_equal(qb, qh) and np.array_equal(sb, sh)


def test_f16_decode_matches_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16).astype(np.float32)
    fin = np.isfinite(f)
    # route each half value through the quantizer's loader: a group whose amax is 448
    # returns the values themselves (multiplier 1) — compare through the F16 path
    vals = f[fin & (np.abs(f) <= 448)]
    bits = vals.astype(np.float16).view(np.uint16)
    G = 32
    n = (bits.size // (G - 1)) * (G - 1)
    body = bits[:n].reshape(-1, G - 1)
    pad = np.full((body.shape[0], 1), np.float16(448).view(np.uint16), dtype=np.uint16)
    xg = np.concatenate([pad, body], axis=1)
    q, s = oracle.group_quant(xg, G, oracle.SCALE_UE8M0, "row", in_dtype=oracle.F16)
    assert np.all(s == 127)
    ref = torch.from_numpy(xg.view(np.float16).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


# ----------------------------------------------------------------------------- exp / silu
def test_exp_spec_accuracy_against_math_exp():
    t = np.linspace(-87.0, 88.0, 400001, dtype=np.float64).astype(np.float32)
    t = np.concatenate([t, np.float32([0.0, -0.0, 1e-8, -1e-8, 0.5, -0.5, 1.0, -1.0])])
    got = oracle.exp_spec(t).astype(np.float64)
    ref = np.array([math.exp(float(v)) for v in t])
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err_ulp = np.abs(got - ref) / ulp
    assert np.max(err_ulp) <= 2.0, float(np.max(err_ulp))
    assert oracle.exp_spec(np.float32([0.0]))[0] == 1.0


def test_exp_spec_clamps_outside_range():
    e = oracle.exp_spec(np.float32([-1000.0, -87.0, 88.0, 1000.0]))
    assert e[0] == e[1] and e[2] == e[3] and np.isfinite(e[3])


def test_silu_mul_special_values_and_accuracy():
    g = np.float32([0.0, 30.0, -30.0, 1.0, -1.0, 2.5])
    u = np.float32([5.0, 2.0, 2.0, 1.0, 1.0, -3.0])
    y = oracle.silu_mul(g, u)
    assert y[0] == 0.0
    assert y[1] == np.float32(60.0)  # exp(-30) < 2^-24: 1 + e == 1 in fp32
    ref = np.array([gg / (1 + math.exp(-gg)) * uu for gg, uu in zip(g.astype(np.float64), u.astype(np.float64))])
    assert np.allclose(y.astype(np.float64), ref, rtol=4e-7, atol=1e-12)
    # sweep: relative error of silu(g)*u within a few fp32 ulps of the fp64 value
    gs = np.linspace(-20, 20, 200001).astype(np.float32)
    us = np.ones_like(gs)
    ys = oracle.silu_mul(gs, us).astype(np.float64)
    gd = gs.astype(np.float64)
    refs = gd / (1 + np.exp(-gd))
    rel = np.abs(ys - refs) / np.maximum(np.abs(refs), 1e-30)
    assert np.max(rel[np.abs(refs) > 1e-30]) < 8 * 2.0 ** -24


def test_fused_silu_quant_equals_quant_of_silu_values():
    E, M, K = 1, 8, 256
    h = synth.activations_bf16(20, M, 2 * K)
    q, s = oracle.group_quant(h, 128, oracle.SCALE_F32, "row", silu=True)
    hf = _bf16_to_f32(h)
    y = oracle.silu_mul(hf[:, :K], hf[:, K:])
    q2, s2 = oracle.group_quant(y, 128, oracle.SCALE_F32, "row", in_dtype=oracle.F32)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ----------------------------------------------------------------- packed UE8M0 layout
def test_pack_ue8m0_known_words():
    """Group g of a row is byte g % 4 of word g / 4, least significant byte first."""
    b = np.array([[1, 2, 3, 4, 5, 6, 7, 0x88], [0x7F, 0x80, 0, 0xFF, 9, 9, 9, 9]], dtype=np.uint8)
    w = oracle.pack_ue8m0(b).astype(np.int64) & 0xFFFFFFFF
    assert w.tolist() == [[0x04030201, 0x88070605], [0xFF00807F, 0x09090909]]


def test_packed_format_constant_matches_header():
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "fp8q.h")).read()
    assert int(re.search(r"#define FP8Q_SCALE_UE8M0_PACKED (\d+)", hdr).group(1)) == oracle.SCALE_UE8M0_PACKED


def test_pack_ue8m0_round_trip_and_shape():
    g = np.random.default_rng(3)
    b = g.integers(0, 256, size=(3, 5, 16), dtype=np.uint8)
    w = oracle.pack_ue8m0(b)
    assert w.shape == (3, 5, 4) and w.dtype == np.int32
    assert np.array_equal(oracle.unpack_ue8m0(w), b)
    with pytest.raises(ValueError):
        oracle.pack_ue8m0(b[..., :6])


# ----------------------------------------------------------------- thread-count independence
def test_results_do_not_depend_on_the_thread_count():
    """The oracle's OpenMP loops give each row (quant) and each output (GEMM) to one thread,
    so one thread and all threads must agree bit for bit, masked and flat."""
    x = synth.activations_bf16(30, 3 * 40, 2 * 384, outlier_p=0.01).reshape(3, 40, 768)
    mm = np.array([40, 0, 17], dtype=np.int32)
    a = synth.weight_codes(31, 37, 512, tensor_id=1, sigma=100.0)
    b = synth.weight_codes(31, 50, 512, tensor_id=2)
    sa = synth.block_scales(31, 37, 4, tensor_id=3)
    sb = synth.block_scales(31, 1, 4, tensor_id=4)
    outs = []
    for n in (1, max(2, oracle.max_threads())):
        with oracle.threads(n):
            q, s = oracle.group_quant(x, 128, oracle.SCALE_UE8M0, "col", silu=True, masked_m=mm, fill=0x5A)
            qf, sf = oracle.group_quant(x[0], 64, oracle.SCALE_F32, "row")
            y, S = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32)
            ys, Ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32, at=(np.arange(30) % 37, np.arange(30)))
        outs.append((q, s, qf, sf, y, S, ys, Ss))
    for u, v in zip(*outs):
        assert np.array_equal(u, v)

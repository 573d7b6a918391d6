"""GPU parity of the group-quant calls against the CPU oracle: every FP8 byte and every
scale byte must be identical (bit-exact), untouched rows must keep their sentinel bytes,
and the result must not depend on expected_m. Calls go through the C ABI via the binding.

Sizes: full oracle comparison at sizes that span several chunks and a ragged tail, and at
the named workloads' full sizes (every row: dense 4096 x 7168, the fused silu 8192 x 2048,
all 7833 valid rows of the 32 masked experts, with the oracle's rows spread over the host
cores), plus properties that hold everywhere.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

FILL = 0xA5


def fq():
    import fp8_group_quant_amd
    return fp8_group_quant_amd


def _to_dev(x: np.ndarray, in_dtype: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if in_dtype == oracle.BF16:
        return t.view(torch.bfloat16)
    if in_dtype == oracle.F16:
        return t.view(torch.float16)
    return t


def _gpu_quant(x_np, in_dtype, G, fmt, layout, silu=False, masked_m=None, expected_m=0, stream=None,
               int8=False):
    """Runs the GPU quant on x ([M, W] or [E, M, W]); returns (q, scale storage) as numpy in
    the oracle's storage layout ([.., M, ng] row-major or [.., ng, M] column-major). q is
    returned as bytes (int8 codes as their two's-complement bytes)."""
    f = fq()
    x = _to_dev(x_np, in_dtype)
    x3 = x if x.dim() == 3 else x[None]
    E, M, W = x3.shape
    K = W // 2 if silu else W
    ng = K // G
    q = torch.full((E, M, K), FILL, dtype=torch.uint8, device="cuda")
    qt = q.view(torch.int8) if int8 else q
    width = 4 if fmt == oracle.SCALE_F32 else 1
    shape = (E, M, ng * width) if layout == "row" else (E, ng, M * width)
    s_store = torch.full(shape, FILL, dtype=torch.uint8, device="cuda")
    s_typed = s_store.view(torch.float32) if fmt == oracle.SCALE_F32 else s_store
    s_view = s_typed if layout == "row" else s_typed.transpose(1, 2)
    mm = None if masked_m is None else torch.from_numpy(np.asarray(masked_m, dtype=np.int32)).cuda()
    fn = f.fp8q_group_quant_int8 if int8 else (f.fp8q_silu_mul_group_quant if silu else f.fp8q_group_quant)
    xin, qin, sin = (x3, qt, s_view) if x.dim() == 3 else (x3[0], qt[0], s_view[0])
    fn(xin, qin, sin, G, masked_m=mm, expected_m=expected_m, stream=stream)
    torch.cuda.synchronize()
    qn = q.cpu().numpy()
    sn = s_typed.cpu().numpy()
    if x.dim() == 2:
        return qn[0], sn[0]
    return qn, sn


def _oracle(x_np, in_dtype, G, fmt, layout, silu=False, masked_m=None, rows=None, int8=False):
    q, sc = oracle.group_quant(x_np, G, fmt, layout, in_dtype=in_dtype, silu=silu, masked_m=masked_m,
                               rows=rows, fill=FILL, out_int8=int8)
    return q.view(np.uint8), sc


def _assert_same(a, b, what):
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatching entries, first at {i}: gpu={a[i]!r} oracle={b[i]!r}")


def _full_case(x_np, in_dtype, G, fmt, layout, silu=False, masked_m=None, expected_m=0, int8=False):
    qg, sg = _gpu_quant(x_np, in_dtype, G, fmt, layout, silu, masked_m, expected_m, int8=int8)
    qo, so = _oracle(x_np, in_dtype, G, fmt, layout, silu, masked_m, int8=int8)
    _assert_same(qg, qo, "q")
    _assert_same(sg.view(np.uint8), so.view(np.uint8), "scales")


# ----------------------------------------------------------------------------- small / full
def test_tiny_workload_full():
    w = synth.TINY
    x = synth.quant_input(w)
    _full_case(x, oracle.BF16, w.G, oracle.SCALE_F32, "row")


@pytest.mark.parametrize("M", [1, 16, 128])
def test_dense_small_m_full(M):
    w = synth.dense(M)
    _full_case(synth.quant_input(w), oracle.BF16, w.G, oracle.SCALE_UE8M0, "col")


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_group_sizes_formats_layouts(G, fmt, layout):
    # 37 rows, 1536 columns = 3 chunks of 512; outliers make groups differ widely
    x = synth.activations_bf16(21, 37, 1536, outlier_p=0.02)
    _full_case(x, oracle.BF16, G, fmt, layout)


@pytest.mark.parametrize("in_dtype", [oracle.F16, oracle.F32])
def test_input_dtypes(in_dtype):
    xb = synth.activations_bf16(22, 29, 1024, outlier_p=0.01)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    x = xf.astype(np.float16).view(np.uint16) if in_dtype == oracle.F16 else xf
    for fmt in (oracle.SCALE_F32, oracle.SCALE_UE8M0):
        _full_case(x, in_dtype, 128, fmt, "row")


@pytest.mark.parametrize("K", [32, 96, 512, 608, 7296])
def test_ragged_widths(K):
    G = 32 if K % 128 else 128
    x = synth.activations_bf16(23, 5, K)
    _full_case(x, oracle.BF16, G, oracle.SCALE_UE8M0, "col")
    _full_case(x, oracle.BF16, G, oracle.SCALE_F32, "row")


def test_silu_small_full():
    x = synth.activations_bf16(24, 300, 2 * 2048)
    _full_case(x, oracle.BF16, 128, oracle.SCALE_F32, "row", silu=True)
    _full_case(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "col", silu=True)


def test_silu_large_magnitudes():
    # gates far into both tails of silu, and inputs whose products land near the clamp
    xb = synth.activations_bf16(25, 64, 2 * 512)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).copy()
    xf[:, :512] *= 40.0
    x = synth.f64_to_bf16_bits(xf.astype(np.float64))
    _full_case(x, oracle.BF16, 128, oracle.SCALE_F32, "row", silu=True)
    _full_case(x, oracle.BF16, 64, oracle.SCALE_UE8M0, "row", silu=True)


def test_silu_division_paths():
    # fp32 gates at the point (-87) below which a wave computes g / (1 + exp(-g)) with the
    # general division instead of the short form, and other edge values of the quotient:
    # rows 0-1 keep every 1024-wide chunk on the short form, rows 2-6 send one chunk or both
    # to the general division. Codes and scales must match the oracle either way.
    K = 2048
    xb = synth.activations_bf16(31, 7, 2 * K)
    x = (xb.astype(np.uint32) << 16).view(np.float32).copy()
    f32 = np.float32
    x[1, 5], x[1, 700], x[1, 1800] = f32(-87.0), f32(-86.99999), f32(-80.0)
    x[2, 3] = np.nextafter(f32(-87.0), f32(-np.inf))
    x[3, 1030], x[3, 1500] = f32(-87.3365479), f32(-88.5)
    x[4, :64] = np.linspace(-100.0, -80.0, 64, dtype=np.float32)
    x[5, 10:15] = [f32(1e-40), f32(-1e-40), f32(0.0), f32(-0.0), f32(1.4e-45)]
    x[5, 1100] = f32(-1e30)
    x[6, 20], x[6, K + 20] = f32(3e38), f32(0.5)
    x[6, 21], x[6, K + 21] = f32(-3e38), f32(0.5)
    x[6, 1200], x[6, K + 1200] = f32(2e9), f32(-3.0)
    for G, fmt, layout in ((128, oracle.SCALE_F32, "row"), (32, oracle.SCALE_UE8M0, "col"),
                           (K, oracle.SCALE_F32, "row"), (K, oracle.SCALE_UE8M0, "col")):
        _full_case(x, oracle.F32, G, fmt, layout, silu=True)


def test_strided_rows():
    # rows of x and q taken from wider buffers (row stride > K)
    f = fq()
    xb = synth.activations_bf16(26, 17, 1024)
    x = torch.from_numpy(xb).cuda().view(torch.bfloat16)[:, :896]
    q = torch.full((17, 1024), FILL, dtype=torch.uint8, device="cuda")[:, :896]
    s = torch.full((17, 7), FILL, dtype=torch.uint8, device="cuda")
    f.fp8q_group_quant(x, q, s, 128)
    torch.cuda.synchronize()
    qo, so = _oracle(np.ascontiguousarray(xb[:, :896]), oracle.BF16, 128, oracle.SCALE_UE8M0, "row")
    _assert_same(q.cpu().numpy(), qo, "q")
    _assert_same(s.cpu().numpy(), so, "scales")
    full = q.as_strided((17, 1024), (1024, 1)).cpu().numpy()
    assert np.all(full[:, 896:] == FILL)


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("in_dtype", [oracle.BF16, oracle.F16, oracle.F32])
def test_col_major_ue8m0_row_quads(G, in_dtype):
    # flat, column-major UE8M0 bytes, rows a multiple of 4: the kernel that writes each group's
    # scale bytes for 4 rows as one word. K = 2560 ends in half a chunk.
    xb = synth.activations_bf16(32, 44, 2560, outlier_p=0.02)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    x = xb if in_dtype == oracle.BF16 else (xf.astype(np.float16).view(np.uint16) if in_dtype == oracle.F16 else xf)
    _full_case(x, in_dtype, G, oracle.SCALE_UE8M0, "col")
    if in_dtype == oracle.BF16:
        xs = synth.activations_bf16(33, 24, 2 * 1536)
        _full_case(xs, in_dtype, G, oracle.SCALE_UE8M0, "col", silu=True)


def test_col_major_ue8m0_unaligned_scale_columns():
    # a column stride that is not a multiple of 4 bytes (and rows not a multiple of 4) keeps
    # the one-byte scale stores; the padding between columns stays untouched
    f = fq()
    for M, pad in ((40, 2), (42, 0), (40, 4)):
        xb = synth.activations_bf16(34, M, 1536)
        x = torch.from_numpy(xb).cuda().view(torch.bfloat16)
        q = torch.empty((M, 1536), dtype=torch.uint8, device="cuda")
        store = torch.full((1536 // 128, M + pad), FILL, dtype=torch.uint8, device="cuda")
        s = store[:, :M].t()
        f.fp8q_group_quant(x, q, s, 128)
        torch.cuda.synchronize()
        qo, so = _oracle(xb, oracle.BF16, 128, oracle.SCALE_UE8M0, "col")
        _assert_same(q.cpu().numpy(), qo, f"q M={M} pad={pad}")
        sn = store.cpu().numpy()
        _assert_same(np.ascontiguousarray(sn[:, :M]), so, f"scales M={M} pad={pad}")
        assert np.all(sn[:, M:] == FILL)


def test_every_bf16_value_through_unit_scale():
    # each group starts with 448, so its UE8M0 byte is 127 and the multiplier is exactly 1:
    # every finite bf16 value in [-448, 448] reaches the fp8 conversion unchanged
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    vals = bits[np.isfinite(f) & (np.abs(f) <= 448)].astype(np.uint16)
    per = 127
    n = -(-vals.size // per)
    body = np.zeros(n * per, dtype=np.uint16)
    body[:vals.size] = vals
    x = np.concatenate([np.full((n, 1), 0x43E0, dtype=np.uint16), body.reshape(n, per)], axis=1)  # 448
    qg, sg = _gpu_quant(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "row")
    assert np.all(sg == 127)
    qo, so = _oracle(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "row")
    _assert_same(qg, qo, "q")


def test_fp32_sweep_through_unit_scale():
    # fp32 inputs (F32 path) covering every exponent of the e4m3 range, mid-points included
    g = np.random.default_rng(5)
    mant = g.integers(0, 1 << 23, size=1 << 20, dtype=np.uint32)
    expo = g.integers(100, 136, size=1 << 20, dtype=np.uint32)
    sign = g.integers(0, 2, size=1 << 20, dtype=np.uint32) << 31
    v = (sign | (expo << 23) | mant).view(np.float32)
    v = np.clip(v, -448, 448)
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    extra = np.concatenate([mids, np.nextafter(mids, np.float32(1e9)), np.nextafter(mids, np.float32(-1)),
                            -mids])
    v = np.concatenate([v, extra]).astype(np.float32)
    per = 127
    n = -(-v.size // per)
    body = np.zeros(n * per, dtype=np.float32)
    body[:v.size] = v
    x = np.concatenate([np.full((n, 1), 448.0, dtype=np.float32), body.reshape(n, per)], axis=1)
    qg, sg = _gpu_quant(x, oracle.F32, 128, oracle.SCALE_UE8M0, "row")
    assert np.all(sg == 127)
    qref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()  # library cast
    _assert_same(qg, qref, "q vs torch cast")
    qo = oracle.e4m3_encode(x[:2048])
    _assert_same(qg[:2048], qo, "q vs oracle encoder")


# Every fp32 bit pattern of magnitude <= 448 (both signs, subnormals and zeros included)
# through the kernel's fp32 -> e4m3 step: rows of one 448 (UE8M0 byte 127, multiplier exactly
# 1) and 127 patterns, so each pattern reaches the clamp and the conversion unchanged
# (anything larger would change the group's scale; the clamp itself is covered by the
# silu and sweep tests). The reference is torch's CPU cast (a library routine).
# 2 x (0x43E00000 + 1) patterns in 8 parts, streamed in chunks of 2^25 magnitudes.
_MAG_END = 0x43E00000 + 1  # bits of 448, plus one


@pytest.mark.parametrize("part", range(8))
def test_fp32_to_e4m3_every_pattern_up_to_448(part):
    f = fq()
    chunk = 1 << 25
    per = 127
    lo = part * (_MAG_END // 8)
    hi = _MAG_END if part == 7 else (part + 1) * (_MAG_END // 8)
    for start in range(lo, hi, chunk):
        mags = np.arange(start, min(start + chunk, hi), dtype=np.uint32)
        v = np.concatenate([mags, mags | np.uint32(0x80000000)]).view(np.float32)
        n = -(-v.size // per)
        body = np.zeros(n * per, dtype=np.float32)
        body[:v.size] = v
        x = np.empty((n, 128), dtype=np.float32)
        x[:, 0] = 448.0
        x[:, 1:] = body.reshape(n, per)
        xd = torch.from_numpy(x).cuda()
        q = torch.empty((n, 128), dtype=torch.uint8, device="cuda")
        sc = torch.empty((n, 1), dtype=torch.uint8, device="cuda")
        f.fp8q_group_quant(xd, q, sc, 128)
        torch.cuda.synchronize()
        assert bool(torch.all(sc == 127)), f"chunk {start:#x}: scale byte is not 127"
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8)
        got = q.cpu()
        if not torch.equal(got, ref):
            i, j = (got != ref).nonzero()[0].tolist()
            raise AssertionError(f"chunk {start:#x}: input bits {x.view(np.uint32)[i, j]:#010x} "
                                 f"gpu {int(got[i, j]):#04x} torch {int(ref[i, j]):#04x}")
        del xd, q


# ----------------------------------------------------------------------------- masked
def _masked_input(E, M, K, seed):
    return np.stack([synth.activations_bf16(seed, M, K, tensor_id=(synth.T_X << 12) | e) for e in range(E)])


@pytest.mark.parametrize("layout", ["col", "row"])
def test_masked_small_full(layout):
    E, M, K = 6, 40, 1024
    x = _masked_input(E, M, K, 31)
    mm = np.array([0, 1, 40, 39, 17, 3], dtype=np.int32)
    _full_case(x, oracle.BF16, 128, oracle.SCALE_UE8M0, layout, masked_m=mm)
    _full_case(x, oracle.BF16, 128, oracle.SCALE_F32, layout, masked_m=mm)


# Up to 64 experts the expert prefix is one wave's scan; beyond, a block-wide scan: both
# sides of the boundary, with empty, full and clamped counts among them
@pytest.mark.parametrize("E", [64, 65, 300])
def test_masked_many_experts(E):
    M, K = 8, 256
    x = _masked_input(E, M, K, 36 + E)
    mm = synth.masked_rows(36 + E, E, M)
    mm[0], mm[E // 2], mm[E - 1] = 0, M, M + 3
    _full_case(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "col", masked_m=mm)
    _full_case(x, oracle.BF16, 128, oracle.SCALE_F32, "row", masked_m=mm)


def test_masked_counts_are_clamped():
    E, M, K = 4, 8, 256
    x = _masked_input(E, M, K, 32)
    mm = np.array([-5, 100, 0, 8], dtype=np.int32)
    _full_case(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "col", masked_m=mm)


def test_masked_result_independent_of_expected_m():
    E, M, K = 8, 64, 512
    x = _masked_input(E, M, K, 33)
    mm = synth.masked_rows(33, E, M)
    ref = None
    for em in (0, 1, 7, 64, 1000):
        q, s = _gpu_quant(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "col", masked_m=mm, expected_m=em)
        if ref is None:
            ref = (q, s)
        else:
            _assert_same(q, ref[0], f"q expected_m={em}")
            _assert_same(s, ref[1], f"s expected_m={em}")


def test_masked_silu_full():
    E, M, K = 5, 24, 512
    x = _masked_input(E, M, 2 * K, 34)
    mm = np.array([24, 0, 5, 23, 1], dtype=np.int32)
    _full_case(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "col", silu=True, masked_m=mm)


@pytest.mark.parametrize("forced", [False, True])
def test_masked_moe_workload_full(forced):
    """Every valid row of all 32 experts (7833 rows; forced: counts 0, 1, 511, 512 in the
    first four experts) compared byte for byte, codes and scales; the oracle leaves the
    sentinel in rows past masked_m, so the same comparison checks that they are untouched."""
    w = synth.MASKED
    x = np.stack([synth.quant_input(w, e) for e in range(w.E)])
    mm = synth.masked_rows(w.seed, w.E, w.M)
    if forced:
        mm[:4] = [0, 1, 511, 512]
    qg, sg = _gpu_quant(x, oracle.BF16, w.G, oracle.SCALE_UE8M0, "col", masked_m=mm, expected_m=256)
    qo, so = _oracle(x, oracle.BF16, w.G, oracle.SCALE_UE8M0, "col", masked_m=mm)
    _assert_same(qg, qo, "q")
    _assert_same(sg, so, "scales")
    for e in range(w.E):
        assert np.all(qg[e, mm[e]:] == FILL), f"expert {e}: rows past masked_m were written"
    assert not np.any((qg[0, :mm[0]] & 0x7F) == 0x7F)


# ----------------------------------------------------------------------------- full-size flat
def test_dense_m4096_full():
    """All 4096 x 7168 codes and 56 x 4096 UE8M0 scales against the oracle."""
    w = synth.dense(4096)
    x = synth.quant_input(w)
    qg, sg = _gpu_quant(x, oracle.BF16, w.G, oracle.SCALE_UE8M0, "col")
    qo, so = _oracle(x, oracle.BF16, w.G, oracle.SCALE_UE8M0, "col")
    _assert_same(qg, qo, "q")
    _assert_same(sg, so, "scales")
    # no NaN code, and each group's largest code is in the top binade
    assert not np.any((qg & 0x7F) == 0x7F)
    top = (qg & 0x7F).reshape(4096, 56, 128).max(-1)
    assert np.all(top >= 0x70)  # |code value| >= 128 > 448/4
    assert sg.min() >= 85 and sg.max() <= 247


def test_silu_workload_full():
    """All 8192 rows of silu(gate) * up -> G=128 codes and fp32 row-major scales."""
    w = synth.SILU
    x = synth.quant_input(w)
    qg, sg = _gpu_quant(x, oracle.BF16, w.G, oracle.SCALE_F32, "row", silu=True)
    qo, so = _oracle(x, oracle.BF16, w.G, oracle.SCALE_F32, "row", silu=True)
    _assert_same(qg, qo, "q")
    _assert_same(sg.view(np.uint8), so.view(np.uint8), "scales")
    assert not np.any((qg & 0x7F) == 0x7F)


# ----------------------------------------------------------------------------- API behaviour
def test_empty_problems_are_noops():
    f = fq()
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((0, 256), dtype=torch.uint8, device="cuda")
    s = torch.zeros((0, 2), dtype=torch.uint8, device="cuda")
    f.fp8q_group_quant(x, q, s, 128)
    x3 = torch.zeros((0, 4, 256), dtype=torch.bfloat16, device="cuda")
    f.fp8q_group_quant(x3, torch.zeros((0, 4, 256), dtype=torch.uint8, device="cuda"),
                       torch.zeros((0, 4, 2), dtype=torch.uint8, device="cuda"), 128,
                       masked_m=torch.zeros(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()


def test_invalid_arguments_write_nothing():
    f = fq()
    x = torch.ones((4, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.full((4, 256), FILL, dtype=torch.uint8, device="cuda")
    s = torch.full((4, 2), FILL, dtype=torch.uint8, device="cuda")
    with pytest.raises(f.Fp8qError) as ei:
        f.fp8q_group_quant(x, q, s, 96)
    assert ei.value.status == f.EUNSUPPORTED
    with pytest.raises(f.Fp8qError) as ei:
        f.fp8q_group_quant(x[:, 1:129], q[:, :128], s[:, :1], 128)  # misaligned x
    assert ei.value.status == f.EALIGN
    bad = torch.full((4, 4), FILL, dtype=torch.uint8, device="cuda")[:, ::2]  # strides (4, 2)
    with pytest.raises(f.Fp8qError) as ei:
        f.fp8q_group_quant(x, q, bad, 128)
    assert ei.value.status == f.EINVAL
    torch.cuda.synchronize()
    assert torch.all(q == FILL) and torch.all(s == FILL)


def test_runs_on_the_callers_stream():
    x = synth.activations_bf16(27, 64, 2048)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        qg, sg = _gpu_quant(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "col", stream=st)
    qo, so = _oracle(x, oracle.BF16, 128, oracle.SCALE_UE8M0, "col")
    _assert_same(qg, qo, "q")
    _assert_same(sg, so, "s")


def test_device_check():
    f = fq()
    assert f.fp8q_device_check(0) == f.OK
    assert f.fp8q_device_check(1000) == f.EDEVICE


# ----------------------------------------------------------------- int8 output
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_int8_group_sizes_and_layouts(G, layout):
    x = synth.activations_bf16(41, 37, 1536, outlier_p=0.02)
    _full_case(x, oracle.BF16, G, oracle.SCALE_F32, layout, int8=True)


@pytest.mark.parametrize("in_dtype", [oracle.F16, oracle.F32])
def test_int8_input_dtypes(in_dtype):
    xb = synth.activations_bf16(42, 29, 1024, outlier_p=0.01)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    x = xf.astype(np.float16).view(np.uint16) if in_dtype == oracle.F16 else xf
    _full_case(x, in_dtype, 128, oracle.SCALE_F32, "row", int8=True)


def test_int8_ties_and_edges_through_unit_scale():
    # each row starts with 127, so s = 1 and the multiplier is exactly 1: every half-integer
    # tie, its neighbours, and values past +-127 reach the rounding unchanged
    halves = np.arange(-254, 255, dtype=np.float64) / 2.0
    v = np.concatenate([halves, np.nextafter(halves, 1e9), np.nextafter(halves, -1e9)]).astype(np.float32)
    v = np.clip(v, -127, 127)
    per = 127
    n = -(-v.size // per)
    body = np.zeros(n * per, dtype=np.float32)
    body[:v.size] = v
    x = np.concatenate([np.full((n, 1), 127.0, dtype=np.float32), body.reshape(n, per)], axis=1)
    qg, sg = _gpu_quant(x, oracle.F32, 128, oracle.SCALE_F32, "row", int8=True)
    assert np.all(sg == 1.0)
    _assert_same(qg.view(np.int8), np.rint(x).astype(np.int8), "q vs numpy rint")


def test_int8_masked_and_per_token():
    E, M, K = 5, 24, 1024
    x = _masked_input(E, M, K, 43)
    mm = np.array([24, 0, 5, 23, 1], dtype=np.int32)
    _full_case(x, oracle.BF16, 128, oracle.SCALE_F32, "col", masked_m=mm, int8=True)
    _full_case(x, oracle.BF16, K, oracle.SCALE_F32, "row", masked_m=mm, int8=True)
    _full_case(synth.activations_bf16(44, 33, 9216), oracle.BF16, 9216, oracle.SCALE_F32, "col", int8=True)


def test_int8_dense_m4096_full():
    w = synth.dense(4096)
    x = synth.quant_input(w)
    qg, sg = _gpu_quant(x, oracle.BF16, 128, oracle.SCALE_F32, "row", int8=True)
    qo, so = _oracle(x, oracle.BF16, 128, oracle.SCALE_F32, "row", int8=True)
    _assert_same(qg, qo, "q")
    _assert_same(sg.view(np.uint8), so.view(np.uint8), "scales")
    # codes in [-127, 127] and each group's largest magnitude at 127
    c = qg.view(np.int8).astype(np.int16)
    assert c.min() >= -127 and c.max() <= 127
    assert np.all(np.abs(c).reshape(4096, 56, 128).max(-1) == 127)


def test_int8_rejects_ue8m0_scales():
    f = fq()
    x = torch.ones((4, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.full((4, 256), FILL, dtype=torch.uint8, device="cuda").view(torch.int8)
    s = torch.full((4, 2), FILL, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        f.fp8q_group_quant_int8(x, q, s, 128)
    torch.cuda.synchronize()
    assert torch.all(q.view(torch.uint8) == FILL)


# ----------------------------------------------------------------- per-token (G = K)
# K: one partial chunk, the per-token example's 1024, a ragged tail, the largest row held
# in registers (8 chunks of bf16), rows read twice (9 and 20 chunks, the last ragged)
@pytest.mark.parametrize("K", [48, 256, 1024, 1040, 7168, 8192, 9216, 20000])
@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_per_token_widths(K, fmt):
    x = synth.activations_bf16(45, 19, K, outlier_p=0.005)
    _full_case(x, oracle.BF16, K, fmt, "row" if fmt == oracle.SCALE_F32 else "col")


def test_per_token_fp16_example_shape():
    # the per-token FP8 example's shape: fp16 [128, 1024], fp32 scales [128, 1]
    xb = synth.activations_bf16(46, 128, 1024)
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float16).view(np.uint16)
    _full_case(x, oracle.F16, 1024, oracle.SCALE_F32, "row")


@pytest.mark.parametrize("K", [2048, 4096, 5120])
def test_per_token_fp32_input(K):
    # fp32 rows: 4 chunks stay in registers, 5 are read twice
    xb = synth.activations_bf16(47, 11, K, outlier_p=0.01)
    x = (xb.astype(np.uint32) << 16).view(np.float32)
    _full_case(x, oracle.F32, K, oracle.SCALE_F32, "row")


@pytest.mark.parametrize("K", [2048, 4096, 6144])
def test_per_token_silu(K):
    # silu rows: 4 chunks of silu values stay in registers; 6 are recomputed on the second read
    x = synth.activations_bf16(48, 13, 2 * K)
    _full_case(x, oracle.BF16, K, oracle.SCALE_F32, "row", silu=True)
    _full_case(x, oracle.BF16, K, oracle.SCALE_UE8M0, "col", silu=True)


def test_per_token_masked():
    E, M, K = 6, 40, 3072
    x = _masked_input(E, M, K, 49)
    mm = np.array([0, 1, 40, 39, 17, 3], dtype=np.int32)
    _full_case(x, oracle.BF16, K, oracle.SCALE_UE8M0, "col", masked_m=mm)
    _full_case(x, oracle.BF16, K, oracle.SCALE_F32, "row", masked_m=mm, expected_m=5)


def test_per_token_dense_m4096_full():
    M, K = 4096, 7168
    x = synth.activations_bf16(50, M, K, outlier_p=0.001)
    qg, sg = _gpu_quant(x, oracle.BF16, K, oracle.SCALE_F32, "col")
    qo, so = _oracle(x, oracle.BF16, K, oracle.SCALE_F32, "col")
    _assert_same(qg, qo, "q")
    _assert_same(sg.view(np.uint8), so.view(np.uint8), "scales")
    # no NaN code, each row's largest code is 448 (0x7E), the scale is amax/448
    assert not np.any((qg & 0x7F) == 0x7F)
    assert np.all((qg & 0x7F).max(-1) == 0x7E)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(sg[0], np.abs(xf).max(-1) / np.float32(448))


def test_per_token_needs_k_multiple_of_16():
    f = fq()
    x = torch.ones((4, 1032), dtype=torch.bfloat16, device="cuda")
    q = torch.full((4, 1040), FILL, dtype=torch.uint8, device="cuda")[:, :1032]
    s = torch.zeros((4, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(f.Fp8qError) as ei:
        f.fp8q_group_quant(x, q, s, 1032)
    assert ei.value.status == f.EINVAL
    torch.cuda.synchronize()
    assert torch.all(q == FILL)


# ----------------------------------------------------------------- packed UE8M0 scales
def _gpu_quant_packed(x_np, G, layout, silu=False, masked_m=None):
    """GPU quant with FP8Q_SCALE_UE8M0_PACKED output: returns (q, words) with the words as
    stored, [.., M, ng/4] ("row") or [.., ng/4, M] ("col"), as int32."""
    f = fq()
    x = _to_dev(x_np, oracle.BF16)
    x3 = x if x.dim() == 3 else x[None]
    E, M, W = x3.shape
    K = W // 2 if silu else W
    nw = K // G // 4
    q = torch.full((E, M, K), FILL, dtype=torch.uint8, device="cuda")
    shape = (E, M, 4 * nw) if layout == "row" else (E, nw, 4 * M)
    s_store = torch.full(shape, FILL, dtype=torch.uint8, device="cuda").view(torch.int32)
    s_view = s_store if layout == "row" else s_store.transpose(1, 2)
    mm = None if masked_m is None else torch.from_numpy(np.asarray(masked_m, dtype=np.int32)).cuda()
    fn = f.fp8q_silu_mul_group_quant if silu else f.fp8q_group_quant
    fn(x3, q, s_view, G, masked_m=mm)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s_store.cpu().numpy()


def _packed_case(x_np, G, layout, silu=False, masked_m=None):
    x3 = x_np if x_np.ndim == 3 else x_np[None]
    qg, wg = _gpu_quant_packed(x3, G, layout, silu, masked_m)
    qo, so = oracle.group_quant(x3, G, oracle.SCALE_UE8M0, "row", silu=silu, masked_m=masked_m, fill=FILL)
    wo = oracle.pack_ue8m0(so)  # [E, M, ng/4]; untouched rows keep FILL bytes in every word
    if layout == "col":
        wo = np.ascontiguousarray(wo.transpose(0, 2, 1))
    _assert_same(qg, qo, "q")
    _assert_same(wg, wo, "packed scale words")


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_packed_ue8m0_scales(G, layout):
    x = synth.activations_bf16(41, 70, 1024, outlier_p=0.01)
    _packed_case(x, G, layout)


def test_packed_ue8m0_masked_and_silu():
    E, M, K = 6, 40, 1024
    x = _masked_input(E, M, K, 42)
    mm = np.array([0, 1, 40, 39, 17, 3], dtype=np.int32)
    _packed_case(x, 128, "col", masked_m=mm)
    xs = _masked_input(5, 24, 2 * 512, 43)
    _packed_case(xs, 128, "col", silu=True, masked_m=np.array([24, 0, 5, 23, 1], dtype=np.int32))


def test_packed_ue8m0_needs_groups_in_fours():
    f = fq()
    x = torch.zeros((4, 384), dtype=torch.bfloat16, device="cuda")  # 3 groups of 128
    q = torch.empty((4, 384), dtype=torch.uint8, device="cuda")
    s = torch.full((4, 1), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="multiple of 4 groups"):
        f.fp8q_group_quant(x, q, s, 128)
    assert torch.all(s == 7)

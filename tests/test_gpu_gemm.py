"""GPU parity of the block-scaled FP8 GEMMs against the fp64 CPU oracle computed from the
same FP8 bytes and scales (both produced by the generator or by the oracle quantizer, never
by the GPU). Tolerance (tests/gemm_check.py): 2 bf16 ulp per element, with a counted fp32
accumulation allowance where the exact result cancels, and 2e-3 relative Frobenius error.

Full comparison at sizes the oracle finishes in seconds (several tiles and ragged tails);
at the named workloads' full sizes, seeded samples of output elements (including tile
corners) are compared, in the same launch configuration the benchmark uses."""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
from gemm_check import check

pytestmark = pytest.mark.gpu

SENT = 0xA5A5
SENT_I16 = SENT - 0x10000  # the same 16 bits as a signed value, for torch.full


def fq():
    import fp8_group_quant_amd
    return fp8_group_quant_amd


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _gpu_block(a, sa, b, sb, sa_layout="row", ldy=None):
    """a [M,K] codes, sa storage ([M,kb] row or [kb,M] col, fp32 or uint8), b [N,K], sb [nb,kb]."""
    f = fq()
    M, K = a.shape
    N = b.shape[0]
    ldy = ldy or N
    y = torch.full((M, ldy), SENT_I16, dtype=torch.int16, device="cuda")
    sa_d = _dev(sa)
    sa_v = sa_d if sa_layout == "row" else sa_d.t()
    f.fp8q_gemm_blockscaled(_dev(a), sa_v, _dev(b), _dev(sb), y.view(torch.bfloat16)[:, :N], f.GEMM_BLOCK128)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


def _fmt(s):
    return oracle.SCALE_F32 if s.dtype == np.float32 else oracle.SCALE_UE8M0


def _sample(M, N, count, seed, tile=256):
    """Output elements to compare at full size: the corners, `count` seeded random ones and
    one complete tile x tile block of outputs at a seeded tile position (ragged where it
    meets the edge)."""
    g = np.random.default_rng(seed)
    ms = np.concatenate([[0, M - 1, 0, M - 1, min(127, M - 1), min(128, M - 1)], g.integers(0, M, count)])
    ns = np.concatenate([[0, N - 1, N - 1, 0, min(128, N - 1), min(127, N - 1)], g.integers(0, N, count)])
    m0 = int(g.integers(0, -(-M // tile))) * tile
    n0 = int(g.integers(0, -(-N // tile))) * tile
    tm, tn = np.meshgrid(np.arange(m0, min(M, m0 + tile)), np.arange(n0, min(N, n0 + tile)), indexing="ij")
    return np.concatenate([ms, tm.ravel()]), np.concatenate([ns, tn.ravel()])


# ----------------------------------------------------------------------------- BLOCK128 full
def test_tiny_workload_full():
    w = synth.TINY
    x = synth.quant_input(w)
    q, s = oracle.group_quant(x, 128, oracle.SCALE_F32, "row")  # oracle-quantized activations
    wq, ws = synth.weights(w)
    y = _gpu_block(q, s, wq, ws)
    ys, ss = oracle.gemm_block128(q, s, wq, ws, oracle.SCALE_F32)
    check(y, ys, ss, w.K, "tiny", cls="outlier")


# M > 128 with M % 4 == 0 reaches the direct-to-LDS kernel for fp32 weight scales (also
# with UE8M0 column-major activation scales); M % 4 != 0 or UE8M0 weight scales take the
# register-staged kernel; K = 128 and 256 cover pipelines shorter than their depth, and
# K % 512 == 0 the four-step scale groups (K = 512: a single group).
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 130, 256), (129, 200, 384), (257, 300, 640),
                                   (64, 1024, 1024), (132, 136, 128), (264, 128, 256),
                                   (260, 300, 640), (516, 136, 384), (132, 136, 512), (260, 300, 1024)])
@pytest.mark.parametrize("sa_kind", ["f32-row", "ue8m0-col", "ue8m0-row"])
@pytest.mark.parametrize("sb_kind", ["f32", "ue8m0"])
def test_ragged_shapes_full(M, N, K, sa_kind, sb_kind):
    w = synth.Workload("t", seed=40 + M, M=M, K=K, N=N, scale_fmt=sa_kind.split("-")[0])
    a, sa = synth.gemm_activation(w)
    b, sbf = synth.weights(w)
    sb = sbf if sb_kind == "f32" else synth.e8m0_exponents(7, sbf.shape[0], sbf.shape[1], tensor_id=77)
    layout = sa_kind.split("-")[1]
    sa_store = sa if layout == "row" else np.ascontiguousarray(sa.T)
    y = _gpu_block(a, sa_store, b, sb, layout)
    ys, ss = oracle.gemm_block128(a, sa_store, b, sb, _fmt(sa), layout, _fmt(sb))
    check(y, ys, ss, K, f"{M}x{N}x{K}")


# Flat problems with at least 256 tiles of 256x256 take the two-stage kernel with
# 256-column tiles (fp32 weight scales; fp32 row or UE8M0 column activation scales; fp32
# ones in four-step groups when K is a multiple of 512). M=4000, N=4200 leaves ragged
# tiles in both directions; K = 128, 256, 384 run 1, 2 and 3 steps (pipelines shorter
# than two stages, and both stages ending the loop), K = 512 and 1024 one and two scale
# groups. Outputs on a grid of rows x columns through tile and wave-tile boundaries plus
# random ones are compared; every output must be written.
@pytest.mark.parametrize("K", [128, 256, 384, 512, 1024])
@pytest.mark.parametrize("sa_kind", ["f32-row", "ue8m0-col", "ue8m0-row"])
def test_wide_tiles_ragged_sampled(K, sa_kind):
    M, N = 4000, 4200
    w = synth.Workload("t", seed=60 + K, M=M, K=K, N=N, scale_fmt=sa_kind.split("-")[0])
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    layout = sa_kind.split("-")[1]
    sa_store = sa if layout == "row" else np.ascontiguousarray(sa.T)
    y = _gpu_block(a, sa_store, b, sb, layout)
    assert not np.any(y == SENT)
    g = np.random.default_rng(K)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 127, 128, 255, 256, 257, 511, 512, 3839, 3840, 3841,
                                      3967, 3968, 3998, 3999], g.integers(0, M, 46)]))
    cols = np.unique(np.concatenate([[0, 63, 64, 127, 128, 129, 191, 192, 255, 256, 4095, 4096, 4097,
                                      4159, 4160, 4198, 4199], g.integers(0, N, 47)]))
    ms, ns = (v.ravel() for v in np.meshgrid(rows, cols, indexing="ij"))
    ys, ss = oracle.gemm_block128(a, sa_store, b, sb, _fmt(sa), layout, oracle.SCALE_F32, at=(ms, ns))
    check(y[ms, ns], ys, ss, K, f"wide {M}x{N}x{K} {sa_kind}")


# 4000 x 4000 is exactly one round of 256 tiles of 256x256: one launch, ragged in both
# directions. (4000 x 4200 above takes two: columns [0, 4096) as 256x256 tiles, the last
# 104 as 128x256 tiles that fill the second round.)
@pytest.mark.parametrize("sa_kind", ["f32-row", "ue8m0-col"])
def test_wide_tiles_one_round_ragged_sampled(sa_kind):
    M, N, K = 4000, 4000, 512
    w = synth.Workload("t", seed=66, M=M, K=K, N=N, scale_fmt=sa_kind.split("-")[0])
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    layout = sa_kind.split("-")[1]
    sa_store = sa if layout == "row" else np.ascontiguousarray(sa.T)
    y = _gpu_block(a, sa_store, b, sb, layout)
    assert not np.any(y == SENT)
    g = np.random.default_rng(66)
    rows = np.unique(np.concatenate([[0, 255, 256, 3839, 3840, 3999], g.integers(0, M, 40)]))
    cols = np.unique(np.concatenate([[0, 255, 256, 3839, 3840, 3999], g.integers(0, N, 40)]))
    ms, ns = (v.ravel() for v in np.meshgrid(rows, cols, indexing="ij"))
    ys, ss = oracle.gemm_block128(a, sa_store, b, sb, _fmt(sa), layout, oracle.SCALE_F32, at=(ms, ns))
    check(y[ms, ns], ys, ss, K, f"wide one round {sa_kind}")


# UE8M0 weight-block scales with UE8M0 column-major activation scales (K a multiple of 512)
# go to the matrix core on both sides with no fold: narrow tiles, 256x256 tiles with the
# column split of a partly empty last round, masked experts; K = 640 keeps the
# register-staged kernel.
def _ue8m0_weights(w, seed):
    b, sbf = synth.weights(w)
    return b, synth.e8m0_exponents(seed, sbf.shape[0], sbf.shape[1], lo=-4, hi=4, tensor_id=98)


@pytest.mark.parametrize("M,N,K", [(300, 260, 512), (4000, 4200, 1024), (136, 1000, 2048), (260, 384, 640)])
def test_ue8m0_weight_scales(M, N, K):
    w = synth.Workload("e8", seed=64, M=M, K=K, N=N, scale_fmt="ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sb = _ue8m0_weights(w, 64)
    sa_col = np.ascontiguousarray(sa.T)
    y = _gpu_block(a, sa_col, b, sb, "col")
    assert not np.any(y == SENT)
    g = np.random.default_rng(M + N)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(0, M, 127), g.integers(0, M, 30)]))
    cols = np.unique(np.concatenate([[0, N - 1], np.arange(0, N, 127), g.integers(0, N, 30)]))
    ms, ns = (v.ravel() for v in np.meshgrid(rows, cols, indexing="ij"))
    ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col", oracle.SCALE_UE8M0, at=(ms, ns))
    check(y[ms, ns], ys, ss, K, f"ue8m0 weights {M}x{N}x{K}")


# The same with packed UE8M0 activation words (row- or column-major words): narrow tiles, the
# 256x256 tiles with the column split, and the full dense shape
@pytest.mark.parametrize("M,N,K", [(300, 260, 512), (4000, 4200, 1024), (136, 1000, 2048), (4096, 7168, 7168)])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_packed_activation_ue8m0_weight_scales(M, N, K, layout):
    w = synth.Workload("pe8", seed=67, M=M, K=K, N=N, scale_fmt="ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sb = _ue8m0_weights(w, 67)
    y = _gpu_block_packed(a, sa, b, sb, layout)
    assert not np.any(y == SENT)
    g = np.random.default_rng(M + N + K)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(0, M, 127), g.integers(0, M, 30)]))
    cols = np.unique(np.concatenate([[0, N - 1], np.arange(0, N, 127), g.integers(0, N, 30)]))
    ms, ns = (v.ravel() for v in np.meshgrid(rows, cols, indexing="ij"))
    ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_UE8M0, "row", oracle.SCALE_UE8M0, at=(ms, ns))
    check(y[ms, ns], ys, ss, K, f"packed {layout} words, ue8m0 weights {M}x{N}x{K}")


# Small M (the LDS-staged split-K kernel) with UE8M0 weight-block scales, decoded to fp32 in
# its table, under each activation-scale layout; N ragged
@pytest.mark.parametrize("M", [1, 16, 33, 100, 128])
@pytest.mark.parametrize("sa_kind", ["f32-row", "ue8m0-row", "ue8m0-col", "packed-col"])
def test_small_m_ue8m0_weight_scales(M, sa_kind):
    N, K = 300, 1024
    w = synth.Workload("sm8", seed=68 + M, M=M, K=K, N=N, scale_fmt="f32" if sa_kind.startswith("f32") else "ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sb = _ue8m0_weights(w, 68)
    if sa_kind.startswith("packed"):
        y = _gpu_block_packed(a, sa, b, sb, "col")
    elif sa_kind.endswith("col"):
        y = _gpu_block(a, np.ascontiguousarray(sa.T), b, sb, "col")
    else:
        y = _gpu_block(a, sa, b, sb)
    ys, ss = oracle.gemm_block128(a, sa, b, sb, _fmt(sa), "row", oracle.SCALE_UE8M0)
    check(y, ys, ss, K, f"small M={M} {sa_kind}, ue8m0 weights")


def test_ue8m0_weight_scales_masked():
    E, cap, N, K = 5, 300, 384, 1024
    a, sa, b, _ = _masked_operands(E, cap, N, K, 65)
    sb = synth.e8m0_exponents(65, E * (N // 128), K // 128, lo=-4, hi=4, tensor_id=97).reshape(E, N // 128, K // 128)
    mm = np.array([300, 0, 129, 7, 256], dtype=np.int32)
    y = _gpu_masked(a, sa, b, sb, mm)
    for e in range(E):
        r = mm[e]
        if r > 0:
            ys, ss = oracle.gemm_block128(a[e, :r], np.ascontiguousarray(sa[e][:, :r]), b[e], sb[e],
                                          oracle.SCALE_UE8M0, "col", oracle.SCALE_UE8M0)
            check(y[e, :r], ys, ss, K, f"expert {e}")
        assert np.all(y[e, r:] == SENT), f"expert {e}: rows past masked_m written"


def test_ue8m0_weight_scales_dense_m4096_sampled():
    w = synth.dense(4096)
    a, sa = synth.gemm_activation(w)
    b, sb = _ue8m0_weights(w, 66)
    sa_col = np.ascontiguousarray(sa.T)
    y = _gpu_block(a, sa_col, b, sb, "col")
    ms, ns = _sample(w.M, w.N, 5000, 12)
    ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col", oracle.SCALE_UE8M0, at=(ms, ns))
    check(y[ms, ns], ys, ss, w.K, "dense M=4096, UE8M0 weight scales")
    assert not np.any(y == SENT)


def test_padded_output_rows_untouched():
    w = synth.Workload("t", seed=50, M=70, K=256, N=130, scale_fmt="f32")
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    y = _gpu_block(a, sa, b, sb, "row", ldy=136)
    ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32)
    check(y[:, :130], ys, ss, 256, "padded")
    assert np.all(y[:, 130:] == SENT)


# ----------------------------------------------------------------------------- BLOCK128 workloads
@pytest.mark.parametrize("M", [1, 16, 128])
def test_dense_small_m(M):
    w = synth.dense(M)
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    sa_col = np.ascontiguousarray(sa.T)
    y = _gpu_block(a, sa_col, b, sb, "col")
    ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col")  # every output
    check(y, ys, ss, w.K, f"dense M={M} (c2)")


# ----------------------------------------------------------------------------- split K
def _gpu_block_ws(a, sa, b, sb, sa_layout="row", workspace=None, packed=False):
    """As _gpu_block through fp8q_gemm_blockscaled_ws: workspace None lets the binding size
    one; a zero-length tensor passes none."""
    f = fq()
    M, K = a.shape
    N = b.shape[0]
    y = torch.full((M, N), SENT_I16, dtype=torch.int16, device="cuda")
    if packed:
        sa_v = _packed_words(sa, sa_layout)
    else:
        sa_d = _dev(sa)
        sa_v = sa_d if sa_layout == "row" else sa_d.t()
    f.fp8q_gemm_blockscaled(_dev(a), sa_v, _dev(b), _dev(sb), y.view(torch.bfloat16), f.GEMM_BLOCK128,
                            workspace=workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


def _split_ranges(M, N, K):
    """K ranges the workspace size implies (1: no workspace)."""
    nbytes = fq().fp8q_gemm_workspace_size(M, N, K, fq().GEMM_BLOCK128)
    assert nbytes % (M * N * 4) == 0
    return max(1, nbytes // (M * N * 4))


# 16 < M <= 128 with a workspace: the split-K kernel (64-row variant for M <= 64, 128-row
# above) with short K ranges (the split's minimum of 4 blocks) of uneven length (K / 128 not
# a multiple of the range count), ragged N and rows past M inside the last 16-row slice,
# under every scale layout
@pytest.mark.parametrize("M,N,K", [(17, 300, 1152), (32, 520, 2176), (33, 300, 1152), (64, 1000, 2176),
                                   (65, 260, 3200), (100, 200, 1664), (128, 130, 1792)])
@pytest.mark.parametrize("sa_kind", ["f32-row", "ue8m0-col", "packed-col", "ue8m0-row"])
@pytest.mark.parametrize("sb_kind", ["f32", "ue8m0"])
def test_split_k_full(M, N, K, sa_kind, sb_kind):
    if sa_kind == "packed-col" and K % 512:
        K += 512 - K % 512
    assert _split_ranges(M, N, K) > 1
    w = synth.Workload("sk", seed=90 + M, M=M, K=K, N=N, scale_fmt=sa_kind.split("-")[0].replace("packed", "ue8m0"))
    a, sa = synth.gemm_activation(w)
    if sb_kind == "f32":
        b, sb = synth.weights(w)
    else:
        b, sb = _ue8m0_weights(w, 91)
    layout = sa_kind.split("-")[1]
    if sa_kind.startswith("packed"):
        y = _gpu_block_ws(a, sa, b, sb, layout, packed=True)
        ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_UE8M0, "row", _fmt(sb))
    else:
        sa_store = sa if layout == "row" else np.ascontiguousarray(sa.T)
        y = _gpu_block_ws(a, sa_store, b, sb, layout)
        ys, ss = oracle.gemm_block128(a, sa_store, b, sb, _fmt(sa), layout, _fmt(sb))
    check(y, ys, ss, K, f"split K {M}x{N}x{K} {sa_kind} {sb_kind}")


# Full-size shapes: the dense projection's K with ranges of 6 and 7 blocks (K / 128 = 57),
# N not a multiple of the column tile, and a problem wide enough for one range (no
# workspace: bf16 stored by the split kernel itself); sampled outputs plus a whole tile
@pytest.mark.parametrize("M,N,K,ranges", [(100, 4096, 7296, "several"), (128, 4100, 7168, "several"),
                                          (48, 16448, 1792, "one")])
def test_split_k_large_sampled(M, N, K, ranges):
    s = _split_ranges(M, N, K)
    assert (s > 1) == (ranges == "several")
    w = synth.Workload("skl", seed=95 + M, M=M, K=K, N=N, scale_fmt="ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    sa_col = np.ascontiguousarray(sa.T)
    y = _gpu_block_ws(a, sa_col, b, sb, "col")
    assert not np.any(y == SENT)
    ms, ns = _sample(M, N, 4096, 13, tile=128)
    ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col", at=(ms, ns))
    check(y[ms, ns], ys, ss, K, f"split K {M}x{N}x{K} ({s} ranges)")


# The workspace contract: a workspace one byte short, or none, runs the kernel of the plain
# call (identical bits); the exact size runs the split path (within tolerance, last bits may
# differ); a negative size and a misaligned workspace are rejected before any launch.
@pytest.mark.parametrize("M", [17, 24, 32])
def test_rows_17_to_32_without_workspace(M):
    """The plain call (no workspace) takes the LDS-staged kernel for 16 < M <= 128."""
    N, K = 300, 1024
    w = synth.Workload("nw", seed=97 + M, M=M, K=K, N=N, scale_fmt="ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    sa_col = np.ascontiguousarray(sa.T)
    y = _gpu_block_ws(a, sa_col, b, sb, "col", workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col")
    check(y, ys, ss, K, f"no workspace M={M}")


def test_split_k_workspace_contract():
    f = fq()
    M, N, K = 64, 4096, 7168
    nbytes = f.fp8q_gemm_workspace_size(M, N, K, f.GEMM_BLOCK128)
    assert nbytes == _split_ranges(M, N, K) * M * N * 4 and nbytes > 0
    assert f.fp8q_gemm_workspace_size(M, N, K, f.GEMM_MX32) == 0
    assert f.fp8q_gemm_workspace_size(16, N, K, f.GEMM_BLOCK128) == 0
    assert f.fp8q_gemm_workspace_size(4096, N, K, f.GEMM_BLOCK128) == 0
    assert f.fp8q_gemm_workspace_size(M, N, 200, f.GEMM_BLOCK128) == 0
    # K ranges of at least 4 blocks: the dense M=64 and M=128 splits (S=4 of 14 blocks, S=8 of
    # 7) keep their workspace; the tiny problem (4 blocks) runs as one range without one
    assert _split_ranges(64, 4096, 7168) == 4 and _split_ranges(128, 4096, 7168) == 8
    assert f.fp8q_gemm_workspace_size(64, 256, 512, f.GEMM_BLOCK128) == 0
    assert _split_ranges(17, 300, 1152) == 2
    w = synth.dense(M)
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    sa_col = np.ascontiguousarray(sa.T)
    ms, ns = _sample(M, N, 4096, 14, tile=128)
    ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col", at=(ms, ns))
    exact = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    short = torch.empty(nbytes - 1, dtype=torch.uint8, device="cuda")
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    y_split = _gpu_block_ws(a, sa_col, b, sb, "col", exact)
    y_short = _gpu_block_ws(a, sa_col, b, sb, "col", short)
    y_none = _gpu_block_ws(a, sa_col, b, sb, "col", none)
    y_plain = _gpu_block(a, sa_col, b, sb, "col")  # the binding sizes a workspace: split path
    assert np.array_equal(y_short, y_none)
    assert np.array_equal(y_split, y_plain)
    for y, what in ((y_split, "split"), (y_none, "no workspace")):
        check(y[ms, ns], ys, ss, K, f"dense M={M}, {what}")
    lib = f.load_library()
    ad, bd, sad, sbd = _dev(a), _dev(b), _dev(sa_col).t(), _dev(sb)
    y = torch.full((M, N), SENT_I16, dtype=torch.int16, device="cuda")
    big = torch.empty(nbytes + 64, dtype=torch.uint8, device="cuda")

    def call(ws_ptr, ws_bytes):
        return lib.fp8q_gemm_blockscaled_ws(
            ad.data_ptr(), K, sad.data_ptr(), oracle.SCALE_UE8M0, sad.stride(0), sad.stride(1),
            bd.data_ptr(), K, sbd.data_ptr(), oracle.SCALE_F32, sbd.stride(0), sbd.stride(1),
            y.data_ptr(), N, M, N, K, f.GEMM_BLOCK128, ws_ptr, ws_bytes, torch.cuda.current_stream().cuda_stream)

    assert call(big.data_ptr(), -1) == f.EINVAL
    assert call(big.data_ptr() + 8, nbytes) == f.EALIGN
    torch.cuda.synchronize()
    assert torch.all(y == SENT_I16)
    assert call(big.data_ptr() + 16, nbytes) == f.OK
    torch.cuda.synchronize()
    check(y.cpu().numpy().view(np.uint16)[ms, ns], ys, ss, K, "offset workspace")


def test_dense_m4096_sampled():
    w = synth.dense(4096)
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    sa_col = np.ascontiguousarray(sa.T)
    y = _gpu_block(a, sa_col, b, sb, "col")
    ms, ns = _sample(w.M, w.N, 5000, 1)
    ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col", at=(ms, ns))
    check(y[ms, ns], ys, ss, w.K, "dense M=4096 (c2)", cls="act")
    assert not np.any(y == SENT)


def test_silu_down_projection_sampled():
    w = synth.SILU
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    y = _gpu_block(a, sa, b, sb, "row")
    ms, ns = _sample(w.M, w.N, 5000, 2)
    ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_F32, "row", at=(ms, ns))
    check(y[ms, ns], ys, ss, w.K, "silu down-proj (c3)", cls="act")


# ----------------------------------------------------------------------------- masked grouped
def _gpu_masked(a, sa_col, b, sb, mm, expected_m=0):
    """a [E,cap,K]; sa_col [E,kb,cap] (UE8M0 column-major storage); b [E,N,K]; sb [E,nb,kb]."""
    f = fq()
    E, cap, K = a.shape
    N = b.shape[1]
    y = torch.full((E, cap, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_grouped_gemm_masked(_dev(a), _dev(sa_col).transpose(1, 2), _dev(b), _dev(sb), y.view(torch.bfloat16),
                               _dev(mm.astype(np.int32)), expected_m)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=2)
def _masked_operands(E, cap, N, K, seed):
    w = synth.Workload("m", seed=seed, M=cap, K=K, N=N, E=E, scale_fmt="ue8m0", layout="col", masked=True)
    a, sa, b, sb = [], [], [], []
    for e in range(E):
        ae, se = synth.gemm_activation(w, e)
        be, sbe = synth.weights(w, e)
        a.append(ae); sa.append(np.ascontiguousarray(se.T)); b.append(be); sb.append(sbe)
    return np.stack(a), np.stack(sa), np.stack(b), np.stack(sb)


def test_masked_small_full():
    E, cap, N, K = 5, 200, 256, 512
    a, sa, b, sb = _masked_operands(E, cap, N, K, 60)
    mm = np.array([0, 1, 200, 130, 129], dtype=np.int32)
    y = _gpu_masked(a, sa, b, sb, mm)
    for e in range(E):
        r = mm[e]
        if r > 0:
            ys, ss = oracle.gemm_block128(a[e, :r], np.ascontiguousarray(sa[e][:, :r]), b[e], sb[e],
                                          oracle.SCALE_UE8M0, "col")
            check(y[e, :r], ys, ss, K, f"expert {e}")
        assert np.all(y[e, r:] == SENT), f"expert {e}: rows past masked_m written"


def test_masked_f32_row_scales():
    """fp32 activation scales stored row-major per expert ([E][cap][K/128]); K not a multiple
    of 512 selects the per-step scale loads; counts around the 128-row tile boundary."""
    E, cap, N, K = 4, 260, 384, 384
    w = synth.Workload("m", seed=62, M=cap, K=K, N=N, E=E, scale_fmt="f32", layout="row", masked=True)
    ops = [synth.gemm_activation(w, e) + synth.weights(w, e) for e in range(E)]
    a, sa, b, sb = (np.stack([o[i] for o in ops]) for i in range(4))
    mm = np.array([260, 0, 129, 37], dtype=np.int32)
    f = fq()
    y = torch.full((E, cap, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_grouped_gemm_masked(_dev(a), _dev(sa), _dev(b), _dev(sb), y.view(torch.bfloat16),
                               _dev(mm), 0)
    torch.cuda.synchronize()
    y = y.cpu().numpy().view(np.uint16)
    for e in range(E):
        r = mm[e]
        if r > 0:
            ys, ss = oracle.gemm_block128(a[e, :r], sa[e, :r], b[e], sb[e], oracle.SCALE_F32, "row")
            check(y[e, :r], ys, ss, K, f"expert {e}")
        assert np.all(y[e, r:] == SENT), f"expert {e}: rows past masked_m written"


# Masked counts on both sides of every 128-row tile boundary up to the capacity, ragged N,
# both per-step activation scale layouts; UE8M0 row-major bytes with K = 1024 (rows of whole
# words: read as packed words, per expert).
@pytest.mark.parametrize("sa_kind", ["ue8m0-col", "f32-row", "ue8m0-row"])
def test_masked_counts_across_tile_boundaries(sa_kind):
    E, cap, N, K = 10, 700, 320, (1024 if sa_kind == "ue8m0-row" else 256)
    fmt, layout = sa_kind.split("-")
    w = synth.Workload("m", seed=63, M=cap, K=K, N=N, E=E, scale_fmt=fmt, layout=layout, masked=True)
    ops = [synth.gemm_activation(w, e) + synth.weights(w, e) for e in range(E)]
    a, sa, b, sb = (np.stack([o[i] for o in ops]) for i in range(4))
    mm = np.array([128, 384, 385, 512, 513, 640, 641, 257, 700, 127], dtype=np.int32)
    f = fq()
    y = torch.full((E, cap, N), SENT_I16, dtype=torch.int16, device="cuda")
    if layout == "col":
        sa_dev = _dev(np.ascontiguousarray(sa.transpose(0, 2, 1))).transpose(1, 2)
    else:
        sa_dev = _dev(sa)
    f.fp8q_grouped_gemm_masked(_dev(a), sa_dev, _dev(b), _dev(sb), y.view(torch.bfloat16), _dev(mm), 0)
    torch.cuda.synchronize()
    y = y.cpu().numpy().view(np.uint16)
    sfmt = oracle.SCALE_UE8M0 if fmt == "ue8m0" else oracle.SCALE_F32
    for e in range(E):
        r = int(mm[e])
        ys, ss = oracle.gemm_block128(a[e, :r], np.ascontiguousarray(sa[e, :r]), b[e], sb[e], sfmt, "row")
        check(y[e, :r], ys, ss, K, f"expert {e} ({r} rows)")
        assert np.all(y[e, r:] == SENT), f"expert {e}: rows past masked_m written"


def test_masked_result_independent_of_expected_m():
    E, cap, N, K = 6, 300, 384, 256
    a, sa, b, sb = _masked_operands(E, cap, N, K, 61)
    mm = np.array([300, 0, 17, 255, 256, 1], dtype=np.int32)
    ref = _gpu_masked(a, sa, b, sb, mm, 0)
    for em in (1, 64, 300, 5000):
        assert np.array_equal(_gpu_masked(a, sa, b, sb, mm, em), ref), em


def test_masked_counts_are_clamped():
    E, cap, N, K = 3, 64, 128, 128
    a, sa, b, sb = _masked_operands(E, cap, N, K, 62)
    y = _gpu_masked(a, sa, b, sb, np.array([-4, 1000, 5], dtype=np.int32))
    assert np.all(y[0] == SENT)
    ys, ss = oracle.gemm_block128(a[1], np.ascontiguousarray(sa[1]), b[1], sb[1], oracle.SCALE_UE8M0, "col")
    check(y[1], ys, ss, K, "clamped to cap")
    assert np.all(y[2, 5:] == SENT)


@pytest.mark.parametrize("forced", [False, True])
def test_masked_moe_workload_sampled(forced):
    w = synth.MASKED
    a, sa, b, sb = _masked_operands(w.E, w.M, w.N, w.K, w.seed)
    mm = synth.masked_rows(w.seed, w.E, w.M)
    if forced:
        mm[:4] = [0, 1, 511, 512]
    y = _gpu_masked(a, sa, b, sb, mm, expected_m=256)
    g = np.random.default_rng(3)
    ys_all, y_all, s_all = [], [], []
    for e in range(w.E):
        r = int(mm[e])
        assert np.all(y[e, r:] == SENT), f"expert {e}: rows past masked_m written"
        if r == 0:
            continue
        ms = np.concatenate([[0, r - 1], g.integers(0, r, 158)])
        ns = np.concatenate([[0, w.N - 1], g.integers(0, w.N, 158)])
        if r == mm.max():  # one complete 128 x 256 output tile of the fullest expert
            n0 = int(g.integers(0, w.N // 256)) * 256
            tm, tn = np.meshgrid(np.arange(min(r, 128)), np.arange(n0, n0 + 256), indexing="ij")
            ms, ns = np.concatenate([ms, tm.ravel()]), np.concatenate([ns, tn.ravel()])
        ys, ss = oracle.gemm_block128(a[e, :r], np.ascontiguousarray(sa[e][:, :r]), b[e], sb[e],
                                      oracle.SCALE_UE8M0, "col", at=(ms, ns))
        check(y[e][ms, ns], ys, ss, w.K, f"expert {e}")
        ys_all.append(ys); y_all.append(y[e][ms, ns]); s_all.append(ss)
    check(np.concatenate(y_all), np.concatenate(ys_all), np.concatenate(s_all), w.K,
          "masked MoE (c4)" + (", forced counts" if forced else ""))


# ----------------------------------------------------------------------------- MX32
def _gpu_mx(a, ea, b, eb, sk_stride=False):
    f = fq()
    M, K = a.shape
    N = b.shape[0]
    y = torch.full((M, N), SENT_I16, dtype=torch.int16, device="cuda")
    ea_d, eb_d = _dev(ea), _dev(eb)
    if sk_stride:  # scales stored [K/32, rows] and passed as a transposed view (K stride != 1)
        ea_d = _dev(np.ascontiguousarray(ea.T)).t()
        eb_d = _dev(np.ascontiguousarray(eb.T)).t()
    f.fp8q_gemm_blockscaled(_dev(a), ea_d, _dev(b), eb_d, y.view(torch.bfloat16), f.GEMM_MX32)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (130, 96, 256), (136, 200, 512), (300, 260, 1024)])
@pytest.mark.parametrize("sk_stride", [False, True])
def test_mx_full(M, N, K, sk_stride):
    a = synth.weight_codes(70, M, K, tensor_id=1)
    b = synth.weight_codes(70, N, K, tensor_id=2)
    ea = synth.e8m0_exponents(70, M, K // 32, tensor_id=3)
    eb = synth.e8m0_exponents(70, N, K // 32, tensor_id=4)
    y = _gpu_mx(a, ea, b, eb, sk_stride)
    ys, ss = oracle.gemm_mx32(a, ea, b, eb)
    check(y, ys, ss, K, f"mx {M}x{N}x{K}", cls="wide")


# At least 256 tiles of 256x256 take the two-stage kernel (per-step scale loads); ragged in
# both directions, 2 and 8 K steps, scales with unit or row stride along K.
@pytest.mark.parametrize("K", [256, 1024])
@pytest.mark.parametrize("sk_stride", [False, True])
def test_mx_wide_ragged_sampled(K, sk_stride):
    M, N = 4000, 4200
    a = synth.weight_codes(71, M, K, tensor_id=1)
    b = synth.weight_codes(71, N, K, tensor_id=2)
    ea = synth.e8m0_exponents(71, M, K // 32, tensor_id=3)
    eb = synth.e8m0_exponents(71, N, K // 32, tensor_id=4)
    y = _gpu_mx(a, ea, b, eb, sk_stride)
    assert not np.any(y == SENT)
    g = np.random.default_rng(K + 1)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 3839, 3840, 3999], g.integers(0, M, 40)]))
    cols = np.unique(np.concatenate([[0, 63, 64, 191, 192, 255, 256, 4095, 4096, 4199], g.integers(0, N, 40)]))
    ms, ns = (v.ravel() for v in np.meshgrid(rows, cols, indexing="ij"))
    ys, ss = oracle.gemm_mx32(a, ea, b, eb, at=(ms, ns))
    check(y[ms, ns], ys, ss, K, f"mx wide {M}x{N}x{K}", cls="wide")


def test_mx_workload_sampled():
    w = synth.MX
    a, b, ea, eb = synth.mx_operands(w)
    y = _gpu_mx(a, ea, b, eb)
    ms, ns = _sample(w.M, w.N, 5000, 4)
    ys, ss = oracle.gemm_mx32(a, ea, b, eb, at=(ms, ns))
    check(y[ms, ns], ys, ss, w.K, "mxfp8 8192^3 (c5)", cls="wide")
    assert not np.any(y == SENT)


# ------------------------------------------------------------ MX32 with packed E8M0 words
def _mx_scales_dev(e, layout):
    """E8M0 bytes [rows, K/32] on the device as: "bytes" (row-major), "bytes_t" (stored
    [K/32, rows], K stride != 1), or packed int32 words [rows, K/128] stored row-major
    ("row") or column-major ("col")."""
    if layout == "bytes":
        return _dev(e)
    if layout == "bytes_t":
        return _dev(np.ascontiguousarray(e.T)).t()
    return _packed_words(e, layout)


def _gpu_mx_layouts(a, ea, b, eb, la, lb):
    f = fq()
    M, K = a.shape
    N = b.shape[0]
    y = torch.full((M, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_gemm_blockscaled(_dev(a), _mx_scales_dev(ea, la), _dev(b), _mx_scales_dev(eb, lb),
                            y.view(torch.bfloat16), f.GEMM_MX32)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


# Packed words on the direct-to-LDS kernel (256x128 tiles), one operand packed and the other
# row-major bytes, and on the register-staged kernel (the other operand's bytes have a K
# stride != 1).
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (130, 96, 256), (300, 260, 1024)])
@pytest.mark.parametrize("la,lb", [("col", "col"), ("row", "row"), ("col", "bytes"), ("bytes", "col"),
                                   ("col", "bytes_t"), ("bytes_t", "row")])
def test_mx_packed_words_full(M, N, K, la, lb):
    a = synth.weight_codes(72, M, K, tensor_id=1)
    b = synth.weight_codes(72, N, K, tensor_id=2)
    ea = synth.e8m0_exponents(72, M, K // 32, tensor_id=3)
    eb = synth.e8m0_exponents(72, N, K // 32, tensor_id=4)
    y = _gpu_mx_layouts(a, ea, b, eb, la, lb)
    ys, ss = oracle.gemm_mx32(a, ea, b, eb)
    check(y, ys, ss, K, f"mx packed {la}/{lb} {M}x{N}x{K}", cls="wide")


# 256x256 tiles (at least 256 of them) with packed words, ragged in both directions
@pytest.mark.parametrize("la,lb", [("col", "col"), ("row", "bytes")])
def test_mx_packed_words_wide_sampled(la, lb):
    M, N, K = 4000, 4200, 1024
    a = synth.weight_codes(73, M, K, tensor_id=1)
    b = synth.weight_codes(73, N, K, tensor_id=2)
    ea = synth.e8m0_exponents(73, M, K // 32, tensor_id=3)
    eb = synth.e8m0_exponents(73, N, K // 32, tensor_id=4)
    y = _gpu_mx_layouts(a, ea, b, eb, la, lb)
    assert not np.any(y == SENT)
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 3839, 3840, 3999], g.integers(0, M, 40)]))
    cols = np.unique(np.concatenate([[0, 63, 64, 255, 256, 4095, 4096, 4199], g.integers(0, N, 40)]))
    ms, ns = (v.ravel() for v in np.meshgrid(rows, cols, indexing="ij"))
    ys, ss = oracle.gemm_mx32(a, ea, b, eb, at=(ms, ns))
    check(y[ms, ns], ys, ss, K, f"mx packed wide {la}/{lb}", cls="wide")


def test_mx_packed_words_workload_sampled():
    w = synth.MX
    a, b, ea, eb = synth.mx_operands(w)
    y = _gpu_mx_layouts(a, ea, b, eb, "col", "col")
    ms, ns = _sample(w.M, w.N, 5000, 6)
    ys, ss = oracle.gemm_mx32(a, ea, b, eb, at=(ms, ns))
    check(y[ms, ns], ys, ss, w.K, "mxfp8 8192^3, column-major packed words", cls="wide")
    assert not np.any(y == SENT)


def test_quant_g32_packed_words_feed_the_mx_gemm():
    """group_size 32 with UE8M0 scales in column-major packed words is the MX activation
    layout: quantize bf16 activations on the GPU, then run the MXFP8 GEMM on its outputs
    directly; the oracle chain is its quantization (row-major bytes) then its MX32 GEMM."""
    f = fq()
    M, N, K = 300, 520, 2048
    xb = synth.activations_bf16(74, M, K, outlier_p=0.01)
    b = synth.weight_codes(74, N, K, tensor_id=2)
    eb = synth.e8m0_exponents(74, N, K // 32, tensor_id=4)
    x = _dev(xb).view(torch.bfloat16)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sw = f.alloc_scales(None, M, K // 32, "ue8m0_packed", "col", "cuda")
    f.fp8q_group_quant(x, q, sw, 32)
    y = torch.full((M, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_gemm_blockscaled(q, sw, _dev(b), _dev(eb), y.view(torch.bfloat16), f.GEMM_MX32)
    torch.cuda.synchronize()
    qo, so = oracle.group_quant(xb, 32, oracle.SCALE_UE8M0, "row")
    assert np.array_equal(q.cpu().numpy(), qo)
    ys, ss = oracle.gemm_mx32(qo, so, b, eb)
    check(y.cpu().numpy().view(np.uint16), ys, ss, K, "quant G=32 packed -> MX32", cls="outlier")


# ----------------------------------------------------------------------------- API behaviour
def test_invalid_arguments_write_nothing():
    f = fq()
    a = torch.zeros((16, 256), dtype=torch.uint8, device="cuda")
    b = torch.zeros((32, 256), dtype=torch.uint8, device="cuda")
    sa = torch.ones((16, 2), dtype=torch.float32, device="cuda")
    sb = torch.ones((1, 2), dtype=torch.float32, device="cuda")
    y = torch.full((16, 32), SENT_I16, dtype=torch.int16, device="cuda")
    with pytest.raises(f.Fp8qError) as ei:  # MX32 needs E8M0 scales
        f.fp8q_gemm_blockscaled(a, sa, b, sb, y.view(torch.bfloat16), f.GEMM_MX32)
    assert ei.value.status == f.EUNSUPPORTED
    with pytest.raises(f.Fp8qError) as ei:  # K not a multiple of 128
        f.fp8q_gemm_blockscaled(a[:, :192], sa[:, :1], b[:, :192], sb[:, :1], y.view(torch.bfloat16))
    assert ei.value.status == f.EINVAL
    with pytest.raises(f.Fp8qError) as ei:  # misaligned a
        f.fp8q_gemm_blockscaled(a.view(-1)[8:8 + 15 * 256].view(15, 256), sa[:15], b, sb,
                                y[:15].view(torch.bfloat16))
    assert ei.value.status == f.EALIGN
    words = torch.zeros((32, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(f.Fp8qError) as ei:  # packed weight scales are an MX32 layout only
        f.fp8q_gemm_blockscaled(a, sa, b, words[:1], y.view(torch.bfloat16))
    assert ei.value.status == f.EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(y == SENT_I16)


def test_empty_gemm_is_noop():
    f = fq()
    y = torch.full((0, 128), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_gemm_blockscaled(torch.zeros((0, 128), dtype=torch.uint8, device="cuda"),
                            torch.ones((0, 1), dtype=torch.float32, device="cuda"),
                            torch.zeros((128, 128), dtype=torch.uint8, device="cuda"),
                            torch.ones((1, 1), dtype=torch.float32, device="cuda"), y.view(torch.bfloat16))
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- packed UE8M0
def _packed_words(sa_bytes, layout):
    """UE8M0 bytes [rows, K/128] -> device int32 words viewed as [rows, K/512] (row- or
    column-major storage)."""
    w = oracle.pack_ue8m0(sa_bytes)
    if layout == "row":
        return _dev(w)
    return _dev(np.ascontiguousarray(w.T)).t()


def _gpu_block_packed(a, sa_bytes, b, sb, layout):
    f = fq()
    M, K = a.shape
    N = b.shape[0]
    y = torch.full((M, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_gemm_blockscaled(_dev(a), _packed_words(sa_bytes, layout), _dev(b), _dev(sb), y.view(torch.bfloat16),
                            f.GEMM_BLOCK128)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


# Packed activation scales (four K blocks per word; K a multiple of 512) on every path: the
# small-M kernel (M <= 128) and the direct-to-LDS 256x128 kernel with ragged M, N (fp32
# weight scales folded, UE8M0 weight scales on the matrix core).
@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (100, 200, 1024), (130, 136, 512), (260, 300, 1024)])
@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("sb_kind", ["f32", "ue8m0"])
def test_packed_activation_scales_full(M, N, K, layout, sb_kind):
    w = synth.Workload("t", seed=80 + M, M=M, K=K, N=N, scale_fmt="ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sbf = synth.weights(w)
    sb = sbf if sb_kind == "f32" else synth.e8m0_exponents(8, sbf.shape[0], sbf.shape[1], tensor_id=78)
    y = _gpu_block_packed(a, sa, b, sb, layout)
    ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_UE8M0, "row", _fmt(sb))
    check(y, ys, ss, K, f"packed {M}x{N}x{K} {layout}")


def test_packed_activation_scales_wide_sampled():
    M, N, K = 4000, 4200, 1024
    w = synth.Workload("t", seed=90, M=M, K=K, N=N, scale_fmt="ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    y = _gpu_block_packed(a, sa, b, sb, "col")
    assert not np.any(y == SENT)
    g = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 127, 128, 255, 256, 3839, 3840, 3999], g.integers(0, M, 40)]))
    cols = np.unique(np.concatenate([[0, 63, 64, 255, 256, 4095, 4096, 4199], g.integers(0, N, 40)]))
    ms, ns = (v.ravel() for v in np.meshgrid(rows, cols, indexing="ij"))
    ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_UE8M0, "row", at=(ms, ns))
    check(y[ms, ns], ys, ss, K, "packed wide")


# The 128x256 kernel with fp32 (folded) or UE8M0 (matrix-core) weight scales; the expert
# offset into packed words counts 4 bytes per word
@pytest.mark.parametrize("sb_kind", ["f32", "ue8m0"])
def test_packed_activation_scales_masked(sb_kind):
    E, cap, N, K = 5, 200, 384, 512
    w = synth.Workload("m", seed=91, M=cap, K=K, N=N, E=E, scale_fmt="ue8m0", masked=True)
    ops = [synth.gemm_activation(w, e) + synth.weights(w, e) for e in range(E)]
    a, sa, b, sb = (np.stack([o[i] for o in ops]) for i in range(4))
    if sb_kind == "ue8m0":
        sb = synth.e8m0_exponents(10, E * sb.shape[1], sb.shape[2], tensor_id=80).reshape(sb.shape)
    words = oracle.pack_ue8m0(sa)  # [E, cap, K/512]
    sa_dev = _dev(np.ascontiguousarray(words.transpose(0, 2, 1))).transpose(1, 2)  # column-major per expert
    mm = np.array([0, 1, 200, 129, 128], dtype=np.int32)
    f = fq()
    y = torch.full((E, cap, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_grouped_gemm_masked(_dev(a), sa_dev, _dev(b), _dev(sb), y.view(torch.bfloat16), _dev(mm), 0)
    torch.cuda.synchronize()
    y = y.cpu().numpy().view(np.uint16)
    for e in range(E):
        r = mm[e]
        if r > 0:
            ys, ss = oracle.gemm_block128(a[e, :r], sa[e, :r], b[e], sb[e], oracle.SCALE_UE8M0, "row", _fmt(sb))
            check(y[e, :r], ys, ss, K, f"expert {e}")
        assert np.all(y[e, r:] == SENT), f"expert {e}: rows past masked_m written"


def test_moe_second_stage_sampled():
    """MoE second stage at full shape (the masked_moe_down workload's first 8 experts:
    capacity 512, gate|up 2x2048 -> K=2048, N=7168): the GPU quantizes with silu into packed
    UE8M0 words and feeds its own output to the masked GEMM. Expected values come from the
    oracle alone: its quantization of sampled rows (compared bit-exactly with the GPU's) and
    its GEMM of those rows on its own quantized operands."""
    w = synth.MASKED_DOWN
    E, cap, K, N, G = 8, w.M, w.K, w.N, w.G
    mm = synth.masked_rows(w.seed, w.E, cap)[:E]
    h = np.stack([synth.quant_input(w, e) for e in range(E)])  # [E, cap, 2K] bf16 bits
    f = fq()
    q = torch.full((E, cap, K), 0x5A, dtype=torch.uint8, device="cuda")
    sq = f.alloc_scales(E, cap, K // G, "ue8m0_packed", "col", "cuda")
    sq.fill_(0x5A5A5A5A)
    mmd = _dev(mm.astype(np.int32))
    f.fp8q_silu_mul_group_quant(_dev(h).view(torch.bfloat16), q, sq, G, masked_m=mmd, expected_m=cap // 2)
    wts = [synth.weights(w, e) for e in range(E)]
    wq = _dev(np.stack([t[0] for t in wts]))
    ws = _dev(np.stack([t[1] for t in wts]))
    y = torch.full((E, cap, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_grouped_gemm_masked(q, sq, wq, ws, y.view(torch.bfloat16), mmd, cap // 2)
    torch.cuda.synchronize()
    qg, wg, yg = q.cpu().numpy(), sq.cpu().numpy(), y.cpu().numpy().view(np.uint16)
    g = np.random.default_rng(12)
    got, want, size = [], [], []  # one compared set over all experts (as the other sampled tests)
    for e in range(E):
        r = int(mm[e])
        assert np.all(yg[e, r:] == SENT), f"expert {e}: rows past masked_m written"
        if r == 0:
            continue
        rows = np.unique(np.concatenate([[0, r - 1], g.integers(0, r, 6)]))
        qo, so = oracle.group_quant(h[e][rows], G, oracle.SCALE_UE8M0, "row", silu=True)
        assert np.array_equal(qg[e][rows], qo), f"expert {e}: codes"
        assert np.array_equal(wg[e][rows], oracle.pack_ue8m0(so)), f"expert {e}: packed scale words"
        cols = np.unique(np.concatenate([[0, 127, 128, N - 1], g.integers(0, N, 100)]))
        ms, ns = (v.ravel() for v in np.meshgrid(np.arange(rows.size), cols, indexing="ij"))
        ys, ss = oracle.gemm_block128(qo, so, wts[e][0], wts[e][1], oracle.SCALE_UE8M0, "row", at=(ms, ns))
        got.append(yg[e][rows][ms, ns]); want.append(ys); size.append(ss)
    check(np.concatenate(got), np.concatenate(want), np.concatenate(size), K, "moe second stage", cls="silu")


# ----------------------------------------------------------------------------- segments / contiguous
def _grouped_operands(T, N, K, W, seed, scale_fmt):
    w = synth.Workload("s", seed=seed, M=T, K=K, N=N, scale_fmt=scale_fmt)
    a, sa = synth.gemm_activation(w)
    ws = [synth.weights(w, e) for e in range(W)]
    return a, sa, np.stack([x[0] for x in ws]), np.stack([x[1] for x in ws])


def _sa_dev(sa, kind):
    """sa [T, K/128] (fp32 or UE8M0 bytes) stored as kind: '<fmt>-row' or '<fmt>-col', fmt
    f32, ue8m0 or packed (UE8M0 words of 4 K blocks)."""
    if kind.startswith("packed"):
        sa = oracle.pack_ue8m0(sa)
    return _dev(sa) if kind.endswith("row") else _dev(np.ascontiguousarray(sa.T)).t()


def _check_rows(yg, Y, S, K, what):
    done = ~np.isnan(Y[:, 0])
    assert np.all(yg[~done] == SENT), f"{what}: rows outside the computed ones were written"
    check(yg[done], Y[done], S[done], K, what)


# fp32 row scales with K % 512 == 0 take the 128x256 kernel with four-step scale groups, fp32
# column scales its per-step loads, packed words their per-step word loads (with either
# weight-scale format); UE8M0 bytes the register-staged kernel (segments start at any row).
@pytest.mark.parametrize("kind", ["f32-row", "f32-col", "packed-col", "packed-row", "ue8m0-col", "ue8m0-row"])
@pytest.mark.parametrize("sb_kind", ["f32", "ue8m0"])
def test_segments_full(kind, sb_kind):
    T, N, K, W = 720, 300, 1024, 3
    a, sa, b, sbf = _grouped_operands(T, N, K, W, 70, "f32" if kind.startswith("f32") else "ue8m0")
    sb = sbf if sb_kind == "f32" else synth.e8m0_exponents(9, W * sbf.shape[1], sbf.shape[2], tensor_id=79).reshape(sbf.shape)
    indptr = np.array([10, 110, 110, 380, 700], dtype=np.int32)  # gaps [0,10) and [700,720)
    weight = np.array([2, 0, 7, 1], dtype=np.int32)               # segment 2 uses no valid weight
    f = fq()
    y = torch.full((T, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_grouped_gemm_segments(_dev(a), _sa_dev(sa, kind), _dev(b), _dev(sb), y.view(torch.bfloat16),
                                 _dev(indptr), _dev(weight), expected_rows=600)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().view(np.uint16)
    Y, S = oracle.gemm_segments(a, sa, _fmt(sa), b, sb, indptr, weight, sb_fmt=_fmt(sb))
    _check_rows(yg, Y, S, K, f"segments {kind} sb {sb_kind}")


def _contiguous_indices():
    """640 rows in 5 blocks of 128: weight 1 (216 rows, then 40 padding), weight 0 (100 rows,
    one stray index 2 at row 300, padding), a padding block, weight 2 with a stray 1."""
    mi = np.full(640, -1, dtype=np.int32)
    mi[0:216] = 1
    mi[256:356] = 0
    mi[300] = 2
    mi[512:600] = 2
    mi[620] = 1
    return mi


@pytest.mark.parametrize("kind", ["f32-row", "ue8m0-col", "packed-col", "ue8m0-row"])
def test_contiguous_full(kind):
    T, N, K, W = 640, 300, 1024, 3
    a, sa, b, sb = _grouped_operands(T, N, K, W, 71, "f32" if kind.startswith("f32") else "ue8m0")
    mi = _contiguous_indices()
    f = fq()
    y = torch.full((T, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_grouped_gemm_contiguous(_dev(a), _sa_dev(sa, kind), _dev(b), _dev(sb), y.view(torch.bfloat16), _dev(mi))
    torch.cuda.synchronize()
    yg = y.cpu().numpy().view(np.uint16)
    Y, S = oracle.gemm_contiguous(a, sa, _fmt(sa), b, sb, mi)
    _check_rows(yg, Y, S, K, f"contiguous {kind}")


# The suite's packed-row MoE workloads at full expert shape (K=7168, N=4096) for the first 8
# experts of masked_moe with their row counts: each expert's rows placed at a 128-aligned
# offset with -1 padding (contiguous, UE8M0 column-major bytes) or back to back (segments,
# packed UE8M0 words). Sampled outputs of every expert are compared with the oracle run on
# that expert's own operands; padding rows must stay untouched.
def _moe_experts(n_exp):
    w = synth.MASKED
    mm = synth.masked_rows(w.seed, w.E, w.M)[:n_exp].astype(np.int64)
    mm[0] = 0  # an empty expert
    acts = [synth.gemm_activation(w, e) for e in range(n_exp)]
    wts = [synth.weights(w, e) for e in range(n_exp)]
    return w, mm, acts, wts


def _moe_samples(mm, N, seed):
    g = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([[0, 127, 128, 255, 256, N - 1], g.integers(0, N, 58)]))
    out = []
    for e, r in enumerate(mm):
        if r == 0:
            continue
        rows = np.unique(np.concatenate([[0, r - 1], g.integers(0, r, 3)]))
        ms, ns = (v.ravel() for v in np.meshgrid(rows, cols, indexing="ij"))
        out.append((e, ms, ns))
    return out


@pytest.mark.parametrize("layout", ["contiguous", "segments"])
def test_moe_packed_rows_workload_sampled(layout):
    f = fq()
    n_exp = 8
    w, mm, acts, wts = _moe_experts(n_exp)
    K, N = w.K, w.N
    if layout == "contiguous":
        offs = np.concatenate([[0], np.cumsum((mm + 127) // 128 * 128)])
    else:
        offs = np.concatenate([[0], np.cumsum(mm)])
    T = int(offs[-1])
    A = np.zeros((T, K), dtype=np.uint8)
    SA = np.zeros((T, K // 128), dtype=np.uint8)
    mi = np.full(T, -1, dtype=np.int32)
    for e in range(n_exp):
        r, o = int(mm[e]), int(offs[e])
        A[o:o + r] = acts[e][0][:r]
        SA[o:o + r] = acts[e][1][:r]
        mi[o:o + r] = e
    B = np.stack([x[0] for x in wts])
    SB = np.stack([x[1] for x in wts])
    y = torch.full((T, N), SENT_I16, dtype=torch.int16, device="cuda")
    if layout == "contiguous":
        f.fp8q_grouped_gemm_contiguous(_dev(A), _dev(np.ascontiguousarray(SA.T)).t(), _dev(B), _dev(SB),
                                       y.view(torch.bfloat16), _dev(mi))
    else:
        f.fp8q_grouped_gemm_segments(_dev(A), _dev(oracle.pack_ue8m0(SA)), _dev(B), _dev(SB), y.view(torch.bfloat16),
                                     _dev(offs.astype(np.int32)), expected_rows=T)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().view(np.uint16)
    y_all, ys_all, s_all = [], [], []
    for e, ms, ns in _moe_samples(mm, N, 11):
        a_e, sa_e = acts[e]
        ys, ss = oracle.gemm_block128(a_e, sa_e, wts[e][0], wts[e][1], oracle.SCALE_UE8M0, "row", at=(ms, ns))
        y_all.append(yg[int(offs[e]) + ms, ns]); ys_all.append(ys); s_all.append(ss)
    check(np.concatenate(y_all), np.concatenate(ys_all), np.concatenate(s_all), K, f"{layout} moe experts")
    if layout == "contiguous":
        assert np.all(yg[mi < 0] == SENT), "padding rows were written"


@pytest.mark.parametrize("kind", ["ue8m0-col", "packed-col", "packed-row"])
def test_contiguous_ue8m0_weight_scales(kind):
    T, N, K, W = 640, 300, 1024, 3
    a, sa, b, sbf = _grouped_operands(T, N, K, W, 72, "ue8m0")
    sb = synth.e8m0_exponents(72, W * sbf.shape[1], sbf.shape[2], lo=-4, hi=4, tensor_id=96).reshape(sbf.shape)
    mi = _contiguous_indices()
    f = fq()
    y = torch.full((T, N), SENT_I16, dtype=torch.int16, device="cuda")
    f.fp8q_grouped_gemm_contiguous(_dev(a), _sa_dev(sa, kind), _dev(b), _dev(sb), y.view(torch.bfloat16),
                                   _dev(mi))
    torch.cuda.synchronize()
    yg = y.cpu().numpy().view(np.uint16)
    Y, S = oracle.gemm_contiguous(a, sa, oracle.SCALE_UE8M0, b, sb, mi, sb_fmt=oracle.SCALE_UE8M0)
    _check_rows(yg, Y, S, K, f"contiguous {kind}, UE8M0 weight scales")
    # a weight stride of the UE8M0 scales that is not a whole number of words is refused
    Wn, nb, kb = sb.shape
    store = torch.zeros(Wn * (nb * kb + 2), dtype=torch.uint8, device="cuda")
    sb_odd = store.as_strided((Wn, nb, kb), (nb * kb + 2, kb, 1))
    y2 = torch.full((T, N), SENT_I16, dtype=torch.int16, device="cuda")
    with pytest.raises(f.Fp8qError) as ei:
        f.fp8q_grouped_gemm_contiguous(_dev(a), _sa_dev(sa, kind), _dev(b), sb_odd, y2.view(torch.bfloat16),
                                       _dev(mi))
    assert ei.value.status == f.EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(y2 == SENT_I16)


def test_contiguous_unsupported_scale_layout_writes_nothing():
    T, N, K, W = 256, 128, 640, 2
    a, sa, b, sb = _grouped_operands(T, N, K, W, 72, "ue8m0")
    f = fq()
    y = torch.full((T, N), SENT_I16, dtype=torch.int16, device="cuda")
    # UE8M0 bytes row-major in rows of 5 bytes (K % 512 != 0): not moved by the 128-row kernel
    with pytest.raises(f.Fp8qError) as ei:
        f.fp8q_grouped_gemm_contiguous(_dev(a), _sa_dev(sa, "ue8m0-row"), _dev(b), _dev(sb), y.view(torch.bfloat16),
                                       _dev(np.zeros(T, dtype=np.int32)))
    assert ei.value.status == f.EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(y == SENT_I16)

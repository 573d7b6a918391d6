"""CPU oracle for per-token-group FP8 quantization and block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path. It shares no code with the HIP library.

The arithmetic lives in plain C (fp8q_oracle.c, built by build.py with IEEE semantics);
this module only marshals numpy arrays into it. The C loops over rows and output elements
run on all host cores (OpenMP; `threads(n)` limits them); each row or output is computed
whole by one thread, so results do not depend on the thread count. Function-level citations are in the C
source; the arguments mirror the C ABI declared in include/fp8q.h, with host arrays in
place of device pointers.

Parity status of each function (what pins it is in tests/test_oracle_*.py):
  e4m3_decode, e4m3_encode  pinned: all 256 codes and a 2^24-value sweep vs torch's cast,
                            hand-derived golden codes
  ue8m0_byte                pinned: exact rational ceil-power-of-two over every bf16 amax
  exp_spec, silu_mul        pinned: accuracy vs math.exp (<= 2 ulp), special values
  group_quant               pinned: golden group, dequant-error bound, layout/mask invariants;
                            per-token (G = K) and int8 output: brute-force rows in plain
                            Python/fractions, the int8 dequant bound
  int8_encode               pinned: hand-written ties, numpy's rint over a dense sweep
  gemm                      pinned: exact Fraction arithmetic, torch float64 dequant-matmul,
                            one-hot operands
  gemm_segments,            compositions of gemm_block128 over row slices (the plain definition);
  gemm_contiguous           pinned: hand-derived row coverage, equality with whole-matrix calls
  pack_ue8m0, unpack_ue8m0  layout only (no arithmetic); pinned: hand-written words of known
                            bytes, round trip
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libfp8q_oracle.so")

BF16, F16, F32 = 0, 1, 2
SCALE_F32, SCALE_UE8M0, SCALE_UE8M0_PACKED = 0, 1, 2
GEMM_BLOCK128, GEMM_MX32 = 0, 1

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.ora_group_quant.restype = ctypes.c_int
    lib.ora_group_quant.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64,
                                    _P, ctypes.c_int, _I64, _I64, _I64, _I64, _P, ctypes.c_int,
                                    ctypes.c_int, _P, _P, _I64]
    lib.ora_gemm.restype = ctypes.c_int
    lib.ora_gemm.argtypes = [_P, _I64, _P, ctypes.c_int, _I64, _I64, _P, _I64, _P, ctypes.c_int,
                             _I64, _I64, _I64, _I64, _I64, ctypes.c_int, _P, _P, _I64, _P, _P]
    for name in ("ora_e4m3_decode_array", "ora_e4m3_encode_array", "ora_ue8m0_byte_array",
                 "ora_exp_spec_array", "ora_int8_encode_array"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [_P, _P, _I64]
    lib.ora_silu_mul_array.restype = None
    lib.ora_silu_mul_array.argtypes = [_P, _P, _P, _I64]
    lib.ora_set_threads.restype = None
    lib.ora_set_threads.argtypes = [ctypes.c_int]
    lib.ora_max_threads.restype = ctypes.c_int
    lib.ora_max_threads.argtypes = []
    _lib = lib
    return lib


def set_threads(n: int) -> None:
    """Threads of the oracle's loops over rows / output elements (results do not depend
    on it: every row or output is computed whole by one thread)."""
    _load().ora_set_threads(int(n))


def max_threads() -> int:
    return int(_load().ora_max_threads())


class threads:
    """Context manager: run the oracle with n threads, then restore the previous count."""

    def __init__(self, n: int):
        self.n = n

    def __enter__(self):
        self.prev = max_threads()
        set_threads(self.n)
        return self

    def __exit__(self, *exc):
        set_threads(self.prev)
        return False


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------- codecs
def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().ora_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_encode(values) -> np.ndarray:
    """Nearest e4m3 code (ties to even) of fp32 values already within [-448, 448]."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().ora_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def int8_encode(values) -> np.ndarray:
    """Nearest integer (ties to even) of fp32 values already within [-127, 127], as int8."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.int8)
    _load().ora_int8_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def ue8m0_byte(amax) -> np.ndarray:
    v = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().ora_ue8m0_byte_array(_ptr(v), _ptr(out), v.size)
    return out


def exp_spec(t) -> np.ndarray:
    v = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.float32)
    _load().ora_exp_spec_array(_ptr(v), _ptr(out), v.size)
    return out


def silu_mul(g, u) -> np.ndarray:
    gv = np.ascontiguousarray(g, dtype=np.float32)
    uv = np.ascontiguousarray(u, dtype=np.float32)
    assert gv.shape == uv.shape
    out = np.empty(gv.shape, dtype=np.float32)
    _load().ora_silu_mul_array(_ptr(gv), _ptr(uv), _ptr(out), gv.size)
    return out


# --------------------------------------------------------------------------- quant
def group_quant_raw(x: np.ndarray, in_dtype: int, E: int, M: int, K: int, x_se: int, x_sm: int,
                    q: np.ndarray, q_se: int, q_sm: int, s: np.ndarray, scale_fmt: int,
                    s_se: int, s_sm: int, s_sg: int, group_size: int,
                    masked_m: np.ndarray | None = None, silu: bool = False,
                    rows: tuple[np.ndarray, np.ndarray] | None = None,
                    out_int8: bool = False) -> None:
    """Same arguments as fp8q_group_quant (strides in elements), on host arrays; with
    out_int8 those of fp8q_group_quant_int8. group_size == K is per-token quantization.
    `rows` = (e_indices, m_indices) restricts the work to those rows."""
    mm = None if masked_m is None else np.ascontiguousarray(masked_m, dtype=np.int32)
    re = rm = None
    n_rows = 0
    if rows is not None:
        re = np.ascontiguousarray(rows[0], dtype=np.int64)
        rm = np.ascontiguousarray(rows[1], dtype=np.int64)
        n_rows = re.size
    rc = _load().ora_group_quant(_ptr(x), in_dtype, E, M, K, x_se, x_sm, _ptr(q), q_se, q_sm,
                                 _ptr(s), scale_fmt, s_se, s_sm, s_sg, group_size, _ptr(mm),
                                 int(silu), int(out_int8), _ptr(re), _ptr(rm), n_rows)
    if rc != 0:
        raise ValueError("oracle group_quant: unsupported arguments")


def group_quant(x: np.ndarray, group_size: int, scale_fmt: int, layout: str = "row",
                in_dtype: int = BF16, silu: bool = False, masked_m: np.ndarray | None = None,
                rows: tuple[np.ndarray, np.ndarray] | None = None,
                fill: int = 0, out_int8: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """Quantizes x ([M, K] or [E, M, K]; with silu the last dim is 2K) into freshly
    allocated outputs: q [.., M, K] uint8 (e4m3 bytes; int8 with out_int8) and scales
    [.., M, K/G] (layout "row") or [.., K/G, M] (layout "col"), float32 or uint8.
    group_size == K gives per-token scales [.., M, 1]. Untouched entries hold `fill`."""
    x3 = x if x.ndim == 3 else x[None]
    E, M, W = x3.shape
    K = W // 2 if silu else W
    ng = K // group_size
    x3 = np.ascontiguousarray(x3)
    q = np.full((E, M, K), fill, dtype=np.uint8)
    width = 4 if scale_fmt == SCALE_F32 else 1
    if layout == "row":
        s = np.full((E, M, ng * width), fill, dtype=np.uint8)
        s_sm, s_sg = ng, 1
    else:
        s = np.full((E, ng, M * width), fill, dtype=np.uint8)
        s_sm, s_sg = 1, M
    if scale_fmt == SCALE_F32:
        s = s.view(np.float32)
    group_quant_raw(x3, in_dtype, E, M, K, M * W, W, q, M * K, K, s, scale_fmt, M * ng, s_sm, s_sg,
                    group_size, masked_m, silu, rows, out_int8)
    if out_int8:
        q = q.view(np.int8)
    if x.ndim == 2:
        return q[0], s[0]
    return q, s


def pack_ue8m0(s: np.ndarray) -> np.ndarray:
    """UE8M0 bytes [.., rows, ng] (ng a multiple of 4) -> int32 words [.., rows, ng / 4].
    Group g of a row becomes byte g % 4 of word g / 4, counting bytes from the least
    significant: the four-groups-per-word layout that the `aligned` trait enables
    ([PR30924] 实现拆解 1; UE8M0 only, number of groups a multiple of 4)."""
    b = np.asarray(s, dtype=np.uint8).astype(np.uint32)
    if b.shape[-1] % 4:
        raise ValueError("packed UE8M0 needs a multiple of 4 groups per row")
    w = b[..., 0::4] | (b[..., 1::4] << 8) | (b[..., 2::4] << 16) | (b[..., 3::4] << 24)
    return w.astype(np.uint32).view(np.int32)


def unpack_ue8m0(w: np.ndarray) -> np.ndarray:
    """Inverse of pack_ue8m0: int32 words [.., rows, n] -> UE8M0 bytes [.., rows, 4 n]."""
    u = np.asarray(w).astype(np.int64) & 0xFFFFFFFF
    out = np.empty(u.shape[:-1] + (4 * u.shape[-1],), dtype=np.uint8)
    for i in range(4):
        out[..., i::4] = (u >> (8 * i)) & 0xFF
    return out


# --------------------------------------------------------------------------- gemm
def gemm_raw(a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, M, N, K, mode,
             at: tuple[np.ndarray, np.ndarray] | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Same arguments as fp8q_gemm_blockscaled (without y), on host arrays. Returns
    (Y*, S): the fp64 dequantize-then-multiply result and the sum of |terms|, either for
    all [M, N] elements or for the (m, n) pairs in `at`."""
    if at is not None:
        ms = np.ascontiguousarray(at[0], dtype=np.int64)
        ns = np.ascontiguousarray(at[1], dtype=np.int64)
        y = np.empty(ms.size, dtype=np.float64)
        s = np.empty(ms.size, dtype=np.float64)
        cnt = ms.size
    else:
        ms = ns = None
        y = np.empty((M, N), dtype=np.float64)
        s = np.empty((M, N), dtype=np.float64)
        cnt = 0
    rc = _load().ora_gemm(_ptr(a), lda, _ptr(sa), sa_fmt, sa_sm, sa_sk, _ptr(b), ldb, _ptr(sb),
                          sb_fmt, sb_sn, sb_sk, M, N, K, mode, _ptr(ms), _ptr(ns), cnt,
                          _ptr(y), _ptr(s))
    if rc != 0:
        raise ValueError("oracle gemm: unsupported arguments")
    return y, s


def gemm_block128(a: np.ndarray, sa: np.ndarray, b: np.ndarray, sb: np.ndarray, sa_fmt: int,
                  sa_layout: str = "row", sb_fmt: int = SCALE_F32,
                  at: tuple[np.ndarray, np.ndarray] | None = None):
    """a [M, K] codes; sa [M, K/128] ("row") or [K/128, M] ("col"); b [N, K] codes;
    sb [ceil(N/128), K/128]."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    sa = np.ascontiguousarray(sa)
    sb = np.ascontiguousarray(sb)
    for arr, fmt in ((sa, sa_fmt), (sb, sb_fmt)):
        if arr.dtype != (np.float32 if fmt == SCALE_F32 else np.uint8):
            raise ValueError("scale array dtype does not match its format")
    M, K = a.shape
    N = b.shape[0]
    kb = K // 128
    sa_sm, sa_sk = (kb, 1) if sa_layout == "row" else (1, M)
    return gemm_raw(a, K, sa, sa_fmt, sa_sm, sa_sk, b, K, sb, sb_fmt, kb, 1, M, N, K,
                    GEMM_BLOCK128, at)


def _rows_of(sa: np.ndarray, lo: int, hi: int, sa_layout: str) -> np.ndarray:
    return sa[lo:hi] if sa_layout == "row" else sa[:, lo:hi]


def gemm_segments(a: np.ndarray, sa: np.ndarray, sa_fmt: int, b: np.ndarray, sb: np.ndarray,
                  seg_indptr, seg_weight=None, sa_layout: str = "row", sb_fmt: int = SCALE_F32):
    """SegmentGEMM over packed rows ([FI] section 7: ragged segments of x mapped by seg_indptr,
    each against one of several weights): rows [seg_indptr[s], seg_indptr[s+1]) of a [T, K]
    (ends clamped to [0, T]; an end below its start is an empty segment) times weight
    w = seg_weight[s] (default s) of b [W, N, K] with scales sb [W, N/128, K/128]; a segment
    whose w is outside [0, W) is skipped. sa is [T, K/128] ("row") or [K/128, T] ("col").
    Returns (Y [T, N], S [T, N]) in fp64 as gemm_block128 does, NaN in rows no segment computes."""
    T, N, W = a.shape[0], b.shape[1], b.shape[0]
    Y = np.full((T, N), np.nan)
    S = np.full((T, N), np.nan)
    for s in range(len(seg_indptr) - 1):
        lo = min(max(int(seg_indptr[s]), 0), T)
        hi = min(int(seg_indptr[s + 1]), T)
        w = s if seg_weight is None else int(seg_weight[s])
        if hi <= lo or not 0 <= w < W:
            continue
        Y[lo:hi], S[lo:hi] = gemm_block128(a[lo:hi], _rows_of(sa, lo, hi, sa_layout), b[w], sb[w], sa_fmt,
                                           sa_layout, sb_fmt)
    return Y, S


def gemm_contiguous(a: np.ndarray, sa: np.ndarray, sa_fmt: int, b: np.ndarray, sb: np.ndarray,
                    m_indices, sa_layout: str = "row", block: int = 128, sb_fmt: int = SCALE_F32):
    """Grouped contiguous layout ([FI] section 7: DeepGEMM packed tokens + m_indices): rows are
    taken in aligned blocks of `block`; a block whose first row holds weight index e in
    [0, W) computes its rows t with m_indices[t] == e against weight e; every other row is
    left out (NaN). Operands as in gemm_segments."""
    T, N, W = a.shape[0], b.shape[1], b.shape[0]
    Y = np.full((T, N), np.nan)
    S = np.full((T, N), np.nan)
    mi = np.asarray(m_indices)
    for b0 in range(0, T, block):
        e = int(mi[b0])
        if not 0 <= e < W:
            continue
        rows = b0 + np.nonzero(mi[b0:b0 + block] == e)[0]
        sar = sa[rows] if sa_layout == "row" else sa[:, rows]
        Y[rows], S[rows] = gemm_block128(a[rows], sar, b[e], sb[e], sa_fmt, sa_layout, sb_fmt)
    return Y, S


def gemm_mx32(a: np.ndarray, ea: np.ndarray, b: np.ndarray, eb: np.ndarray,
              at: tuple[np.ndarray, np.ndarray] | None = None):
    """a [M, K], b [N, K] codes; ea [M, K/32], eb [N, K/32] E8M0 bytes (row-major)."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    ea = np.ascontiguousarray(ea)
    eb = np.ascontiguousarray(eb)
    M, K = a.shape
    N = b.shape[0]
    return gemm_raw(a, K, ea, SCALE_UE8M0, K // 32, 1, b, K, eb, SCALE_UE8M0, K // 32, 1, M, N, K,
                    GEMM_MX32, at)

"""Python binding of libfp8q.so: per-token-group FP8 quantization and block-scaled FP8
GEMMs for AMD Instinct MI355X (gfx950).

This module only marshals torch tensors (device memory, strides, the current HIP
stream) into the C ABI declared in include/fp8q.h; every step of the computation runs
in the library's HIP kernels. The functions named fp8q_* mirror the C entry points one
to one and write into caller-allocated tensors; group_quant() additionally allocates
its outputs (the role of _allocate_outputs in the sglang PR #30924 design, prhub
report section "实现拆解" item 2).

There is no fallback: if libfp8q.so is missing or the device is not a gfx950, calls
raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8q.so")

# constants of include/fp8q.h
OK, EINVAL, EUNSUPPORTED, EALIGN, EDEVICE, ELAUNCH = 0, 1, 2, 3, 4, 5
DTYPE_BF16, DTYPE_F16, DTYPE_F32 = 0, 1, 2
SCALE_F32, SCALE_UE8M0, SCALE_UE8M0_PACKED = 0, 1, 2
GEMM_BLOCK128, GEMM_MX32 = 0, 1

_DTYPES = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16, torch.float32: DTYPE_F32}
_SCALE_FMT = {"f32": SCALE_F32, "ue8m0": SCALE_UE8M0, "ue8m0_packed": SCALE_UE8M0_PACKED}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int

_SIGNATURES = {
    "fp8q_group_quant": [_P, _INT, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P, _INT, _I64, _I64,
                         _I64, _INT, _P, _I64, _P],
    "fp8q_silu_mul_group_quant": [_P, _INT, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P, _INT, _I64,
                                  _I64, _I64, _INT, _P, _I64, _P],
    "fp8q_group_quant_int8": [_P, _INT, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P, _INT, _I64,
                              _I64, _I64, _INT, _P, _I64, _P],
    "fp8q_gemm_blockscaled": [_P, _I64, _P, _INT, _I64, _I64, _P, _I64, _P, _INT, _I64, _I64, _P, _I64,
                              _I64, _I64, _I64, _INT, _P],
    "fp8q_gemm_blockscaled_ws": [_P, _I64, _P, _INT, _I64, _I64, _P, _I64, _P, _INT, _I64, _I64, _P, _I64,
                                 _I64, _I64, _I64, _INT, _P, _I64, _P],
    "fp8q_gemm_workspace_size": [_I64, _I64, _I64, _INT],
    "fp8q_gemm_blockscaled_noalloc": [_P, _I64, _P, _INT, _I64, _I64, _P, _I64, _P, _INT, _I64, _I64, _P, _I64,
                                      _I64, _I64, _I64, _INT, _P],
    "fp8q_grouped_gemm_masked": [_P, _I64, _I64, _P, _INT, _I64, _I64, _I64, _P, _I64, _I64, _P, _INT,
                                 _I64, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _I64, _I64, _I64, _P],
    "fp8q_grouped_gemm_segments": [_P, _I64, _P, _INT, _I64, _I64, _P, _I64, _I64, _P, _INT, _I64, _I64, _I64,
                                   _P, _I64, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P],
    "fp8q_grouped_gemm_contiguous": [_P, _I64, _P, _INT, _I64, _I64, _P, _I64, _I64, _P, _INT, _I64, _I64, _I64,
                                     _P, _I64, _P, _I64, _I64, _I64, _I64, _P],
    "fp8q_status_string": [_INT],
    "fp8q_last_error": [],
    "fp8q_device_check": [_INT],
}


class Fp8qError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} [{_status_string(status)}]")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libfp8q.so (built by fp8_group_quant_amd/build.py). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run fp8_group_quant_amd/build.py (there is no fallback)")
    lib = ctypes.CDLL(path)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name, None)
        if fn is None:  # calling it later raises AttributeError; tests check every export
            continue
        fn.argtypes = args
        fn.restype = (ctypes.c_char_p if name in ("fp8q_status_string", "fp8q_last_error")
                      else _I64 if name == "fp8q_gemm_workspace_size" else _INT)
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    return load_library().fp8q_status_string(status).decode()


def _check(status: int) -> None:
    if status != OK:
        raise Fp8qError(status, load_library().fp8q_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _as3(t: torch.Tensor) -> tuple[int, int, int, int, int]:
    """(E, M, W, stride_e, stride_m) of a [M, W] or [E, M, W] tensor with unit inner stride."""
    if t.dim() == 2:
        if t.size(1) > 1 and t.stride(1) != 1:
            raise ValueError("innermost dimension must be contiguous")
        return 1, t.size(0), t.size(1), t.size(0) * t.stride(0), t.stride(0)
    if t.dim() == 3:
        if t.size(2) > 1 and t.stride(2) != 1:
            raise ValueError("innermost dimension must be contiguous")
        return t.size(0), t.size(1), t.size(2), t.stride(0), t.stride(1)
    raise ValueError("expected a 2-D or 3-D tensor")


def _scale_strides(s: torch.Tensor) -> tuple[int, int, int]:
    """(s_se, s_sm, s_sg) of the logical [M, ng] or [E, M, ng] scale view."""
    if s.dim() == 2:
        return 0, s.stride(0), s.stride(1)
    if s.dim() == 3:
        return s.stride(0), s.stride(1), s.stride(2)
    raise ValueError("expected a 2-D or 3-D scale view")


def _scale_fmt_of(s: torch.Tensor) -> int:
    if s.dtype == torch.float32:
        return SCALE_F32
    if s.dtype == torch.uint8:
        return SCALE_UE8M0
    if s.dtype == torch.int32:
        return SCALE_UE8M0_PACKED
    raise ValueError("scales must be float32 (fp32 scales), uint8 (UE8M0 bytes) or int32 "
                     "(UE8M0 bytes packed 4 groups per word)")


# ------------------------------------------------------------------------------ quant
def _quant(entry: str, x, q, s, group_size, masked_m, expected_m, stream, silu):
    E, M, W, x_se, x_sm = _as3(x)
    K = W // 2 if silu else W
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    qE, qM, qK, q_se, q_sm = _as3(q.view(torch.uint8))
    if (qE, qM, qK) != (E, M, K):
        raise ValueError(f"q has shape {tuple(q.shape)}, expected {(E, M, K) if x.dim() == 3 else (M, K)}")
    s_se, s_sm, s_sg = _scale_strides(s)
    mm = None
    if masked_m is not None:
        if masked_m.dtype != torch.int32 or masked_m.numel() != E or not masked_m.is_cuda:
            raise ValueError("masked_m must be a device int32 tensor with one entry per expert")
        mm = masked_m
    fn = getattr(load_library(), entry)
    _check(fn(_ptr(x), _DTYPES[x.dtype], E, M, K, x_se, x_sm, _ptr(q), q_se, q_sm, _ptr(s),
              _scale_fmt_of(s), s_se, s_sm, s_sg, group_size, _ptr(mm), int(expected_m),
              _stream(stream)))


def fp8q_group_quant(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, group_size: int = 128,
                     masked_m: torch.Tensor | None = None, expected_m: int = 0, stream=None) -> None:
    """x [M, K] or [E, M, K] (bf16/f16/f32) -> q (uint8 or float8_e4m3fn, same shape) and
    s: a [.., M, K/G] view (float32 = fp32 scales, uint8 = UE8M0); its strides choose the
    row- or column-major layout. group_size == K is per-token quantization (s [.., M, 1])."""
    _quant("fp8q_group_quant", x, q, s, group_size, masked_m, expected_m, stream, False)


def fp8q_group_quant_int8(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, group_size: int = 128,
                          masked_m: torch.Tensor | None = None, expected_m: int = 0, stream=None) -> None:
    """As fp8q_group_quant with int8 codes in q (torch.int8) and float32 scales
    s = amax / 127."""
    if q.dtype != torch.int8:
        raise ValueError("q must be an int8 tensor")
    if s.dtype != torch.float32:
        raise ValueError("int8 output takes float32 scales")
    _quant("fp8q_group_quant_int8", x, q, s, group_size, masked_m, expected_m, stream, False)


def fp8q_silu_mul_group_quant(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, group_size: int = 128,
                              masked_m: torch.Tensor | None = None, expected_m: int = 0,
                              stream=None) -> None:
    """As fp8q_group_quant, with x [.., M, 2K] = gate | up and silu(gate) * up quantized."""
    _quant("fp8q_silu_mul_group_quant", x, q, s, group_size, masked_m, expected_m, stream, True)


def alloc_scales(E: int | None, M: int, ng: int, scale_fmt: str, layout: str, device) -> torch.Tensor:
    """Scale tensor viewed as [.., M, ng]: row-major storage, or column-major storage
    [.., ng, M] returned transposed (the strides carry the layout). "ue8m0_packed" returns
    int32 words of 4 groups each, viewed as [.., M, ng / 4]."""
    dt = {"f32": torch.float32, "ue8m0": torch.uint8, "ue8m0_packed": torch.int32}[scale_fmt]
    if scale_fmt == "ue8m0_packed":
        if ng % 4:
            raise ValueError("packed UE8M0 scales need a multiple of 4 groups per row")
        ng //= 4
    lead = () if E is None else (E,)
    if layout == "row":
        return torch.empty(*lead, M, ng, dtype=dt, device=device)
    return torch.empty(*lead, ng, M, dtype=dt, device=device).transpose(-1, -2)


def group_quant(x: torch.Tensor, group_size: int = 128, scale_fmt: str = "ue8m0", layout: str = "col",
                silu: bool = False, masked_m: torch.Tensor | None = None, expected_m: int = 0,
                stream=None, int8: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Allocating form: returns (q uint8 [.., M, K] of e4m3 bytes, or int8 codes with
    int8=True (fp32 scales), scales viewed as [.., M, K/G]). group_size == K is per-token."""
    W = x.shape[-1]
    K = W // 2 if silu else W
    lead = tuple(x.shape[:-2])
    M = x.shape[-2]
    q = torch.empty(*lead, M, K, dtype=torch.int8 if int8 else torch.uint8, device=x.device)
    s = alloc_scales(lead[0] if lead else None, M, K // group_size, scale_fmt, layout, x.device)
    if int8:
        if silu:
            raise ValueError("int8 output has no fused silu variant")
        fp8q_group_quant_int8(x, q, s, group_size, masked_m, expected_m, stream)
    elif silu:
        fp8q_silu_mul_group_quant(x, q, s, group_size, masked_m, expected_m, stream)
    else:
        fp8q_group_quant(x, q, s, group_size, masked_m, expected_m, stream)
    return q, s


# ------------------------------------------------------------------------------ GEMM
def _u8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


_WS_SIZES: dict = {}


def fp8q_gemm_workspace_size(M: int, N: int, K: int, mode: int = GEMM_BLOCK128) -> int:
    """Bytes of workspace with which fp8q_gemm_blockscaled_ws takes its split-K path for this
    shape on the current device (0: none needed)."""
    key = (torch.cuda.current_device(), M, N, K, mode)
    if key not in _WS_SIZES:
        _WS_SIZES[key] = int(load_library().fp8q_gemm_workspace_size(M, N, K, mode))
    return _WS_SIZES[key]


def fp8q_gemm_blockscaled(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                          y: torch.Tensor, mode: int = GEMM_BLOCK128, stream=None,
                          workspace: torch.Tensor | None = None) -> None:
    """Y[M, N] (bf16) = dequant(a [M, K]) @ dequant(b [N, K])^T.
    BLOCK128: sa viewed as [M, K/128], sb as [ceil(N/128), K/128] (float32 or uint8 UE8M0;
    sa may be int32 packed UE8M0 words [M, K/512]).
    MX32: sa [M, K/32], sb [N, K/32], uint8 E8M0; or either as int32 packed words [rows, K/128]
    (the four E8M0 bytes of one 128-wide K step per word; a [K/128, rows] storage viewed
    transposed gives the column-major words that load fastest).
    Calls fp8q_gemm_blockscaled_ws: when the shape can use a workspace and none is given, one
    is taken from torch's allocator on a's device (stream-ordered, capturable)."""
    a8, b8 = _u8(a), _u8(b)
    M, K = a8.shape
    N = b8.shape[0]
    if b8.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError("shape mismatch")
    if a8.stride(1) != 1 or b8.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("innermost dimensions must be contiguous")
    if workspace is None and mode == GEMM_BLOCK128:
        nbytes = fp8q_gemm_workspace_size(M, N, K, mode)
        if nbytes > 0:
            # allocated on the stream the kernels run on, so that the caching allocator hands
            # the block to no other stream's work before they finish
            if stream is None:
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=a8.device)
            else:
                st = stream if isinstance(stream, torch.cuda.Stream) else \
                    torch.cuda.ExternalStream(int(stream), device=a8.device)
                with torch.cuda.stream(st):
                    workspace = torch.empty(nbytes, dtype=torch.uint8, device=a8.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().fp8q_gemm_blockscaled_ws(
        _ptr(a8), a8.stride(0), _ptr(sa), _scale_fmt_of(sa), sa.stride(0), sa.stride(1),
        _ptr(b8), b8.stride(0), _ptr(sb), _scale_fmt_of(sb), sb.stride(0), sb.stride(1),
        _ptr(y), y.stride(0), M, N, K, mode, ws_ptr, ws_bytes, _stream(stream)))


def fp8q_gemm_blockscaled_noalloc(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                                  y: torch.Tensor, mode: int = GEMM_BLOCK128, stream=None) -> None:
    """fp8q_gemm_blockscaled with the split-K partial sums in the library's own device array
    (no allocation anywhere; calls that overlap on one device race on that array)."""
    a8, b8 = _u8(a), _u8(b)
    M, K = a8.shape
    N = b8.shape[0]
    if b8.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError("shape mismatch")
    if a8.stride(1) != 1 or b8.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("innermost dimensions must be contiguous")
    _check(load_library().fp8q_gemm_blockscaled_noalloc(
        _ptr(a8), a8.stride(0), _ptr(sa), _scale_fmt_of(sa), sa.stride(0), sa.stride(1),
        _ptr(b8), b8.stride(0), _ptr(sb), _scale_fmt_of(sb), sb.stride(0), sb.stride(1),
        _ptr(y), y.stride(0), M, N, K, mode, _stream(stream)))


def fp8q_grouped_gemm_masked(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                             y: torch.Tensor, masked_m: torch.Tensor, expected_m: int = 0,
                             stream=None) -> None:
    """Per expert e: Y[e, :masked_m[e]] = BLOCK128 product of a[e] [cap, K] and b[e] [N, K].
    sa viewed as [E, cap, K/128]; sb as [E, ceil(N/128), K/128]; y [E, cap, N] bf16."""
    a8, b8 = _u8(a), _u8(b)
    E, cap, K = a8.shape
    N = b8.shape[1]
    if b8.shape[0] != E or b8.shape[2] != K or tuple(y.shape) != (E, cap, N):
        raise ValueError("shape mismatch")
    if masked_m.dtype != torch.int32 or masked_m.numel() != E or not masked_m.is_cuda:
        raise ValueError("masked_m must be a device int32 tensor with one entry per expert")
    _check(load_library().fp8q_grouped_gemm_masked(
        _ptr(a8), a8.stride(0), a8.stride(1), _ptr(sa), _scale_fmt_of(sa), sa.stride(0), sa.stride(1),
        sa.stride(2), _ptr(b8), b8.stride(0), b8.stride(1), _ptr(sb), _scale_fmt_of(sb), sb.stride(0),
        sb.stride(1), sb.stride(2), _ptr(y), y.stride(0), y.stride(1), _ptr(masked_m), int(expected_m),
        E, cap, N, K, _stream(stream)))


def _packed_rows_operands(a, sa, b, sb, y):
    a8, b8 = _u8(a), _u8(b)
    T, K = a8.shape
    W, N = b8.shape[0], b8.shape[1]
    if b8.dim() != 3 or b8.shape[2] != K or tuple(y.shape) != (T, N) or sb.dim() != 3:
        raise ValueError("shape mismatch: a [T, K], b [W, N, K], sb [W, N/128, K/128], y [T, N]")
    if a8.stride(1) != 1 or b8.stride(2) != 1 or y.stride(1) != 1:
        raise ValueError("a, b and y must have unit stride along their last dimension")
    return a8, b8, T, K, W, N


def _dev_i32(t: torch.Tensor, what: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_cuda or t.dim() != 1 or t.stride(0) != 1:
        raise ValueError(f"{what} must be a contiguous 1-D device int32 tensor")
    return t


def fp8q_grouped_gemm_segments(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                               y: torch.Tensor, seg_indptr: torch.Tensor, seg_weight: torch.Tensor | None = None,
                               expected_rows: int = 0, stream=None) -> None:
    """Rows [seg_indptr[s], seg_indptr[s+1]) of a [T, K] times weight seg_weight[s] (default s)
    of b [W, N, K] into the same rows of y [T, N] (bf16). sa viewed as [T, K/128] (or packed
    words [T, K/512]); sb as [W, N/128, K/128]."""
    a8, b8, T, K, W, N = _packed_rows_operands(a, sa, b, sb, y)
    si = _dev_i32(seg_indptr, "seg_indptr")
    sw = None if seg_weight is None else _dev_i32(seg_weight, "seg_weight")
    S = si.numel() - 1
    if S < 0 or (sw is not None and sw.numel() != S):
        raise ValueError("seg_indptr needs S + 1 entries and seg_weight S")
    _check(load_library().fp8q_grouped_gemm_segments(
        _ptr(a8), a8.stride(0), _ptr(sa), _scale_fmt_of(sa), sa.stride(0), sa.stride(1),
        _ptr(b8), b8.stride(0), b8.stride(1), _ptr(sb), _scale_fmt_of(sb), sb.stride(0), sb.stride(1),
        sb.stride(2), _ptr(y), y.stride(0), _ptr(si), _ptr(sw), S, T, W, N, K, int(expected_rows),
        _stream(stream)))


def fp8q_grouped_gemm_contiguous(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                                 y: torch.Tensor, m_indices: torch.Tensor, stream=None) -> None:
    """Rows of a [T, K] tagged m_indices[t] (-1: padding; blocks of 128 rows, see the header)
    times weight m_indices[t] of b [W, N, K] into y [T, N] (bf16)."""
    a8, b8, T, K, W, N = _packed_rows_operands(a, sa, b, sb, y)
    mi = _dev_i32(m_indices, "m_indices")
    if mi.numel() != T:
        raise ValueError("m_indices needs one entry per row of a")
    _check(load_library().fp8q_grouped_gemm_contiguous(
        _ptr(a8), a8.stride(0), _ptr(sa), _scale_fmt_of(sa), sa.stride(0), sa.stride(1),
        _ptr(b8), b8.stride(0), b8.stride(1), _ptr(sb), _scale_fmt_of(sb), sb.stride(0), sb.stride(1),
        sb.stride(2), _ptr(y), y.stride(0), _ptr(mi), T, W, N, K, _stream(stream)))


def fp8q_device_check(device: int = 0) -> int:
    return load_library().fp8q_device_check(device)


def fp8q_status_string(status: int) -> str:
    return _status_string(status)


def fp8q_last_error() -> str:
    return load_library().fp8q_last_error().decode()

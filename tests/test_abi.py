"""CPU-side checks of the C ABI boundary (no compute calls): the built library loads and
exports every function declared in include/fp8q.h, status strings are stable, the device
check refuses when there is no gfx950, and the binding's stride marshalling reads layouts
the way the header defines them."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")
LIB = os.path.join(ROOT, "fp8_group_quant_amd", "libfp8q.so")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|int64_t|const char\*)\s+(fp8q_\w+)\s*\(", text, flags=re.M)))


def _lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("fp8q_group_quant", "fp8q_silu_mul_group_quant", "fp8q_group_quant_int8", "fp8q_gemm_blockscaled",
              "fp8q_gemm_blockscaled_ws", "fp8q_gemm_workspace_size", "fp8q_gemm_blockscaled_noalloc",
              "fp8q_grouped_gemm_masked", "fp8q_grouped_gemm_segments", "fp8q_grouped_gemm_contiguous",
              "fp8q_status_string", "fp8q_last_error", "fp8q_device_check"):
        assert n in names


def test_binding_has_a_signature_for_every_compute_entry():
    import fp8_group_quant_amd as fq
    sigs = set(fq._SIGNATURES)
    missing = [n for n in _declared() if n not in sigs and n not in ("fp8q_status_string", "fp8q_last_error")]
    assert not missing, missing


def test_library_exports_every_declared_symbol():
    lib = _lib()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    lib = _lib()
    lib.fp8q_status_string.restype = ctypes.c_char_p
    lib.fp8q_status_string.argtypes = [ctypes.c_int]
    for code, prefix in [(0, b"FP8Q_OK"), (1, b"FP8Q_EINVAL"), (2, b"FP8Q_EUNSUPPORTED"), (3, b"FP8Q_EALIGN"),
                         (4, b"FP8Q_EDEVICE"), (5, b"FP8Q_ELAUNCH")]:
        assert lib.fp8q_status_string(code).startswith(prefix)
    assert lib.fp8q_status_string(99) == b"unknown fp8q status"
    lib.fp8q_last_error.restype = ctypes.c_char_p
    assert lib.fp8q_last_error() is not None


def test_header_constants_match_binding():
    import fp8_group_quant_amd as fq
    text = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (FP8Q_\w+) (\d+)", text))
    assert consts["FP8Q_OK"] == fq.OK and consts["FP8Q_EINVAL"] == fq.EINVAL
    assert consts["FP8Q_EUNSUPPORTED"] == fq.EUNSUPPORTED and consts["FP8Q_EALIGN"] == fq.EALIGN
    assert consts["FP8Q_EDEVICE"] == fq.EDEVICE and consts["FP8Q_ELAUNCH"] == fq.ELAUNCH
    assert consts["FP8Q_DTYPE_BF16"] == fq.DTYPE_BF16 and consts["FP8Q_DTYPE_F32"] == fq.DTYPE_F32
    assert consts["FP8Q_SCALE_F32"] == fq.SCALE_F32 and consts["FP8Q_SCALE_UE8M0"] == fq.SCALE_UE8M0
    assert consts["FP8Q_SCALE_UE8M0_PACKED"] == fq.SCALE_UE8M0_PACKED
    assert consts["FP8Q_GEMM_BLOCK128"] == fq.GEMM_BLOCK128 and consts["FP8Q_GEMM_MX32"] == fq.GEMM_MX32


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the refusal path on a machine without a GPU")
def test_device_check_refuses_without_gpu():
    lib = _lib()
    lib.fp8q_device_check.argtypes = [ctypes.c_int]
    assert lib.fp8q_device_check(0) == 4  # FP8Q_EDEVICE


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks host validation on a machine without a GPU")
@pytest.mark.parametrize("entry,K,G,fmt,status", [
    ("fp8q_group_quant_int8", 512, 128, 1, 2),   # int8 with UE8M0 scales: EUNSUPPORTED
    ("fp8q_group_quant_int8", 512, 128, 2, 2),   # int8 with packed UE8M0: EUNSUPPORTED
    ("fp8q_group_quant", 512, 256, 0, 2),        # G not in {32, 64, 128} and != K: EUNSUPPORTED
    ("fp8q_group_quant", 1032, 1032, 0, 1),      # per-token with K % 16 != 0: EINVAL
    ("fp8q_group_quant", 1024, 1024, 2, 1),      # per-token, packed: 1 group per row: EINVAL
    ("fp8q_group_quant", 1024, 1024, 0, 4),      # valid per-token: passes validation, EDEVICE here
    ("fp8q_group_quant_int8", 1024, 1024, 0, 4), # valid int8 per-token: EDEVICE here
    ("fp8q_group_quant_int8", 512, 64, 0, 4),    # valid int8 groups: EDEVICE here
])
def test_quant_variant_validation_before_any_device_call(entry, K, G, fmt, status):
    # Host validation returns before the library touches a pointer or the device; the
    # addresses below are never dereferenced.
    lib = _lib()
    fn = getattr(lib, entry)
    I64, P = ctypes.c_int64, ctypes.c_void_p
    fn.argtypes = [P, ctypes.c_int, I64, I64, I64, I64, I64, P, I64, I64, P, ctypes.c_int, I64, I64, I64,
                   ctypes.c_int, P, I64, P]
    fn.restype = ctypes.c_int
    M = 8
    ng = max(K // G, 1)
    s_sm = 1 if fmt == 2 else ng
    rc = fn(0x10000, 0, 1, M, K, M * K, K, 0x20000, M * K, K, 0x30000, fmt, M * ng, s_sm, 1, G, None, 0, None)
    assert rc == status, lib.fp8q_last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks host validation on a machine without a GPU")
@pytest.mark.parametrize("mode,sa_fmt,sb_fmt,sa_ptr,status", [
    (1, 2, 2, 0x30000, 4),   # MX32, both packed words: passes validation, EDEVICE here
    (1, 2, 1, 0x30000, 4),   # MX32, packed activation words and E8M0 weight bytes
    (1, 2, 2, 0x30002, 3),   # packed words not 4-byte aligned: EALIGN
    (1, 0, 1, 0x30000, 2),   # MX32 with fp32 scales: EUNSUPPORTED
    (0, 0, 2, 0x30000, 2),   # BLOCK128 with packed weight scales: EUNSUPPORTED
    (0, 2, 0, 0x30000, 4),   # BLOCK128 with packed activation words (K % 512 == 0)
])
def test_gemm_scale_format_validation_before_any_device_call(mode, sa_fmt, sb_fmt, sa_ptr, status):
    # Host validation returns before the library touches a pointer or the device; the
    # addresses below are never dereferenced.
    lib = _lib()
    I64, P = ctypes.c_int64, ctypes.c_void_p
    fn = lib.fp8q_gemm_blockscaled
    fn.argtypes = [P, I64, P, ctypes.c_int, I64, I64, P, I64, P, ctypes.c_int, I64, I64, P, I64, I64, I64, I64,
                   ctypes.c_int, P]
    fn.restype = ctypes.c_int
    M, N, K = 256, 256, 1024
    rc = fn(0x10000, K, sa_ptr, sa_fmt, 1, M, 0x20000, K, 0x40000, sb_fmt, 1, N, 0x50000, N, M, N, K, mode, None)
    assert rc == status


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks host validation on a machine without a GPU")
@pytest.mark.parametrize("S,T,N,status", [
    (2048, 2 ** 22, 4096, 2),   # 2048 segments that may each span 32768 row tiles x 32 column tiles: EUNSUPPORTED
    (16, 4096, 4096, 4),        # a modest call passes validation (EDEVICE here)
])
def test_segments_tile_count_bound(S, T, N, status):
    """The device builds a 32-bit prefix of the segments' tile counts; segments may overlap,
    so the host refuses calls whose bound S * ceil(T/128) * ceil(N/128) reaches 2^31."""
    lib = _lib()
    I64, P, I = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    fn = lib.fp8q_grouped_gemm_segments
    fn.argtypes = [P, I64, P, I, I64, I64, P, I64, I64, P, I, I64, I64, I64, P, I64, P, P, I64, I64, I64, I64, I64,
                   I64, P]
    fn.restype = ctypes.c_int
    K = 1024
    rc = fn(0x10000, K, 0x30000, 0, K // 128, 1, 0x20000, N * K, K, 0x40000, 0, (N // 128) * (K // 128), K // 128, 1,
            0x50000, N, 0x60000, None, S, T, 1, N, K, 0, None)
    assert rc == status


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks host validation on a machine without a GPU")
def test_workspace_entries_validate_before_any_device_call():
    # Host validation returns before the library touches a pointer or the device; the
    # addresses below are never dereferenced.
    lib = _lib()
    I64, P, I = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    args = [P, I64, P, I, I64, I64, P, I64, P, I, I64, I64, P, I64, I64, I64, I64, I]
    lib.fp8q_gemm_blockscaled_ws.argtypes = args + [P, I64, P]
    lib.fp8q_gemm_blockscaled_noalloc.argtypes = args + [P]
    lib.fp8q_gemm_workspace_size.argtypes = [I64, I64, I64, I]
    lib.fp8q_gemm_workspace_size.restype = I64
    M, N, K = 64, 4096, 7168
    op = [0x10000, K, 0x30000, 1, 1, M, 0x20000, K, 0x40000, 0, K // 128, 1, 0x50000, N, M, N, K, 0]
    assert lib.fp8q_gemm_blockscaled_ws(*op, 0x60000, -1, None) == 1       # negative workspace size: EINVAL
    assert lib.fp8q_gemm_blockscaled_ws(*op, 0x60008, 1 << 24, None) == 3  # misaligned workspace: EALIGN
    assert lib.fp8q_gemm_blockscaled_ws(*op, 0x60000, 1 << 24, None) == 4  # valid: EDEVICE here
    assert lib.fp8q_gemm_blockscaled_noalloc(*op, None) == 4                # valid: EDEVICE here
    bad = list(op)
    bad[16] = 200                                                            # K % 128 != 0
    assert lib.fp8q_gemm_blockscaled_noalloc(*bad, None) == 1
    assert lib.fp8q_gemm_workspace_size(M, N, K, 0) == 0                    # no device: no workspace


def test_binding_reads_scale_layout_from_strides():
    import fp8_group_quant_amd as fq
    row = fq.alloc_scales(None, 6, 4, "f32", "row", "cpu")
    col = fq.alloc_scales(None, 6, 4, "ue8m0", "col", "cpu")
    assert fq._scale_strides(row) == (0, 4, 1)      # s_sg == 1: row-major
    assert fq._scale_strides(col) == (0, 1, 6)      # s_sm == 1: column-major
    col3 = fq.alloc_scales(3, 6, 4, "ue8m0", "col", "cpu")
    assert fq._scale_strides(col3) == (24, 1, 6)
    x = torch.empty(2, 5, 64, dtype=torch.bfloat16)
    assert fq._as3(x) == (2, 5, 64, 320, 64)
    assert fq._as3(x[0]) == (1, 5, 64, 320, 64)
    with pytest.raises(ValueError):
        fq._as3(torch.empty(4, 8)[:, ::2])


def test_package_has_no_fallback_when_library_missing(tmp_path):
    import fp8_group_quant_amd as fq
    saved = fq._lib
    try:
        fq._lib = None
        with pytest.raises(ImportError):
            fq.load_library(str(tmp_path / "missing.so"))
    finally:
        fq._lib = saved


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "fp8_group_quant_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), errors="ignore").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "fp8q_oracle" not in text, f

"""fp8q_gemm_blockscaled_noalloc (the call for callers that cannot allocate) against the
workspace entry point it varies, through the C ABI: two calls in a row on one device, the
second smaller, so the second reuses the library's scratch array holding the first call's
partial sums. Both paths run the same kernels in the same order, so the outputs must be
identical bit for bit (which is within the GEMM tolerance); a sampled oracle check pins both.
A shape needing more scratch than the library holds is refused with nothing written."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gemm_check import check

pytestmark = pytest.mark.gpu

SENT_I16 = 0xA5A5 - 0x10000


def _fq():
    import fp8_group_quant_amd
    return fp8_group_quant_amd


def _operands(M, N, K, seed):
    w = synth.Workload("na", seed=seed, M=M, K=K, N=N, scale_fmt="ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    sa_col = np.ascontiguousarray(sa.T)
    return a, sa_col, b, sb


def _call(entry, a, sa_col, b, sb, M, N, K, workspace=None):
    """Raw C-ABI call; returns (status, y bits)."""
    f = _fq()
    lib = f.load_library()
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    sad = torch.from_numpy(sa_col).cuda().t()
    sbd = torch.from_numpy(sb).cuda()
    y = torch.full((M, N), SENT_I16, dtype=torch.int16, device="cuda")
    args = [ad.data_ptr(), K, sad.data_ptr(), oracle.SCALE_UE8M0, sad.stride(0), sad.stride(1),
            bd.data_ptr(), K, sbd.data_ptr(), oracle.SCALE_F32, sbd.stride(0), sbd.stride(1),
            y.data_ptr(), N, M, N, K, f.GEMM_BLOCK128]
    if entry == "ws":
        rc = lib.fp8q_gemm_blockscaled_ws(*args, workspace.data_ptr(), workspace.numel(),
                                          torch.cuda.current_stream().cuda_stream)
    else:
        rc = lib.fp8q_gemm_blockscaled_noalloc(*args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc, y.cpu().numpy().view(np.uint16)


def test_noalloc_matches_workspace_call_twice():
    f = _fq()
    for (M, N, K, seed) in [(128, 4096, 7168, 101), (40, 1000, 2048, 102)]:
        need = f.fp8q_gemm_workspace_size(M, N, K, f.GEMM_BLOCK128)
        assert 0 < need <= 32 << 20
        a, sa_col, b, sb = _operands(M, N, K, seed)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        rc_ws, y_ws = _call("ws", a, sa_col, b, sb, M, N, K, ws)
        rc_na, y_na = _call("noalloc", a, sa_col, b, sb, M, N, K)
        assert rc_ws == f.OK and rc_na == f.OK
        assert np.array_equal(y_na, y_ws), f"{M}x{N}x{K}"
        g = np.random.default_rng(seed)
        ms = np.concatenate([[0, M - 1], g.integers(0, M, 2048)])
        ns = np.concatenate([[0, N - 1], g.integers(0, N, 2048)])
        ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col", at=(ms, ns))
        check(y_na[ms, ns], ys, ss, K, f"no-alloc {M}x{N}x{K}")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    f = _fq()
    M, N, K = 128, 16384, 7168
    assert f.fp8q_gemm_workspace_size(M, N, K, f.GEMM_BLOCK128) > 32 << 20
    a = np.zeros((M, K), np.uint8)
    sa_col = np.full((K // 128, M), 127, np.uint8)
    b = np.zeros((N, K), np.uint8)
    sb = np.ones((N // 128, K // 128), np.float32)
    rc, y = _call("noalloc", a, sa_col, b, sb, M, N, K)
    assert rc == f.EUNSUPPORTED
    assert np.all(y == 0xA5A5)


def test_noalloc_without_scratch_need():
    """Shapes that need no workspace (M <= 16, large M) run as the plain call."""
    f = _fq()
    for M in (16, 300):
        N, K = 256, 1024
        a, sa_col, b, sb = _operands(M, N, K, 103 + M)
        assert f.fp8q_gemm_workspace_size(M, N, K, f.GEMM_BLOCK128) == 0
        rc, y = _call("noalloc", a, sa_col, b, sb, M, N, K)
        assert rc == f.OK
        ys, ss = oracle.gemm_block128(a, sa_col, b, sb, oracle.SCALE_UE8M0, "col")
        check(y, ys, ss, K, f"no-alloc M={M}")

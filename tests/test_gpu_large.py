"""GPU parity at byte offsets past 2 GiB and 4 GiB: the quant's input, codes and scales and
the GEMM's activation operand are larger than 4 GiB, so any 32-bit row or byte offset
would wrap. The tensors are zero except for seeded synthetic rows placed on both sides of
the 2^31- and 2^32-byte boundaries (and at both ends); those rows are compared with the
oracle run on the same rows alone, bit-exact for the quant and to the GEMM tolerance, and
a zero row is checked too."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gemm_check import check

pytestmark = pytest.mark.gpu

SENT = 0xA5A5
SENT_I16 = SENT - 0x10000


def fq():
    import fp8_group_quant_amd
    return fp8_group_quant_amd


def _rows_across(M, row_bytes, seed):
    """Rows at both ends, the rows whose byte offsets straddle 2^31 and 2^32 for rows of
    row_bytes bytes, and a few seeded random ones (sorted, unique)."""
    pick = [0, 1, M - 2, M - 1]
    for edge in (2 ** 31, 2 ** 32):
        r = edge // row_bytes
        pick += [r - 1, r, r + 1]
    pick += list(np.random.default_rng(seed).integers(0, M, 8))
    return np.unique(np.array([r for r in pick if 0 <= r < M], dtype=np.int64))


@pytest.mark.parametrize("fmt,layout", [("ue8m0", "col"), ("f32", "row")])
def test_quant_offsets_beyond_4gib(fmt, layout):
    K, G = 7168, 128
    M = 2 ** 32 // (2 * K) + 600  # bf16 input 4.3 GB, codes 2.15 GB
    rows = _rows_across(M, 2 * K, 11)
    assert rows.max() * 2 * K > 2 ** 32
    vals = synth.activations_bf16(31, len(rows), K, outlier_p=0.01)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    idx = torch.from_numpy(rows).cuda()
    x.view(torch.int16)[idx] = torch.from_numpy(vals.view(np.int16)).cuda()
    zero_row = int(rows[len(rows) // 2]) + 1
    while zero_row in rows:
        zero_row += 1
    q, s = fq().group_quant(x, G, fmt, layout)
    torch.cuda.synchronize()
    del x
    ofmt = oracle.SCALE_UE8M0 if fmt == "ue8m0" else oracle.SCALE_F32
    qo, so = oracle.group_quant(vals, G, ofmt, layout)
    if layout == "col":
        so = so.T
    assert np.array_equal(q[idx].cpu().numpy(), qo), "codes of the sampled rows"
    assert np.array_equal(s[idx].cpu().numpy().view(np.uint8), np.ascontiguousarray(so).view(np.uint8)), "scales"
    zq, zs = oracle.group_quant(np.zeros((1, K), dtype=np.uint16), G, ofmt, layout)
    assert np.array_equal(q[zero_row].cpu().numpy(), zq[0])
    assert np.array_equal(s[zero_row].cpu().numpy().view(np.uint8), np.ascontiguousarray(zs.reshape(-1)).view(np.uint8))


@pytest.mark.parametrize("sa_kind", ["ue8m0-col", "f32-row"])
def test_gemm_offsets_beyond_4gib(sa_kind):
    K, N = 7168, 300
    # A 4.3 GB; column-major UE8M0 scales are moved 4 rows per word (M % 4 == 0), fp32 row
    # scales take a ragged M
    M = (2 ** 32 // K + 1500) // 4 * 4 + (0 if sa_kind == "ue8m0-col" else 3)
    rows = _rows_across(M, K, 12)
    assert rows.max() * K > 2 ** 32
    fmt, layout = sa_kind.split("-")
    w = synth.Workload("big", seed=13, M=len(rows), K=K, N=N, scale_fmt=fmt)
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    idx = torch.from_numpy(rows).cuda()
    A = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    A[idx] = torch.from_numpy(a).cuda()
    if layout == "col":  # [K/128, M] storage, viewed [M, K/128]
        S = torch.full((K // 128, M), 127, dtype=torch.uint8, device="cuda")
        S[:, idx] = torch.from_numpy(np.ascontiguousarray(sa.T)).cuda()
        S = S.t()
    else:
        S = torch.ones((M, K // 128), dtype=torch.float32, device="cuda")
        S[idx] = torch.from_numpy(sa).cuda()
    y = torch.full((M, N), SENT_I16, dtype=torch.int16, device="cuda")
    fq().fp8q_gemm_blockscaled(A, S, torch.from_numpy(b).cuda(), torch.from_numpy(sb).cuda(),
                               y.view(torch.bfloat16))
    torch.cuda.synchronize()
    del A, S
    assert not bool((y == SENT_I16).any()), "every output written"
    ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_UE8M0 if fmt == "ue8m0" else oracle.SCALE_F32, "row")
    check(y[idx].cpu().numpy().view(np.uint16), ys, ss, K, f"rows past 4 GiB ({sa_kind})")
    others = torch.ones(M, dtype=torch.bool, device="cuda")
    others[idx] = False
    assert not bool((y[others] & 0x7FFF).any()), "zero rows give (signed) zero outputs"


def test_masked_quant_expert_offsets_beyond_4gib():
    """Masked quant of [E, cap, K] bf16 (4.7 GB) where only experts past the 4 GiB mark (and
    expert 0) hold rows: expert strides times the expert index exceed 32 bits."""
    E, cap, K, G = 80, 4096, 7168, 128
    mm = np.zeros(E, dtype=np.int32)
    mm[[0, 75, 79]] = [3, 129, 1]
    assert 75 * cap * K * 2 > 2 ** 32
    x = torch.zeros((E, cap, K), dtype=torch.bfloat16, device="cuda")
    vals = {}
    for e in np.nonzero(mm)[0]:
        v = synth.activations_bf16(40 + int(e), int(mm[e]), K)
        x[e, :mm[e]].view(torch.int16).copy_(torch.from_numpy(v.view(np.int16)))
        vals[int(e)] = v
    f = fq()
    q = torch.full((E, cap, K), 0xA5, dtype=torch.uint8, device="cuda")
    s = f.alloc_scales(E, cap, K // G, "ue8m0", "col", "cuda")
    f.fp8q_group_quant(x, q, s, G, torch.from_numpy(mm).cuda(), 0)
    torch.cuda.synchronize()
    del x
    for e, v in vals.items():
        qo, so = oracle.group_quant(v, G, oracle.SCALE_UE8M0, "col")
        assert np.array_equal(q[e, :mm[e]].cpu().numpy(), qo), f"expert {e} codes"
        assert np.array_equal(s[e, :mm[e]].cpu().numpy(), np.ascontiguousarray(so.T)), f"expert {e} scales"
        assert bool((q[e, mm[e]:] == 0xA5).all()), f"expert {e}: rows past masked_m written"


def test_masked_gemm_expert_offsets_beyond_4gib():
    """Masked grouped GEMM over A [E, cap, K] (4.7 GB) with rows only in expert 0 and in
    experts whose A, scales and Y blocks start past the 4 GiB mark."""
    E, cap, K, N = 160, 4096, 7168, 256
    mm = np.zeros(E, dtype=np.int32)
    mm[[0, 150, 159]] = [5, 130, 2]
    assert 150 * cap * K > 2 ** 32
    A = torch.zeros((E, cap, K), dtype=torch.uint8, device="cuda")
    SA = torch.full((E, K // 128, cap), 127, dtype=torch.uint8, device="cuda")
    B = torch.zeros((E, N, K), dtype=torch.uint8, device="cuda")
    SB = torch.ones((E, N // 128, K // 128), dtype=torch.float32, device="cuda")
    ops = {}
    for e in np.nonzero(mm)[0]:
        e = int(e)
        w = synth.Workload("bigm", seed=50 + e, M=int(mm[e]), K=K, N=N, scale_fmt="ue8m0")
        a, sa = synth.gemm_activation(w)
        b, sb = synth.weights(w)
        A[e, :mm[e]] = torch.from_numpy(a).cuda()
        SA[e, :, :mm[e]] = torch.from_numpy(np.ascontiguousarray(sa.T)).cuda()
        B[e] = torch.from_numpy(b).cuda()
        SB[e] = torch.from_numpy(sb).cuda()
        ops[e] = (a, sa, b, sb)
    y = torch.full((E, cap, N), SENT_I16, dtype=torch.int16, device="cuda")
    fq().fp8q_grouped_gemm_masked(A, SA.transpose(1, 2), B, SB, y.view(torch.bfloat16),
                                  torch.from_numpy(mm).cuda(), 64)
    torch.cuda.synchronize()
    del A
    for e, (a, sa, b, sb) in ops.items():
        ys, ss = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_UE8M0, "row")
        check(y[e, :mm[e]].cpu().numpy().view(np.uint16), ys, ss, K, f"expert {e}")
        assert bool((y[e, mm[e]:] == SENT_I16).all()), f"expert {e}: rows past masked_m written"
    empty = torch.from_numpy(np.nonzero(mm == 0)[0]).cuda()
    assert bool((y[empty] == SENT_I16).all()), "experts without rows untouched"

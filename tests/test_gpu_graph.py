"""The quant -> GEMM step captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI calls):
the library allocates nothing and enqueues only kernels on the caller's stream, so a captured
step replays like the eager one. Each replay gets new activations copied into the captured
input buffer, with eager work and synchronizations between replays, and every replay is
compared byte for byte with the eager result on the same input (and the eager quant with the
oracle)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


# M = 24, 64 and 128 take the split-K GEMM (two kernels and a workspace the binding takes
# from torch's allocator inside the capture)
@pytest.mark.parametrize("M", [1, 16, 24, 64, 128, 300])
def test_quant_gemm_step_replays_in_a_graph(M):
    import fp8_group_quant_amd as fq
    w = synth.dense(M) if M in (1, 16, 64, 128) else synth.Workload("g", seed=80, M=M, K=7168, N=4096)
    K, N, G = w.K, w.N, 128
    b, sb = synth.weights(w)
    bd, sbd = torch.from_numpy(b).cuda(), torch.from_numpy(sb).cuda()
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = fq.alloc_scales(None, M, K // G, "ue8m0", "col", "cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        fq.fp8q_group_quant(x, q, s, G)
        fq.fp8q_gemm_blockscaled(q, s, bd, sbd, y)

    inputs = [synth.activations_bf16(81 + i, M, K, outlier_p=0.01) for i in range(4)]
    x.copy_(torch.from_numpy(inputs[0]).view(torch.bfloat16))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i, xin in enumerate(inputs):
        x.copy_(torch.from_numpy(xin).view(torch.bfloat16))
        step()  # eager reference
        torch.cuda.synchronize()
        q_e, s_e, y_e = q.clone(), s.clone(), y.clone()
        q.fill_(0xA5)
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, q_e), f"replay {i}: codes differ from the eager step"
        assert torch.equal(s, s_e), f"replay {i}: scales differ from the eager step"
        assert torch.equal(y.view(torch.int16), y_e.view(torch.int16)), f"replay {i}: Y differs"
        if i == 0:
            qo, so = oracle.group_quant(xin, G, oracle.SCALE_UE8M0, "col")
            assert np.array_equal(q_e.cpu().numpy(), qo) and np.array_equal(s_e.cpu().numpy(), so.T)


def test_masked_moe_step_replays_with_new_counts():
    """The MoE second stage (masked silu+quant into column-major UE8M0 scales, then the masked
    grouped GEMM) captured once and replayed with new activations AND new per-expert row
    counts written into the captured masked_m buffer: the kernels read the counts on the
    device, so no re-capture is needed. Rows past each count keep their sentinels."""
    import fp8_group_quant_amd as fq
    E, cap, K, N, G = 8, 256, 1024, 512, 128
    w = synth.Workload("gm", seed=90, M=cap, K=K, N=N, E=E, scale_fmt="ue8m0", masked=True)
    wts = [synth.weights(w, e) for e in range(E)]
    bd = torch.from_numpy(np.stack([t[0] for t in wts])).cuda()
    sbd = torch.from_numpy(np.stack([t[1] for t in wts])).cuda()
    x = torch.empty((E, cap, 2 * K), dtype=torch.bfloat16, device="cuda")
    mm = torch.zeros(E, dtype=torch.int32, device="cuda")
    q = torch.empty((E, cap, K), dtype=torch.uint8, device="cuda")
    s = fq.alloc_scales(E, cap, K // G, "ue8m0", "col", "cuda")
    y = torch.empty((E, cap, N), dtype=torch.bfloat16, device="cuda")

    def step():
        fq.fp8q_silu_mul_group_quant(x, q, s, G, mm, 64)
        fq.fp8q_grouped_gemm_masked(q, s, bd, sbd, y, mm, 64)

    counts = [np.array(c, dtype=np.int32) for c in ([0, 1, 255, 256, 17, 128, 129, 3],
                                                    [256, 0, 0, 64, 200, 1, 127, 255],
                                                    [5, 5, 5, 5, 5, 5, 5, 5],
                                                    [0, 0, 0, 0, 0, 0, 0, 0])]
    inputs = [synth.activations_bf16(91 + i, E * cap, 2 * K, outlier_p=0.01).reshape(E, cap, 2 * K)
              for i in range(len(counts))]

    def load(i):
        x.copy_(torch.from_numpy(inputs[i]).view(torch.bfloat16))
        mm.copy_(torch.from_numpy(counts[i]))
        q.fill_(0xA5)
        s.fill_(0xA5)
        y.view(torch.int16).fill_(-23131)  # 0xA5A5

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i in range(len(counts)):
        load(i)
        step()  # eager reference
        torch.cuda.synchronize()
        q_e, s_e, y_e = q.clone(), s.clone(), y.clone()
        load(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, q_e), f"replay {i}: codes differ from the eager step"
        assert torch.equal(s, s_e), f"replay {i}: scales differ from the eager step"
        assert torch.equal(y.view(torch.int16), y_e.view(torch.int16)), f"replay {i}: Y differs"
        for e in range(E):
            r = int(counts[i][e])
            assert bool((y_e[e, r:].view(torch.int16) == -23131).all()), f"count set {i}, expert {e}: rows past masked_m"
        if i == 0:
            for e in (2, 6):
                r = int(counts[i][e])
                qo, so = oracle.group_quant(inputs[i][e, :r], G, oracle.SCALE_UE8M0, "col", silu=True)
                assert np.array_equal(q_e[e, :r].cpu().numpy(), qo), f"expert {e}: codes vs the oracle"
                assert np.array_equal(s_e[e, :r].cpu().numpy(), so.T), f"expert {e}: scales vs the oracle"


def test_noalloc_gemm_replays_in_a_graph():
    """The allocation-free GEMM (split-K partial sums in the library's own array) captured
    and replayed: every replay, with new activations and eager work between replays, equals
    the eager call bit for bit."""
    import fp8_group_quant_amd as fq
    M, N, K = 128, 4096, 7168
    w = synth.Workload("gna", seed=85, M=M, K=K, N=N, scale_fmt="ue8m0")
    b, sb = synth.weights(w)
    bd, sbd = torch.from_numpy(b).cuda(), torch.from_numpy(sb).cuda()
    a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((K // 128, M), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def call():
        fq.fp8q_gemm_blockscaled_noalloc(a, sa.t(), bd, sbd, y)

    ops = []
    for i in range(3):
        wi = synth.Workload("gna", seed=86 + i, M=M, K=K, N=N, scale_fmt="ue8m0")
        ai, sai = synth.gemm_activation(wi)
        ops.append((torch.from_numpy(ai), torch.from_numpy(np.ascontiguousarray(sai.T))))
    a.copy_(ops[0][0])
    sa.copy_(ops[0][1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i, (ai, sai) in enumerate(ops):
        a.copy_(ai)
        sa.copy_(sai)
        call()
        torch.cuda.synchronize()
        y_e = y.clone()
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_e.view(torch.int16)), f"replay {i}: Y differs from the eager call"

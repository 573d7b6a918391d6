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


@pytest.mark.parametrize("M", [1, 16, 128, 300])
def test_quant_gemm_step_replays_in_a_graph(M):
    import fp8_group_quant_amd as fq
    w = synth.dense(M) if M in (1, 16, 128) else synth.Workload("g", seed=80, M=M, K=7168, N=4096)
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

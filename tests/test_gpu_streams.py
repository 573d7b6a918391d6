"""Calls from several host threads, each on its own HIP stream with its own buffers, at the
same time: the library keeps no shared mutable state besides a per-device check cache (atomic)
and a thread-local error string, so every thread must get exactly the result of a serial run."""
import threading

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


# M = 64 takes the split-K GEMM: the binding allocates each call's workspace on the stream
# the call runs on
@pytest.mark.parametrize("M", [256, 64])
def test_concurrent_streams_match_serial_results(M):
    import fp8_group_quant_amd as fq
    n_threads, iters = 4, 12
    K, N, G = 2048, 512, 128
    w = synth.Workload("c", seed=90, M=M, K=K, N=N)
    assert (fq.fp8q_gemm_workspace_size(M, N, K) > 0) == (M == 64)
    b, sb = synth.weights(w)
    bd, sbd = torch.from_numpy(b).cuda(), torch.from_numpy(sb).cuda()
    xs = [torch.from_numpy(synth.activations_bf16(91 + t, M, K)).cuda().view(torch.bfloat16) for t in range(n_threads)]

    def step(x, stream):
        q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        s = fq.alloc_scales(None, M, K // G, "ue8m0", "col", "cuda")
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        fq.fp8q_group_quant(x, q, s, G, stream=stream)
        fq.fp8q_gemm_blockscaled(q, s, bd, sbd, y, stream=stream)
        return q, s, y

    ref = []
    for t in range(n_threads):
        q, s, y = step(xs[t], torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref.append((q.cpu(), s.cpu(), y.view(torch.int16).cpu()))

    errors = []

    def worker(t):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(iters):
                    q, s, y = step(xs[t], st)
                    st.synchronize()
                    if not (torch.equal(q.cpu(), ref[t][0]) and torch.equal(s.cpu(), ref[t][1])
                            and torch.equal(y.view(torch.int16).cpu(), ref[t][2])):
                        errors.append(f"thread {t}: result differs from the serial run")
                        return
        except Exception as ex:  # reported below
            errors.append(f"thread {t}: {ex!r}")

    # a raw stream handle (not the current stream) also works
    st = torch.cuda.Stream()
    q, s, y = step(xs[0], st.cuda_stream)
    st.synchronize()
    assert torch.equal(y.view(torch.int16).cpu(), ref[0][2])

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors

"""The GEMM tolerance rule accepts the exact result rounded to bf16 and rejects plausible
kernel mistakes, planted here in oracle outputs on the CPU."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gemm_check import check


def _case():
    w = synth.Workload("t", seed=90, M=96, K=1024, N=256, scale_fmt="ue8m0")
    a, sa = synth.gemm_activation(w)
    b, sb = synth.weights(w)
    y, s = oracle.gemm_block128(a, sa, b, sb, oracle.SCALE_UE8M0)
    return a, sa, b, sb, y, s


def _bits(v):
    return torch.from_numpy(v).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_rounded_exact_result_passes():
    *_, y, s = _case()
    st = check(_bits(y), y, s, 1024)
    assert st["n_cancel"] == 0 and st["frob"] < 2e-3


def test_dropped_k_block_fails():
    a, sa, b, sb, y, s = _case()
    a2 = a.copy()
    a2[:, 896:] = 0  # the last 128-wide K block is lost
    y2, _ = oracle.gemm_block128(a2, sa, b, sb, oracle.SCALE_UE8M0)
    with pytest.raises(AssertionError):
        check(_bits(y2), y, s, 1024)


def test_wrong_block_scale_fails():
    a, sa, b, sb, y, s = _case()
    sb2 = sb[::-1].copy()  # N blocks swapped
    y2, _ = oracle.gemm_block128(a, sa, b, sb2, oracle.SCALE_UE8M0)
    with pytest.raises(AssertionError):
        check(_bits(y2), y, s, 1024)


def test_one_ulp_bias_everywhere_fails_frobenius_floor():
    *_, y, s = _case()
    yb = (_bits(y).astype(np.int32) + 3).astype(np.uint16)  # 3 ulp off everywhere
    with pytest.raises(AssertionError):
        check(yb, y, s, 1024)


def _perturbed(y, s, idx, amount):
    """y with amount * S added to the listed elements, rounded to bf16 bits."""
    y2 = y.copy()
    y2.flat[idx] += amount * s.flat[idx]
    return _bits(y2)


def test_cancellation_allowance_is_eta_plus_gamma_and_counted():
    """An error of half the allowance on two cancelling elements passes and is counted; one
    of 1.5 times the allowance fails. (Planted in the oracle's own output.)"""
    from gemm_check import ETA, gamma, ulp_bf16
    *_, y, s = _case()
    allow = ETA["act"] + gamma(1024)
    # elements where the allowance is far above 2 ulp of the result (near-cancellation)
    ratio = allow * s / (2 * ulp_bf16(y))
    idx = np.argsort(ratio.ravel())[-2:]
    assert ratio.flat[idx].min() > 8
    st = check(_perturbed(y, s, idx, 0.5 * allow), y, s, 1024)
    assert st["n_cancel"] == 2 and st["max_excess_over_S"] < 0.5 * allow
    with pytest.raises(AssertionError):
        check(_perturbed(y, s, idx, 1.5 * allow), y, s, 1024)


def test_allowance_depends_on_the_operand_class():
    from gemm_check import ETA, gamma, ulp_bf16
    *_, y, s = _case()
    ratio = ETA["outlier"] * s / (2 * ulp_bf16(y))
    idx = np.argsort(ratio.ravel())[-1:]
    bad = _perturbed(y, s, idx, 0.5 * (ETA["outlier"] + gamma(1024)))
    check(bad, y, s, 1024, cls="outlier")
    with pytest.raises(AssertionError):
        check(bad, y, s, 1024, cls="act")

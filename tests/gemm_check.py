"""Tolerance rule shared by the GEMM parity tests (test helper, not product code).

Reading of "within 2 bf16 ulp per element and 2e-3 relative Frobenius error of an fp64
oracle" used here:

Per element, a GPU bf16 output y matches the fp64 value Y* when
    |y - Y*| <= 2 ulp_bf16(Y*).
Where Y* nearly cancels (|Y*| much smaller than S = sum_k |term_k|), 2 ulp of Y* is below
what any finite-precision accumulation can promise, so those elements may instead meet
    |y - Y*| <= 2 ulp_bf16(Y*) + (eta_c + gamma(K)) * S
and they are counted: at most max(2, 0.5%) of the compared elements may need it.
  - gamma(K) = (4 ceil(K/128) + 2) 2^-24 bounds the fp32 accumulation across K blocks.
  - eta_c bounds the error of one 128-term FP8 dot product of the gfx950 matrix core,
    relative to that block's S, for operand class c (ETA below). The matrix core does not
    sum 128 products to fp32 accuracy: tests/test_gpu_accumulation.py measures its error
    on outputs whose exact value is 0 and asserts these bounds (the largest errors seen
    there are about half of each bound).
The sum of the block errors is at most eta_c * S, so the rule is a bound, not a fit. On real
data the block errors are independent and mostly cancel: the same test measures the whole
error of a GEMM at 2^-19.9 S for K = 7168 and 2^-18.2 S for K = 2048, within gamma(K) alone;
each check reports how far the worst element went (excess_over_S) against gamma(K).

Frobenius: ||y - Y*|| / ||Y*|| <= 2e-3 over every compared set of at least 4096 elements.
Rounding the exact Y* to bf16 alone costs about 1.66e-3 for Gaussian-like outputs, so on
small samples that ratio scatters around 2e-3; every set, whatever its size, must also stay
within 3e-4 of the error of bf16(Y*) itself (the accumulation may add at most that much).
"""
import json
import os

import numpy as np
import torch

# Bound of one matrix-core block's error, as a multiple of the block's S, per operand class
# (largest measured value in parentheses, log2):
#   act      activation-like codes of N(0, 100^2) x N(0, 1) weight codes          (-15.0)
#   quant    G=128 UE8M0 quantization of N(0, 1) bf16 rows x N(0, 1) weight codes  (-15.0)
#   outlier  the same with 1% of the inputs x50 (a group's S then rests on one
#            outlier product)                                                      (-11.7)
#   silu     G=128 quantization of silu(g) * u, g, u ~ N(0, 1) x N(0, 1) weights    (-13.1)
#   wide     N(0, 1) codes on both operands (MXFP8 workload)                        (-15.1)
#   full     codes uniform over every finite e4m3 value                             (-12.0)
ETA = {"act": 2.0 ** -14, "quant": 2.0 ** -14, "outlier": 2.0 ** -10, "silu": 2.0 ** -12,
       "wide": 2.0 ** -14, "full": 2.0 ** -11}
FROB = 2e-3
FROB_MIN_N = 4096


def gamma(K: int) -> float:
    """fp32 summation bound for the accumulation across ceil(K/128) blocks."""
    return (4 * -(-K // 128) + 2) * 2.0 ** -24


def record(kind: str, stats: dict) -> None:
    """Appends a JSON line to the file named by FP8Q_PARITY_STATS (if set): the per-test
    figures that the design notes quote (elements needing the allowance, Frobenius, ...)."""
    path = os.environ.get("FP8Q_PARITY_STATS")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"kind": kind, **stats}) + "\n")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Y* rounded to bf16 (fp64 -> fp32 -> bf16, RNE), as float64."""
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).to(torch.float32).to(torch.bfloat16) \
        .to(torch.float64).numpy()


def check(y_bits: np.ndarray, ystar: np.ndarray, s: np.ndarray, K: int, what: str = "",
          cls: str = "act") -> dict:
    """Applies the rule above to bf16 outputs y_bits (uint16) against the oracle's Y* and S.
    cls names the operand class (a key of ETA). Returns the figures of the comparison:
    n, n_cancel (elements beyond 2 ulp), their share, the largest excess beyond 2 ulp in
    units of S and of ulp, how many went beyond gamma(K) * S, and the Frobenius ratios."""
    y = bf16_bits_to_f64(y_bits)
    assert y.shape == ystar.shape, (y.shape, ystar.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    n = y.size
    err = np.abs(y - ystar)
    ulp = ulp_bf16(ystar)
    tol = 2.0 * ulp
    over = err > tol
    allow = (ETA[cls] + gamma(K)) * s
    bad = err > tol + allow
    assert not np.any(bad), (f"{what}: {int(bad.sum())} elements outside 2 ulp + (eta + gamma) S; first at "
                             f"{np.argwhere(bad)[0].tolist()} (err {err[bad][0]}, 2ulp {tol[bad][0]}, S {s[bad][0]})")
    n_over = int(over.sum())
    assert n_over <= max(2, int(0.005 * n)), f"{what}: {n_over} of {n} elements needed the cancellation allowance"
    excess = np.where(over, err - tol, 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        ex_s = np.where(over, excess / np.maximum(s, 1e-300), 0.0)
    stats = {"what": what, "K": int(K), "cls": cls, "n": int(n), "n_cancel": n_over,
             "frac_cancel": n_over / max(n, 1), "max_excess_over_S": float(ex_s.max()) if n else 0.0,
             "max_excess_ulp": float((excess / ulp).max()) if n else 0.0, "gamma": gamma(K),
             "n_beyond_gamma": int(np.sum(over & (err > tol + gamma(K) * s)))}
    den = np.linalg.norm(ystar)
    if den > 0:
        rel = np.linalg.norm(y - ystar) / den
        floor = np.linalg.norm(bf16_round(ystar) - ystar) / den
        stats.update(frob=float(rel), frob_bf16_floor=float(floor))
        assert rel <= floor + 3e-4, f"{what}: Frobenius {rel:.3e} exceeds the bf16 rounding floor {floor:.3e} + 3e-4"
        if n >= FROB_MIN_N:
            assert rel <= FROB, f"{what}: relative Frobenius error {rel:.3e} > 2e-3 over {n} elements"
    record("gemm_check", stats)
    return stats

"""Tolerance rule shared by the GEMM parity tests (test helper, not product code).

Reading of "within 2 bf16 ulp per element and 2e-3 relative Frobenius error of an fp64
oracle" used here:

Per element, a GPU bf16 output y matches the fp64 value Y* when
    |y - Y*| <= 2 ulp_bf16(Y*).
Where Y* nearly cancels (|Y*| much smaller than S = sum_k |term_k|), 2 ulp of Y* is below
what any finite-precision accumulation can promise, so those elements may instead meet
    |y - Y*| <= 2 ulp_bf16(Y*) + eta * S,    eta = 2^-12,
and they are counted: at most max(2, 0.5%) of the compared elements may need it. eta is the
in-instruction accumulation precision of the gfx950 fp8 matrix core, measured on random
full-range e4m3 operands (largest error 2^-12.6 * S per 128-wide K block); exact-fp32 fold
arithmetic between blocks adds far less.

Frobenius: ||y - Y*|| / ||Y*|| <= 2e-3 over every compared set of at least 4096 elements.
Rounding the exact Y* to bf16 alone costs about 1.66e-3 for Gaussian-like outputs, so on
small samples that ratio scatters around 2e-3; every set, whatever its size, must also stay
within 3e-4 of the error of bf16(Y*) itself (the accumulation may add at most that much).
"""
import numpy as np
import torch

ETA = 2.0 ** -12
FROB = 2e-3
FROB_MIN_N = 4096


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


def check(y_bits: np.ndarray, ystar: np.ndarray, s: np.ndarray, K: int, what: str = "") -> dict:
    y = bf16_bits_to_f64(y_bits)
    assert y.shape == ystar.shape, (y.shape, ystar.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    n = y.size
    err = np.abs(y - ystar)
    tol = 2.0 * ulp_bf16(ystar)
    over = err > tol
    bad = err > tol + ETA * s
    assert not np.any(bad), (f"{what}: {int(bad.sum())} elements outside 2 ulp + eta*S; first at "
                             f"{np.argwhere(bad)[0].tolist()} (err {err[bad][0]}, 2ulp {tol[bad][0]}, S {s[bad][0]})")
    n_over = int(over.sum())
    assert n_over <= max(2, int(0.005 * n)), f"{what}: {n_over} of {n} elements needed the cancellation allowance"
    stats = {"n": n, "n_cancel": n_over}
    den = np.linalg.norm(ystar)
    if den > 0:
        rel = np.linalg.norm(y - ystar) / den
        floor = np.linalg.norm(bf16_round(ystar) - ystar) / den
        stats.update(frob=rel, frob_bf16_floor=floor)
        assert rel <= floor + 3e-4, f"{what}: Frobenius {rel:.3e} exceeds the bf16 rounding floor {floor:.3e} + 3e-4"
        if n >= FROB_MIN_N:
            assert rel <= FROB, f"{what}: relative Frobenius error {rel:.3e} > 2e-3 over {n} elements"
    return stats

"""Pins of the oracle's e4m3fn codec and UE8M0 scale rule against things other than
itself: torch's float8_e4m3fn cast (an independent library routine), exact rational
arithmetic, and hand-derived golden values (tests/golden/*.txt)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((parts[0], parts[1]))
    return rows


def _torch_e4m3(values: np.ndarray) -> np.ndarray:
    return torch.from_numpy(values.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ----------------------------------------------------------------------------- decode
def test_decode_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_mine = np.isnan(mine)
    assert np.array_equal(nan_mine, np.isnan(ref))
    assert sorted(np.nonzero(nan_mine)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(mine[~nan_mine], ref[~nan_mine])
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x01] == 2.0 ** -9
    assert np.signbit(mine[0x80]) and mine[0x80] == 0.0


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_decode_is_monotone_over_non_negative_codes():
    v = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


# ----------------------------------------------------------------------------- encode
def test_encode_golden_values():
    rows = _read_golden("e4m3_codes.txt")
    assert len(rows) >= 15
    vals = np.array([float(eval(v)) for v, _ in rows], dtype=np.float32)
    want = np.array([int(c, 16) for _, c in rows], dtype=np.uint8)
    got = oracle.e4m3_encode(vals)
    for v, w, g in zip(vals, want, got):
        assert w == g, f"{v!r}: want {w:#04x} got {g:#04x}"


def _boundary_values() -> np.ndarray:
    """Midpoints between consecutive e4m3 values and their fp32 neighbours."""
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    v = np.concatenate([mids, up, dn, pos.astype(np.float32)])
    v = v[np.abs(v) <= 448]
    return np.concatenate([v, -v])


def test_encode_boundaries_match_torch():
    v = _boundary_values()
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_encode_every_bf16_value_in_range_matches_torch():
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    v = bits[np.isfinite(bits) & (np.abs(bits) <= 448)]
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_encode_fp32_sweep_matches_torch():
    # every 193rd fp32 pattern whose magnitude is below 512, both signs, clamped to +-448
    bits = np.arange(0, 0x44000000, 193, dtype=np.uint32)
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    v = np.clip(v, -448, 448).astype(np.float32)
    assert v.size > 2 ** 23
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_encode_every_fp32_pattern_after_the_clamp():
    """Every fp32 pattern through the clamp to [-448, 448] and the encoder, against torch's
    cast: the 2 x 1,138,753,537 patterns of magnitude <= 448 (both signs, zeros and
    subnormals) one by one, in chunks; every larger finite or infinite magnitude becomes
    +-448 at the clamp, so it meets the encoder as that one value (checked with its
    neighbours). NaN is outside the contract (finite inputs)."""
    top = 0x43E00000  # 448.0
    assert np.array([top], np.uint32).view(np.float32)[0] == 448.0
    step = 1 << 25
    n = 0
    for lo in range(0, top + 1, step):
        bits = np.arange(lo, min(lo + step, top + 1), dtype=np.uint32)
        v = bits.view(np.float32)
        for sv in (v, -v):
            assert np.array_equal(oracle.e4m3_encode(sv), _torch_e4m3(sv)), f"chunk from {lo:#x}"
            n += sv.size
    assert n == 2 * (top + 1)
    big = np.array([448.0, np.nextafter(np.float32(448), np.float32(np.inf)), 480.0, 3.4e38, np.inf], np.float32)
    for sv in (big, -big):
        c = np.clip(sv, -448, 448).astype(np.float32)
        assert np.array_equal(oracle.e4m3_encode(c), _torch_e4m3(c))
        assert set(oracle.e4m3_encode(c).tolist()) == {0x7E if sv[0] > 0 else 0xFE}


def test_encode_tiny_values_round_to_signed_zero():
    v = np.array([1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10), 1e-40], dtype=np.float32)
    assert oracle.e4m3_encode(v).tolist() == [0x00, 0x80, 0x00, 0x80, 0x00]


# ----------------------------------------------------------------------------- UE8M0
def _exact_ceil_pow2_byte(amax: float) -> int:
    """smallest b with 2^(b-127) >= amax/448, in exact rational arithmetic."""
    r = Fraction(amax) / 448
    e = math.floor(math.log2(r))
    while Fraction(2) ** e < r:
        e += 1
    while Fraction(2) ** (e - 1) >= r:
        e -= 1
    return e + 127


def test_ue8m0_golden_values():
    rows = _read_golden("ue8m0_bytes.txt")
    amax = np.array([float(eval(a)) for a, _ in rows], dtype=np.float32)
    want = [int(b) for _, b in rows]
    assert oracle.ue8m0_byte(amax).tolist() == want


def test_ue8m0_is_smallest_power_of_two_over_every_bf16_amax():
    bits = (np.arange(0x0000, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    amax = bits[bits >= np.float32(1e-10)]
    got = oracle.ue8m0_byte(amax)
    # exact check through integer arithmetic: amax = mant * 2^exp2 with integers
    for a, g in zip(amax[::7].tolist(), got[::7].tolist()):
        assert g == _exact_ceil_pow2_byte(a)
    # vectorised exact check on all values: 2^(b-127) >= amax/448 > 2^(b-128)
    s = np.ldexp(1.0, got.astype(np.int64) - 127)
    a64 = amax.astype(np.float64)
    assert np.all(s * 448 >= a64) and np.all(s * 224 < a64)  # exact in fp64 (power-of-two scaling)


def test_ue8m0_near_seven_times_powers_of_two():
    # 448 = 7 * 64: amax near 7*2^k puts amax/448 next to a power of two
    vals = []
    for k in range(-30, 120):
        c = np.float32(7.0 * 2.0 ** k)
        if not np.isfinite(c):
            continue
        vals += [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(0))]
    vals = np.array(vals, dtype=np.float32)
    got = oracle.ue8m0_byte(vals)
    for a, g in zip(vals.tolist(), got.tolist()):
        assert g == _exact_ceil_pow2_byte(a), a

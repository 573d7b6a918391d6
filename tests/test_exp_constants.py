"""The constants of the fixed exp sequence inside silu(g) * u, derived here from exact
rationals and compared with the hex-float literals written in the oracle and in the HIP
kernel.

The pages leave exp unspecified (sglang PR #30924 report, prhub, 实现拆解 item 1: the
fuse_silu_and_mul trait names the fusion, not its exp); the reading fixed in include/fp8q.h
is a Cody-Waite reduction by ln 2 and a degree-7 Taylor polynomial whose constants are the
fp32 values nearest to log2(e), ln 2, the remainder ln 2 - fl32(ln 2), and 1/k!. An accuracy
test against math.exp cannot tell a constant one ulp off; this one can: every literal must
equal the correctly rounded fp32 value of its exact definition.

ln 2 comes from a 60-digit Decimal evaluation (its error, < 10^-58, is checked to be far
from any fp32 rounding boundary), 1/k! from Fractions.
"""
import math
import os
import re
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "fp8q_oracle.c")
QUANT_MATH = os.path.join(ROOT, "fp8_group_quant_amd", "csrc", "quant_math.h")

_HEX = r"-?0x[0-9a-fA-F]\.[0-9a-fA-F]+p[+-]?\d+f"


def _ln2() -> Fraction:
    getcontext().prec = 60
    return Fraction(Decimal(2).ln())


def _round_f32(x: Fraction) -> tuple[float, Fraction]:
    """Nearest binary32 value of the rational x (ties to even), and the distance of x from
    the nearest rounding boundary (half-way point), in units of the result's ulp."""
    if x == 0:
        return 0.0, Fraction(1, 2)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:  # exact exponent: 2^e <= a < 2^(e+1)
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "normal range only"
    scaled = a / Fraction(2) ** (e - 23)  # in [2^23, 2^24)
    lo = math.floor(scaled)
    frac = scaled - lo
    m = lo + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1) else 0)
    margin = abs(frac - Fraction(1, 2))
    return sign * math.ldexp(m, e - 23), margin


def _derived() -> dict:
    ln2 = _ln2()
    log2e, m0 = _round_f32(1 / ln2)
    hi, m1 = _round_f32(ln2)
    lo, m2 = _round_f32(ln2 - Fraction(hi))
    # the 60-digit ln 2 is within 1e-58 of the true value: far from any rounding boundary
    for m in (m0, m1, m2):
        assert m > Fraction(1, 10 ** 20)
    out = {"log2e": log2e, "ln2_hi": hi, "ln2_lo": lo}
    for k in range(8):
        out[f"c{k}"], _ = _round_f32(Fraction(1, math.factorial(k)))
    return out


def _hexf(lit: str) -> float:
    return float.fromhex(lit.rstrip("f"))


def test_derivation_itself():
    d = _derived()
    # sanity of the derivation, independent of the sources: 1/k! for k <= 2 are exact
    assert d["c0"] == 1.0 and d["c1"] == 1.0 and d["c2"] == 0.5
    assert d["ln2_hi"] == float(np.float32(math.log(2.0)))
    assert abs(d["log2e"] - 1 / math.log(2.0)) < 2.0 ** -23
    assert d["ln2_lo"] < 0  # fl32(ln 2) lies above ln 2
    # rounding helper on known values: 1/3 -> 0x1.555556p-2 (rounds up), 0.1 -> 0x1.99999ap-4
    assert _round_f32(Fraction(1, 3))[0] == float.fromhex("0x1.555556p-2")
    assert _round_f32(Fraction(1, 10))[0] == float(np.float32(0.1))
    # ties go to the even mantissa
    assert _round_f32(Fraction(2 ** 24 + 1))[0] == 2.0 ** 24
    assert _round_f32(Fraction(2 ** 24 + 3))[0] == 2.0 ** 24 + 4


def test_oracle_literals_equal_their_definitions():
    src = open(ORACLE_C, encoding="utf-8").read()
    body = src[src.index("float ora_exp_spec("):]
    body = body[:body.index("\n}\n")]
    d = _derived()
    for name, want in d.items():
        m = re.search(r"const float " + name + r"\s*=\s*(" + _HEX + r")\s*;", body)
        assert m, f"oracle: no hex literal for {name}"
        got = _hexf(m.group(1))
        assert got == want, f"oracle {name}: {got.hex()} != nearest fp32 {want.hex()}"


def test_kernel_literals_equal_their_definitions():
    src = open(QUANT_MATH, encoding="utf-8").read()
    body = src[src.index("float exp_fixed(float t)"):]
    body = body[:body.index("\n}\n")]
    code = "\n".join(re.sub(r"//.*$", "", line) for line in body.splitlines())
    lits = [_hexf(x) for x in re.findall(_HEX, code)]
    d = _derived()
    # order of use: log2e, ln2_hi, ln2_lo, then Horner from 1/7! down to 1/2!; 1/1! and
    # 1/0! are written as 1.0f
    want = [d["log2e"], d["ln2_hi"], d["ln2_lo"]] + [d[f"c{k}"] for k in range(7, 1, -1)]
    assert lits == want, [v.hex() for v in lits]
    assert len(re.findall(r"fmaf\(p, r, 1\.0f\)", code)) == 2
    assert d["c1"] == 1.0 and d["c0"] == 1.0

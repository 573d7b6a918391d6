"""The short correctly rounded fp32 forms used by the quantization kernels (csrc/quant_math.h),
checked on every fp32 input of their stated domains.

The silu quotient g / (1 + exp(-g)), the scale amax / 448 (or / 127) and its reciprocal are
computed in the kernels by shorter instruction sequences than the general IEEE division. Their
results must be the correctly rounded quotients, bit for bit, or the quantizer would no longer
match the oracle. The bench library's fp8q_check_division runs each short form and the
compiler's IEEE operation on all 2^32 bit patterns and counts disagreements; the exp case
checks that scaling by v_ldexp_f32 equals the multiply by 2^n that the exp sequence states,
and the int8 case that the one-add encode gives the code of the clamp, rint and conversion.
"""
import ctypes
import os

import pytest
import torch

from fp8_group_quant_amd import build

pytestmark = pytest.mark.gpu

_EPS_BITS = 0x2EDBE6FF   # 1e-10f, the amax floor
_LO_BITS = 0x29E12E13    # 1e-13f
_HI_BITS = 0x7CF0BDC2    # 1e37f
_NAN_PER_SIGN = 0x7FFFFF

# inputs each check covers (both signs of the bit patterns)
EXPECTED_CHECKED = {
    0: (1 << 31) + (0x42AE0000 + 1) + _NAN_PER_SIGN,           # every g >= -87 (bits of 87.0f)
    1: 2 * ((1 << 31) - _EPS_BITS),                             # every |x| >= 1e-10, inf, NaN
    2: 2 * ((1 << 31) - _EPS_BITS),
    3: 2 * ((_HI_BITS - _LO_BITS + 1) + 1 + _NAN_PER_SIGN),     # [1e-13, 1e37], inf, NaN
    4: 1 << 32,
    5: 1 << 32,
}


def _lib():
    if not os.path.exists(build.BENCH_LIB):
        pytest.fail(f"{build.BENCH_LIB} is not built")
    lib = ctypes.CDLL(build.BENCH_LIB)
    lib.fp8q_check_division.restype = ctypes.c_int
    lib.fp8q_check_division.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("which", [0, 1, 2, 3, 4, 5],
                         ids=["silu_quotient", "amax_div_448", "amax_div_127", "reciprocal", "exp_ldexp",
                              "int8_code"])
def test_short_form_matches_ieee_on_every_input(which):
    lib = _lib()
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    rc = lib.fp8q_check_division(which, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    bad, checked = (int(v) for v in out.cpu())
    assert checked == EXPECTED_CHECKED[which]
    assert bad == 0, f"{bad} inputs disagree"


def test_rejects_unknown_check():
    lib = _lib()
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    assert lib.fp8q_check_division(6, out.data_ptr(), None) != 0
    assert lib.fp8q_check_division(0, None, None) != 0

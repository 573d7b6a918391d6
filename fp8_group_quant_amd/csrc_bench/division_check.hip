// division_check.hip — exhaustive check of the short fp32 forms in csrc/quant_math.h (the
// divisions, the exp's scaling step and the int8 encode)
// (libfp8q_bench.so; run by the tests, not part of the fp8q boundary).
//
// For every one of the 2^32 fp32 bit patterns x that falls in a form's domain, the short
// form is compared with the compiler's correctly rounded IEEE operation (this file is built
// with the library's flags: -fhip-fp32-correctly-rounded-divide-sqrt, no contraction, fp32
// denormals on). Two results agree when their bits are equal or both are NaN.
//   which 0  silu quotient  div_short(g, d) vs g / d, d = 1 + exp_fixed(-g);  domain !(g < -87)
//   which 1  amax / 448     div_by_const<448>(a) vs a / 448, a = |x|;        domain !(a < 1e-10)
//   which 2  amax / 127     div_by_const<127>(a) vs a / 127, a = |x|;        domain !(a < 1e-10)
//   which 3  1 / r          div_short(1, r) vs 1 / r, r = |x|;   domain r in [1e-13, 1e37], inf, NaN
//   which 4  exp_fixed      ldexp form vs p * 2^n with 2^n built from its exponent bits; all x
//   which 5  int8 code      low byte of int8_code_bits(x) vs (int)rint(clamp(x, +-127)); all x
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "quant_math.h"

#pragma clang fp contract(off)

namespace {

constexpr float kEps = 0x1.b7cdfep-34f;  // 1e-10f, the amax floor of the quantizer

__device__ __forceinline__ bool agree(float a, float b) {
  return __float_as_uint(a) == __float_as_uint(b) || (a != a && b != b);
}

// exp_fixed with the final scaling written as a multiply by 2^n (the plain form of the step)
__device__ __forceinline__ float exp_mul_form(float t) {
  t = fminf(fmaxf(t, -87.0f), 88.0f);
  const float n = rintf(t * 0x1.715476p+0f);
  float r = fmaf(-n, 0x1.62e430p-1f, t);
  r = fmaf(-n, -0x1.05c610p-29f, r);
  float p = 0x1.a01a02p-13f;
  p = fmaf(p, r, 0x1.6c16c2p-10f);
  p = fmaf(p, r, 0x1.111112p-7f);
  p = fmaf(p, r, 0x1.555556p-5f);
  p = fmaf(p, r, 0x1.555556p-3f);
  p = fmaf(p, r, 0x1.000000p-1f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return p * __uint_as_float(static_cast<uint32_t>(static_cast<int>(n) + 127) << 23);
}

__global__ __launch_bounds__(256) void check_division(int which, unsigned long long* out) {
  unsigned long long bad = 0, checked = 0;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 256;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x; i < (1ull << 32); i += stride) {
    const float x = __uint_as_float(static_cast<uint32_t>(i));
    const float a = fabsf(x);
    bool in = true, ok = true;
    if (which == 0) {
      in = !(x < -87.0f);
      if (in) {
        const float d = 1.0f + fp8q::exp_fixed(-x);
        ok = agree(fp8q::div_short(x, d), x / d);
      }
    } else if (which == 1 || which == 2) {
      in = !(a < kEps);
      if (in) ok = which == 1 ? agree(fp8q::div_by_const<448>(a), a / 448.0f)
                              : agree(fp8q::div_by_const<127>(a), a / 127.0f);
    } else if (which == 3) {
      in = (a >= 1e-13f && a <= 1e37f) || a == __builtin_inff() || a != a;
      if (in) ok = agree(fp8q::div_short(1.0f, a), 1.0f / a);
    } else if (which == 4) {
      ok = agree(fp8q::exp_fixed(x), exp_mul_form(x));
    } else {
      const uint32_t want = static_cast<uint32_t>(static_cast<int>(rintf(fminf(fmaxf(x, -127.0f), 127.0f)))) & 0xFFu;
      ok = (fp8q::int8_code_bits(x) & 0xFFu) == want;
    }
    checked += in ? 1 : 0;
    bad += (in && !ok) ? 1 : 0;
  }
  atomicAdd(out, bad);
  atomicAdd(out + 1, checked);
}

}  // namespace

extern "C" {

// which in 0..5 (see above). out: device array of two zeroed unsigned 64-bit counters that
// receive (mismatches, inputs checked). Returns 0 or a HIP error code.
int fp8q_check_division(int which, void* out, void* stream) {
  if (which < 0 || which > 5 || out == nullptr) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(check_division, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream), which,
                     static_cast<unsigned long long*>(out));
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"

// quant_math.h — the fp32 arithmetic of the quantization kernels that is more than one
// instruction: the fixed exp of the fused silu, correctly rounded division in short forms, and
// the int8 encode.
//
// Every function here returns exactly the value its plain definition gives (the fixed exp
// sequence, the correctly rounded quotient, the rounded int8 code); the short forms only take
// fewer instructions.
// Each domain stated below was checked on every fp32 input against the compiler's IEEE
// division by fp8q_check_division in the benchmark library (csrc_bench/division_check.hip).
//
// Compile without contraction (-ffp-contract=off) and with fp32 denormals enabled (the HIP
// default for gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// exp(t) as a fixed fp32 sequence: Cody-Waite reduction by ln 2 (two-part constant, fma),
// degree-7 Taylor polynomial in Horner form (fma), scaling by 2^n. Constants are the fp32
// values nearest to log2(e), ln 2, the remainder of ln 2, and 1/k!. After the clamp n lies in
// [-126, 127], so 2^n is a normal fp32 value and v_ldexp_f32 returns the correctly rounded
// p * 2^n, the same value as a multiply by 2^n.
__device__ __forceinline__ float exp_fixed(float t) {
  t = fminf(fmaxf(t, -87.0f), 88.0f);
  const float n = rintf(t * 0x1.715476p+0f);
  float r = fmaf(-n, 0x1.62e430p-1f, t);
  r = fmaf(-n, -0x1.05c610p-29f, r);
  float p = 0x1.a01a02p-13f;        // 1/7!
  p = fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
  p = fmaf(p, r, 0x1.111112p-7f);   // 1/5!
  p = fmaf(p, r, 0x1.555556p-5f);   // 1/4!
  p = fmaf(p, r, 0x1.555556p-3f);   // 1/3!
  p = fmaf(p, r, 0x1.000000p-1f);   // 1/2!
  p = fmaf(p, r, 1.0f);             // 1/1!
  p = fmaf(p, r, 1.0f);             // 1/0!
  return __builtin_amdgcn_ldexpf(p, static_cast<int>(n));
}

// a / b correctly rounded, in 7 instructions (the general sequence takes 12). One Newton step
// takes the hardware reciprocal (v_rcp_f32, within 1 ulp) to y = RN(1/b); the quotient a * y
// is then corrected once by its exact fma residual, which gives RN(a / b) when y = RN(1/b) and
// the first quotient is within an ulp (Markstein's theorem; Muller et al., Handbook of
// Floating-Point Arithmetic, ch. 4). v_div_fixup_f32 gives the IEEE results for infinite, NaN
// and zero operands. The theorem needs 1/b and a / b clear of the subnormal range, so callers
// keep to checked domains:
//   - b = 1 + exp_fixed(-a) with a >= -87 (the fused silu), and a NaN;
//   - a = 1 and b in [1e-13, 1e37], infinite or NaN (the reciprocal of a scale).
__device__ __forceinline__ float div_short(float a, float b) {
  float y = __builtin_amdgcn_rcpf(b);
  const float e = fmaf(-b, y, 1.0f);
  y = fmaf(e, y, y);
  float q = a * y;
  const float r = fmaf(-b, q, a);
  q = fmaf(r, y, q);
  return __builtin_amdgcn_div_fixupf(q, b, a);
}

// a / C for the integer constant C, correctly rounded: as div_short with y = RN(1/C) folded
// at compile time. Checked domain (C = 448 and 127): a >= 1e-10 (the amax floor), including
// infinity and NaN.
template <int C>
__device__ __forceinline__ float div_by_const(float a) {
  constexpr float kC = static_cast<float>(C);
  constexpr float kInv = 1.0f / kC;  // correctly rounded by the compiler
  float q = a * kInv;
  const float r = fmaf(-kC, q, a);
  q = fmaf(r, kInv, q);
  return __builtin_amdgcn_div_fixupf(q, kC, a);
}

// The int8 code of v (clamped to +-127, rounded to the nearest integer with ties to even) in
// the low byte of the result, in two's complement. After the clamp the fp32 sum
// v + 1.5 * 2^23 lies in [2^23, 2^24), where the spacing is 1, so the add itself rounds v to an
// integer n (ties to even, the value rint gives) and the sum's bits are 0x4B400000 + n.
// Checked on all 2^32 inputs against the clamp followed by rint and a conversion.
__device__ __forceinline__ uint32_t int8_code_bits(float v) {
  return __float_as_uint(fminf(fmaxf(v, -127.0f), 127.0f) + 0x1.8p23f);
}

}  // namespace fp8q

// api_quant.hip — C ABI of the group-quant calls: argument validation (host only, before
// any device call), the device check, then the launch. Semantics: include/fp8q.h.
#include "fp8q_internal.h"

namespace fp8q {
namespace {

constexpr int64_t kMaxMaskedExperts = 4096;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int quant_entry(const void* x, int in_dtype, int64_t E, int64_t M, int64_t K, int64_t x_se,
                int64_t x_sm, uint8_t* q, int64_t q_se, int64_t q_sm, void* s, int scale_fmt,
                int64_t s_se, int64_t s_sm, int64_t s_sg, int group_size, const int32_t* masked_m,
                int64_t expected_m, void* stream, bool silu, bool i8) {
  set_error("");
  const char* fn = i8 ? "fp8q_group_quant_int8" : (silu ? "fp8q_silu_mul_group_quant" : "fp8q_group_quant");
  const std::string pre = std::string(fn) + ": ";
  if (in_dtype != FP8Q_DTYPE_BF16 && in_dtype != FP8Q_DTYPE_F16 && in_dtype != FP8Q_DTYPE_F32)
    return fail(FP8Q_EUNSUPPORTED, pre + "in_dtype must be BF16, F16 or F32");
  if (scale_fmt != FP8Q_SCALE_F32 && scale_fmt != FP8Q_SCALE_UE8M0 && scale_fmt != FP8Q_SCALE_UE8M0_PACKED)
    return fail(FP8Q_EUNSUPPORTED, pre + "scale_fmt must be F32, UE8M0 or UE8M0_PACKED");
  if (i8 && scale_fmt != FP8Q_SCALE_F32) return fail(FP8Q_EUNSUPPORTED, pre + "int8 output takes F32 scales");
  if (E < 0 || M < 0 || K < 0) return fail(FP8Q_EINVAL, pre + "negative size");
  const bool per_token = group_size > 0 && group_size == K && group_size != 32 && group_size != 64 && group_size != 128;
  if (group_size != 32 && group_size != 64 && group_size != 128 && !per_token)
    return fail(FP8Q_EUNSUPPORTED, pre + "group_size must be 32, 64, 128 or K (per-token)");
  if (per_token && K % 16 != 0) return fail(FP8Q_EINVAL, pre + "per-token quantization needs K % 16 == 0");
  if (per_token && K > (int64_t(1) << 30)) return fail(FP8Q_EUNSUPPORTED, pre + "per-token rows are limited to 2^30 elements");
  if (x_se < 0 || x_sm < 0 || q_se < 0 || q_sm < 0 || s_se < 0 || s_sm < 0 || s_sg < 0)
    return fail(FP8Q_EINVAL, pre + "negative stride");
  if (expected_m < 0) return fail(FP8Q_EINVAL, pre + "expected_m must be >= 0");
  if (K % group_size != 0) return fail(FP8Q_EINVAL, pre + "K must be a multiple of group_size");
  const bool packed = scale_fmt == FP8Q_SCALE_UE8M0_PACKED;
  if (packed && (K / group_size) % 4 != 0)
    return fail(FP8Q_EINVAL, pre + "packed UE8M0 scales need a multiple of 4 groups per row");
  if (masked_m && E > kMaxMaskedExperts)
    return fail(FP8Q_EUNSUPPORTED, pre + "masked dispatch supports at most 4096 experts");
  if (masked_m && E * M >= (int64_t(1) << 31))
    return fail(FP8Q_EUNSUPPORTED, pre + "masked dispatch needs E * M < 2^31");
  if (E == 0 || M == 0 || K == 0) return FP8Q_OK;
  if (!x || !q || !s) return fail(FP8Q_EINVAL, pre + "null tensor pointer");

  const int64_t width = silu ? 2 * K : K;  // input row length
  const int64_t ng = packed ? K / group_size / 4 : K / group_size;  // scale elements per row
  const int64_t esz = in_dtype == FP8Q_DTYPE_F32 ? 4 : 2;
  // outputs must not overlap themselves (inputs may)
  if (M > 1 && q_sm < K) return fail(FP8Q_EINVAL, pre + "q rows overlap (q_sm < K)");
  if (E > 1 && q_se < (M - 1) * q_sm + K) return fail(FP8Q_EINVAL, pre + "q experts overlap");
  if (M > 1 && x_sm < width) return fail(FP8Q_EINVAL, pre + "x rows overlap (x_sm < row width)");
  const bool row_major = s_sg == 1 && (M <= 1 || s_sm >= ng);
  const bool col_major = s_sm == 1 && (ng <= 1 || s_sg >= M);
  if (!row_major && !col_major)
    return fail(FP8Q_EINVAL, pre + "scale strides are neither row-major (s_sg == 1) nor column-major (s_sm == 1)");
  const int64_t s_extent = row_major ? (M - 1) * s_sm + ng : (ng - 1) * s_sg + M;
  if (E > 1 && s_se < s_extent) return fail(FP8Q_EINVAL, pre + "scale experts overlap");
  if (!aligned16(x) || (x_sm * esz) % 16 != 0 || (x_se * esz) % 16 != 0)
    return fail(FP8Q_EALIGN, pre + "x and its row/expert strides must be 16-byte aligned");
  if (!aligned16(q) || q_sm % 16 != 0 || q_se % 16 != 0)
    return fail(FP8Q_EALIGN, pre + "q and its row/expert strides must be 16-byte aligned");
  if (scale_fmt != FP8Q_SCALE_UE8M0 && (reinterpret_cast<uintptr_t>(s) & 3u) != 0)
    return fail(FP8Q_EALIGN, pre + "fp32 scales and packed UE8M0 words must be 4-byte aligned");

  const int dev = check_current_device();
  if (dev != FP8Q_OK) return dev;

  QuantParams p{};
  p.x = x;
  p.q = q;
  p.s = s;
  p.masked_m = masked_m;
  p.E = E;
  p.M = M;
  p.K = K;
  p.x_se = x_se;
  p.x_sm = x_sm;
  p.q_se = q_se;
  p.q_sm = q_sm;
  p.s_se = s_se;
  p.s_sm = s_sm;
  p.s_sg = s_sg;
  p.packed = packed ? 1 : 0;
  return launch_group_quant(in_dtype, packed ? FP8Q_SCALE_UE8M0 : scale_fmt, group_size, silu, i8, p, expected_m,
                            static_cast<hipStream_t>(stream));
}

}  // namespace
}  // namespace fp8q

extern "C" {

int fp8q_group_quant(const void* x, int in_dtype, int64_t E, int64_t M, int64_t K, int64_t x_se,
                     int64_t x_sm, uint8_t* q, int64_t q_se, int64_t q_sm, void* s, int scale_fmt,
                     int64_t s_se, int64_t s_sm, int64_t s_sg, int group_size,
                     const int32_t* masked_m, int64_t expected_m, void* stream) {
  return fp8q::quant_entry(x, in_dtype, E, M, K, x_se, x_sm, q, q_se, q_sm, s, scale_fmt, s_se, s_sm,
                           s_sg, group_size, masked_m, expected_m, stream, false, false);
}

int fp8q_silu_mul_group_quant(const void* x, int in_dtype, int64_t E, int64_t M, int64_t K,
                              int64_t x_se, int64_t x_sm, uint8_t* q, int64_t q_se, int64_t q_sm,
                              void* s, int scale_fmt, int64_t s_se, int64_t s_sm, int64_t s_sg,
                              int group_size, const int32_t* masked_m, int64_t expected_m,
                              void* stream) {
  return fp8q::quant_entry(x, in_dtype, E, M, K, x_se, x_sm, q, q_se, q_sm, s, scale_fmt, s_se, s_sm,
                           s_sg, group_size, masked_m, expected_m, stream, true, false);
}

int fp8q_group_quant_int8(const void* x, int in_dtype, int64_t E, int64_t M, int64_t K, int64_t x_se,
                          int64_t x_sm, int8_t* q, int64_t q_se, int64_t q_sm, float* s, int scale_fmt,
                          int64_t s_se, int64_t s_sm, int64_t s_sg, int group_size,
                          const int32_t* masked_m, int64_t expected_m, void* stream) {
  return fp8q::quant_entry(x, in_dtype, E, M, K, x_se, x_sm, reinterpret_cast<uint8_t*>(q), q_se, q_sm, s,
                           scale_fmt, s_se, s_sm, s_sg, group_size, masked_m, expected_m, stream, false, true);
}

}  // extern "C"

/*
 * fp8q_oracle.c — plain, slow CPU oracle for per-token-group FP8 quantization and
 * block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * constant with the HIP library: everything here is written out from the sources
 * cited below and from the definitions of the number formats.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared (see
 * build.py). All float arithmetic is IEEE-754 binary32/binary64 with round-to-nearest-even;
 * no contraction into fused multiply-add except where fmaf() is written explicitly.
 * The only parallelism is an OpenMP loop over independent rows (quantization) or output
 * elements (GEMM): each result is computed by one thread with the same sequential
 * arithmetic, so results do not depend on the thread count (ora_set_threads).
 *
 * Sources:
 *   [PR30924] prhub report of sglang PR #30924 "[JIT] Trait-driven per_token_group_quant:
 *             unify the quant kernel family (flat + masked)": section "实现拆解" items 1-2 and
 *             section "关键源码片段" (the test reference ref_fp8_ue8m0: group amax floored at
 *             EPS, division by FMAX = 448, the UE8M0 exponent rounded up from the fp32 bits,
 *             multiplier 2^(254-e) built from bits, clamp to +-448 then cast to e4m3fn).
 *   [TF]      TeleFuser "tf-kernel 安装与使用": silu_and_mul splits the last dimension into
 *             two halves; per-token FP8 output into caller-allocated tensors.
 *   [FI]      "FlashInfer GEMM 学习笔记" sections 6-7: FP8 e4m3 operands, block-scaled
 *             (MXFP8 block 32) and DeepSeek-style groupwise NT GEMM.
 *   OCP 8-bit floating point specification: the E4M3 (fn) and E8M0 encodings.
 *
 * Readings where the sources are silent (each also listed in the design notes):
 *   - EPS (the amax floor) is not printed: 1e-10f is used.
 *   - The fp32-scale reference body is not printed: s = amax/448 is stored and the
 *     multiplier is 1/s (IEEE), the same "multiply by the reciprocal of the stored
 *     scale" shape as the printed UE8M0 reference.
 *   - Rounding to e4m3 is round-to-nearest, ties to even mantissa, after the clamp.
 *   - exp inside silu is a fixed fp32 sequence (declared in fp8q.h and ora_exp_spec).
 *   - Per-token quantization ([TF] per-token FP8 example: scale [M, 1]) is the group rule
 *     with one group spanning the whole row (G = K).
 *   - The int8 output ([PR30924] 关键文件: the ref_int8 test reference; 风险与影响: int8
 *     codes that move by one when the division is approximate) is not printed: the same
 *     shape as the fp32-scale rule with 127 in place of 448, i.e. s = amax/127 stored as
 *     fp32, multiplier 1/s, clamp to +-127, round to the nearest integer with ties to
 *     even, stored as a two's-complement byte. fp32 scales only.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------
 * OCP E4M3FN codec
 * byte = s eeee mmm, bias 7. e == 0: subnormal m * 2^-9. e == 15 && m == 7: NaN.
 * otherwise (1 + m/8) * 2^(e-7). Largest finite value 0x7E = 1.75 * 2^8 = 448.
 * ---------------------------------------------------------------------------------- */
double ora_e4m3_decode(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = (double)m * ldexp(1.0, -9);
  else
    mag = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
  return s ? -mag : mag;
}

/* The values of the 127 non-negative finite codes, in code order: ora_e4m3_decode of each
 * (filled once when the library loads, so the search below does not decode 127 codes for
 * every value). */
static double ora_e4m3_values[0x7F];

__attribute__((constructor)) static void ora_fill_e4m3_values(void) {
  for (int c = 0; c <= 0x7E; c++) ora_e4m3_values[c] = ora_e4m3_decode((uint8_t)c);
}

/* Nearest finite e4m3 value to v, ties to the even code (the code's low bit is the low
 * mantissa bit). v must be finite with |v| <= 448 (the caller clamps first). The search
 * walks the 127 non-negative finite codes in increasing order of value, and stops at the
 * first code farther above |v| than the nearest one so far: every later code is farther
 * still (a code exactly as far is still compared, for the tie rule). */
uint8_t ora_e4m3_encode(float v) {
  double a = fabs((double)v);
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; c++) {
    if (ora_e4m3_values[c] - a > bestd) break;
    double d = fabs(ora_e4m3_values[c] - a);
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)((signbit(v) ? 0x80 : 0x00) | best);
}

/* ------------------------------------------------------------------------------------
 * int8 code: nearest integer, ties to the even integer. v must be finite with
 * |v| <= 127 (the caller clamps first). Written out with floor so the tie rule is visible.
 * ---------------------------------------------------------------------------------- */
int8_t ora_int8_encode(float v) {
  double d = (double)v; /* exact */
  double f = floor(d);
  double frac = d - f; /* exact: f and d are within one unit */
  double r;
  if (frac > 0.5)
    r = f + 1.0;
  else if (frac < 0.5)
    r = f;
  else
    r = (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
  return (int8_t)(int)r;
}

/* ------------------------------------------------------------------------------------
 * input dtypes
 * ---------------------------------------------------------------------------------- */
float ora_bf16_to_f32(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16; /* bf16 is the top half of a binary32 */
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

float ora_f16_to_f32(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double mag;
  if (e == 31)
    mag = m ? NAN : INFINITY;
  else if (e == 0)
    mag = (double)m * ldexp(1.0, -24);
  else
    mag = (1.0 + (double)m / 1024.0) * ldexp(1.0, e - 15);
  return (float)(s ? -mag : mag); /* exact: every binary16 value is a binary32 value */
}

enum { ORA_BF16 = 0, ORA_F16 = 1, ORA_F32 = 2 };
enum { ORA_SCALE_F32 = 0, ORA_SCALE_UE8M0 = 1 };

static float load_elem(const void* base, int dtype, int64_t idx) {
  if (dtype == ORA_BF16) return ora_bf16_to_f32(((const uint16_t*)base)[idx]);
  if (dtype == ORA_F16) return ora_f16_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

/* ------------------------------------------------------------------------------------
 * group scale  [PR30924 ref_fp8_ue8m0]
 * ---------------------------------------------------------------------------------- */
#define ORA_FMAX 448.0f
#define ORA_IMAX 127.0f /* int8 output: largest code used */
#define ORA_EPS 1e-10f

/* UE8M0 byte: fp32 r = amax / 448; exponent field of r, plus one when r's mantissa
 * field is non-zero (i.e. round the power of two up). */
uint8_t ora_ue8m0_byte(float amax) {
  float r = amax / ORA_FMAX;
  uint32_t bits;
  memcpy(&bits, &r, 4);
  uint32_t e = ((bits >> 23) & 0xFFu) + ((bits & 0x7FFFFFu) != 0u ? 1u : 0u);
  return (uint8_t)e;
}

/* Multiplier for a UE8M0 byte e: the float whose exponent field is 254 - e, i.e.
 * 2^(127 - (e - 127)) = 1 / 2^(e-127), exactly. */
float ora_ue8m0_multiplier(uint8_t e) {
  uint32_t bits = (uint32_t)(254 - (int)e) << 23;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

/* ------------------------------------------------------------------------------------
 * exp and silu, fixed fp32 sequence (Cody-Waite reduction + degree-7 Taylor/Horner)
 * Constants: fp32 nearest to log2(e); ln 2 split into the fp32 nearest to ln 2 and the
 * fp32 nearest to the remainder; fp32 nearest to 1/k!.
 * ---------------------------------------------------------------------------------- */
float ora_exp_spec(float t) {
  const float log2e = 0x1.715476p+0f;
  const float ln2_hi = 0x1.62e430p-1f;
  const float ln2_lo = -0x1.05c610p-29f;
  const float c0 = 0x1.000000p+0f;  /* 1/0! */
  const float c1 = 0x1.000000p+0f;  /* 1/1! */
  const float c2 = 0x1.000000p-1f;  /* 1/2! */
  const float c3 = 0x1.555556p-3f;  /* 1/3! */
  const float c4 = 0x1.555556p-5f;  /* 1/4! */
  const float c5 = 0x1.111112p-7f;  /* 1/5! */
  const float c6 = 0x1.6c16c2p-10f; /* 1/6! */
  const float c7 = 0x1.a01a02p-13f; /* 1/7! */
  if (t < -87.0f) t = -87.0f;
  if (t > 88.0f) t = 88.0f;
  float n = rintf(t * log2e); /* in [-126, 127] after the clamp */
  float r = fmaf(-n, ln2_hi, t);
  r = fmaf(-n, ln2_lo, r);
  float p = c7;
  p = fmaf(p, r, c6);
  p = fmaf(p, r, c5);
  p = fmaf(p, r, c4);
  p = fmaf(p, r, c3);
  p = fmaf(p, r, c2);
  p = fmaf(p, r, c1);
  p = fmaf(p, r, c0);
  uint32_t bits = (uint32_t)((int)n + 127) << 23; /* 2^n, a normal float */
  float two_n;
  memcpy(&two_n, &bits, 4);
  return p * two_n;
}

/* silu(g) * u in fp32: g / (1 + exp(-g)), then times u. */
float ora_silu_mul(float g, float u) {
  float d = 1.0f + ora_exp_spec(-g);
  float sg = g / d;
  return sg * u;
}

/* ------------------------------------------------------------------------------------
 * group quantization of one row  [PR30924 items 1-2, ref_fp8_ue8m0; TF]
 * row_in points at element (e, m, 0); with silu the row holds 2K elements
 * (gate = [0, K), up = [K, 2K)). vals is caller scratch of at least G floats.
 * out_int8: int8 codes and fp32 scales s = amax/127 (reading above); otherwise e4m3.
 * ---------------------------------------------------------------------------------- */
static void quant_row(const void* x, int in_dtype, int64_t row_off, int64_t K, int silu,
                      uint8_t* q_row, void* s, int scale_fmt, int64_t s_row_off, int64_t s_sg,
                      int64_t G, int out_int8, float* vals) {
  int64_t ngroups = K / G;
  float qmax = out_int8 ? ORA_IMAX : ORA_FMAX;
  for (int64_t g = 0; g < ngroups; g++) {
    /* values of this group, in fp32 */
    for (int64_t i = 0; i < G; i++) {
      int64_t k = g * G + i;
      if (silu)
        vals[i] = ora_silu_mul(load_elem(x, in_dtype, row_off + k),
                               load_elem(x, in_dtype, row_off + K + k));
      else
        vals[i] = load_elem(x, in_dtype, row_off + k);
    }
    /* group absmax, not below EPS */
    float amax = 0.0f;
    for (int64_t i = 0; i < G; i++) {
      float a = fabsf(vals[i]);
      if (a > amax) amax = a;
    }
    if (amax < ORA_EPS) amax = ORA_EPS;
    /* scale and multiplier */
    float inv;
    int64_t sidx = s_row_off + g * s_sg;
    if (scale_fmt == ORA_SCALE_UE8M0) {
      uint8_t e = ora_ue8m0_byte(amax);
      ((uint8_t*)s)[sidx] = e;
      inv = ora_ue8m0_multiplier(e);
    } else {
      float sc = amax / qmax;
      ((float*)s)[sidx] = sc;
      inv = 1.0f / sc;
    }
    /* multiply, clamp to [-qmax, qmax], round to the output code */
    for (int64_t i = 0; i < G; i++) {
      float v = vals[i] * inv;
      if (v > qmax) v = qmax;
      if (v < -qmax) v = -qmax;
      if (out_int8)
        q_row[g * G + i] = (uint8_t)ora_int8_encode(v);
      else
        q_row[g * G + i] = ora_e4m3_encode(v);
    }
  }
}

/* Mirrors fp8q_group_quant / fp8q_silu_mul_group_quant (out_int8 = 0) and
 * fp8q_group_quant_int8 (out_int8 = 1) on host memory. G is 32, 64, 128, or K (one group
 * per row: per-token quantization). masked_m is a host int32[E] or NULL (flat). If
 * rows_e/rows_m are non-NULL only those n_rows rows are processed (they must be rows the
 * call would process); otherwise all rows are. Returns 0, or -1 for arguments the oracle
 * does not handle. */
int ora_group_quant(const void* x, int in_dtype, int64_t E, int64_t M, int64_t K,
                    int64_t x_se, int64_t x_sm, uint8_t* q, int64_t q_se, int64_t q_sm,
                    void* s, int scale_fmt, int64_t s_se, int64_t s_sm, int64_t s_sg,
                    int64_t G, const int32_t* masked_m, int silu, int out_int8,
                    const int64_t* rows_e, const int64_t* rows_m, int64_t n_rows) {
  if (G != 32 && G != 64 && G != 128 && G != K) return -1;
  if (G <= 0 || K % G != 0) return -1;
  if (out_int8 && scale_fmt != ORA_SCALE_F32) return -1;
  int failed = 0;
  /* rows are independent: one thread quantizes a whole row */
#pragma omp parallel
  {
    float* vals = (float*)malloc((size_t)G * sizeof(float));
    if (!vals) {
#pragma omp atomic write
      failed = 1;
    }
    if (vals && rows_e && rows_m) {
#pragma omp for schedule(dynamic, 4)
      for (int64_t i = 0; i < n_rows; i++) {
        int64_t e = rows_e[i], m = rows_m[i];
        quant_row(x, in_dtype, e * x_se + m * x_sm, K, silu, q + e * q_se + m * q_sm, s,
                  scale_fmt, e * s_se + m * s_sm, s_sg, G, out_int8, vals);
      }
    } else if (vals) {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < E * M; r++) {
        int64_t e = r / M, m = r % M;
        int64_t rows = M;
        if (masked_m) {
          rows = masked_m[e];
          if (rows < 0) rows = 0;
          if (rows > M) rows = M;
        }
        if (m < rows)
          quant_row(x, in_dtype, e * x_se + m * x_sm, K, silu, q + e * q_se + m * q_sm, s,
                    scale_fmt, e * s_se + m * s_sm, s_sg, G, out_int8, vals);
      }
    }
    free(vals);
  }
  return failed ? -1 : 0;
}

/* Thread count of the OpenMP loops (n >= 1), and the count they will use. */
void ora_set_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
}

int ora_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------------------
 * block-scaled GEMM: dequantize, then multiply, in fp64  [FI sections 6-7]
 * Y*[m][n] = sum_k (dec(a[m][k]) * sa(m, k)) * (dec(b[n][k]) * sb(n, k))
 * BLOCK128: sa(m, k) = scale at (m, k/128); sb(n, k) = scale at (n/128, k/128).
 * MX32:     sa(m, k) = 2^(byte(m, k/32) - 127); sb(n, k) = 2^(byte(n, k/32) - 127).
 * Also returns S[m][n] = sum_k |term|, used by the tests' rounding-error bound.
 * ---------------------------------------------------------------------------------- */
static double scale_value(const void* s, int fmt, int64_t idx) {
  if (fmt == ORA_SCALE_UE8M0) return ldexp(1.0, (int)((const uint8_t*)s)[idx] - 127);
  return (double)((const float*)s)[idx];
}

enum { ORA_GEMM_BLOCK128 = 0, ORA_GEMM_MX32 = 1 };

static void gemm_elem(const uint8_t* a, int64_t lda, const void* sa, int sa_fmt, int64_t sa_sm,
                      int64_t sa_sk, const uint8_t* b, int64_t ldb, const void* sb, int sb_fmt,
                      int64_t sb_sn, int64_t sb_sk, int64_t K, int mode, const double* dec,
                      int64_t m, int64_t n, double* y_out, double* s_out) {
  double acc = 0.0, sabs = 0.0;
  for (int64_t k = 0; k < K; k++) {
    double fa, fb;
    if (mode == ORA_GEMM_MX32) {
      fa = scale_value(sa, ORA_SCALE_UE8M0, m * sa_sm + (k / 32) * sa_sk);
      fb = scale_value(sb, ORA_SCALE_UE8M0, n * sb_sn + (k / 32) * sb_sk);
    } else {
      fa = scale_value(sa, sa_fmt, m * sa_sm + (k / 128) * sa_sk);
      fb = scale_value(sb, sb_fmt, (n / 128) * sb_sn + (k / 128) * sb_sk);
    }
    double av = dec[a[m * lda + k]] * fa;
    double bv = dec[b[n * ldb + k]] * fb;
    double t = av * bv;
    acc += t;
    sabs += fabs(t);
  }
  *y_out = acc;
  *s_out = sabs;
}

/* Computes Y* and S for the listed (ms[i], ns[i]) elements, or for all M x N elements
 * (row-major into y_out / s_out) when ms == NULL. */
int ora_gemm(const uint8_t* a, int64_t lda, const void* sa, int sa_fmt, int64_t sa_sm,
             int64_t sa_sk, const uint8_t* b, int64_t ldb, const void* sb, int sb_fmt,
             int64_t sb_sn, int64_t sb_sk, int64_t M, int64_t N, int64_t K, int mode,
             const int64_t* ms, const int64_t* ns, int64_t count, double* y_out,
             double* s_out) {
  double dec[256];
  for (int c = 0; c < 256; c++) dec[c] = ora_e4m3_decode((uint8_t)c);
  if (mode != ORA_GEMM_BLOCK128 && mode != ORA_GEMM_MX32) return -1;
  /* output elements are independent: one thread computes each whole sum */
  if (ms && ns) {
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; i++)
      gemm_elem(a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, K, mode,
                dec, ms[i], ns[i], &y_out[i], &s_out[i]);
    return 0;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++)
      gemm_elem(a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, K, mode,
                dec, m, n, &y_out[m * N + n], &s_out[m * N + n]);
  return 0;
}

/* ------------------------------------------------------------------------------------
 * element-wise array forms of the scalar functions above (plain loops), for the tests
 * ---------------------------------------------------------------------------------- */
void ora_e4m3_decode_array(const uint8_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = ora_e4m3_decode(in[i]);
}

void ora_e4m3_encode_array(const float* in, uint8_t* out, int64_t n) {
  /* elements are independent: one thread encodes each */
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; i++) out[i] = ora_e4m3_encode(in[i]);
}

void ora_int8_encode_array(const float* in, int8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = ora_int8_encode(in[i]);
}

void ora_ue8m0_byte_array(const float* amax, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = ora_ue8m0_byte(amax[i]);
}

void ora_exp_spec_array(const float* t, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = ora_exp_spec(t[i]);
}

void ora_silu_mul_array(const float* g, const float* u, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = ora_silu_mul(g[i], u[i]);
}

// quant.hip — per-token-group FP8 (e4m3fn) quantization for gfx950.
//
// What is computed (per group of G consecutive elements of a row) follows the sglang
// PR #30924 report (prhub), sections "实现拆解" items 1-2 and "关键源码片段"
// (ref_fp8_ue8m0): amax floored at EPS, scale = amax/448 either as an fp32 value or
// rounded up to a power of two (UE8M0 byte), multiply by the reciprocal of the scale,
// clamp to +-448, round to e4m3fn. The fused variant first forms silu(gate) * up from
// the two halves of each input row (TeleFuser "tf-kernel 安装与使用", silu_and_mul
// example; the PR's fuse_silu_and_mul trait).
//
// Two variants share that rule. int8 output (the PR's ref_int8 reference) uses 127 in place
// of 448: s = amax/127 in fp32, multiplier 1/s, clamp to +-127, nearest integer with ties
// to even. Per-token quantization (TeleFuser's per-token FP8 example, scale [M, 1]) is the
// rule with one group per row (G = K), run by the whole-row kernels below (one block per row,
// or one wave per row for rows past 8192 elements).
//
// Mapping to CDNA4:
//   - one wavefront (64 lanes) streams a segment of one row; each lane owns 16
//     consecutive elements (32 bytes of bf16) of every 1024-element chunk: two adjacent
//     16-byte loads in, one 16-byte store of e4m3 codes out (the pages' "32B/lane"
//     tiling). All chunk loads of a segment are issued before any arithmetic.
//   - a group of G elements lives in G/16 adjacent lanes; its amax is a 1-3 step DPP
//     butterfly (quad_perm, row_half_mirror) inside one 8-lane half row.
//   - fp32 -> e4m3fn uses the hardware v_cvt_pk_fp8_f32 (round to nearest even), after
//     the explicit clamp to +-448, so saturation never depends on the instruction.
//   - masked (EP-MoE) dispatch: each block turns masked_m into a prefix sum in LDS and
//     the waves walk the flattened list of valid rows only, so the launch scales with
//     the number of valid rows, never with the capacity.
//   - flat problems with column-major UE8M0 scales give the 4 waves of a block 4
//     consecutive rows of one chunk, so each group's scale bytes go out as one word.
//
// Floating point: this file must be compiled without contraction (-ffp-contract=off) and
// with correctly rounded fp32 division; the arithmetic sequence is part of the contract
// (bit-exact results), see fp8q.h. Divisions whose operands stay in a checked domain use the
// shorter correctly rounded forms of quant_math.h (same results, fewer instructions).
#include "fp8q_internal.h"
#include "quant_math.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 64 * kWavesPerBlock;
constexpr int kPerLane = 16;    // consecutive elements owned by one lane per chunk (32 B of bf16)
constexpr int kChunk = 64 * kPerLane;  // elements per wave-wide chunk
constexpr int kMaxChunks = 1;   // chunks per wave item (one: see launch_group_quant)
constexpr int kTokenRegB = 2;   // chunks per wave of the one-block-per-row per-token kernel
constexpr float kFmax = 448.0f;
constexpr float kImax = 127.0f;  // int8 output: largest code used
constexpr float kEps = 0x1.b7cdfep-34f;  // 1e-10f, the amax floor

// ------------------------------------------------------------------ wave helpers
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}

// Max over the LANES (2, 4 or 8) adjacent lanes holding one group; every lane of the
// group receives the result. All 64 lanes must be active.
template <int LANES>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));                              // quad_perm [1,0,3,2]
  if constexpr (LANES >= 4) v = fmaxf(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (LANES >= 8) v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
  return v;
}

// Index of the calling wave in its block as a wave-uniform (scalar) value: the per-item row
// and address arithmetic derived from it then runs on the scalar unit, not the vector ALU.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ------------------------------------------------------------------ element loads
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Raw storage of the 16 consecutive input elements of one lane (32 or 64 bytes).
template <int DT>
struct Raw16;
template <>
struct Raw16<FP8Q_DTYPE_BF16> { u32x4 w[2]; };
template <>
struct Raw16<FP8Q_DTYPE_F16> { u32x4 w[2]; };
template <>
struct Raw16<FP8Q_DTYPE_F32> { f32x4 w[4]; };

// 16-byte loads of adjacent addresses with the default cache policy (measured ~6% faster
// than non-temporal loads on MI355X, although the input is read once).
template <int DT>
__device__ __forceinline__ void load_raw(const void* base, int64_t idx, Raw16<DT>& r) {
  if constexpr (DT == FP8Q_DTYPE_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
#pragma unroll
    for (int h = 0; h < 4; h++) r.w[h] = p[h];
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
}

template <int DT>
__device__ __forceinline__ void zero_raw(Raw16<DT>& r) {
  if constexpr (DT == FP8Q_DTYPE_F32) {
#pragma unroll
    for (int h = 0; h < 4; h++) r.w[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    r.w[0] = u32x4{0u, 0u, 0u, 0u};
    r.w[1] = r.w[0];
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

template <int DT>
__device__ __forceinline__ void widen(const Raw16<DT>& r, float (&v)[16]) {
  if constexpr (DT == FP8Q_DTYPE_F32) {
#pragma unroll
    for (int h = 0; h < 4; h++) {
      v[4 * h] = r.w[h].x; v[4 * h + 1] = r.w[h].y; v[4 * h + 2] = r.w[h].z; v[4 * h + 3] = r.w[h].w;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint32_t w = r.w[h][q];
        if constexpr (DT == FP8Q_DTYPE_BF16) {
          v[8 * h + 2 * q] = bf16_lo(w);
          v[8 * h + 2 * q + 1] = bf16_hi(w);
        } else {
          v[8 * h + 2 * q] = f16_lo(w);
          v[8 * h + 2 * q + 1] = f16_hi(w);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ silu(g) * u
// silu(g) * u = (g / (1 + exp(-g))) * u for the 16 values of a lane, each step rounded to
// fp32 (exp_fixed, then an IEEE add, a correctly rounded division and a multiply). The
// division takes the short form unless some lane of the wave holds a gate below -87, where
// 1 + exp(-g) exceeds 2^126 and its reciprocal is subnormal: that wave takes the general
// division for its 16 values. The choice is a ballot over the active lanes; both forms give
// the same correctly rounded quotient, so it never changes a result.
__device__ __forceinline__ void silu_mul16(float (&v)[16], const float (&u)[16]) {
  float d[16];
  bool low = false;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    d[j] = 1.0f + exp_fixed(-v[j]);
    low |= v[j] < -87.0f;
  }
  if (__builtin_amdgcn_ballot_w64(low) == 0) {
#pragma unroll
    for (int j = 0; j < 16; j++) v[j] = div_short(v[j], d[j]) * u[j];
  } else {
    asm volatile("");  // keeps this branch from being speculated into the common path
#pragma unroll
    for (int j = 0; j < 16; j++) v[j] = (v[j] / d[j]) * u[j];
  }
}

// ------------------------------------------------------------------ scale rules
template <int FMT, bool I8>
__device__ __forceinline__ float group_multiplier(float amax, uint32_t& scale_bits) {
  static_assert(!I8 || FMT == FP8Q_SCALE_F32, "int8 output takes fp32 scales");
  // amax >= 1e-10 (the floor), so both divisions are in their short forms' checked domains:
  // r = amax / C, then 1 / r with r in [2e-13, 3e36] or infinite
  const float r = I8 ? div_by_const<127>(amax) : div_by_const<448>(amax);
  if constexpr (FMT == FP8Q_SCALE_UE8M0) {
    const uint32_t bits = __float_as_uint(r);
    const uint32_t ex = ((bits >> 23) & 0xFFu) + ((bits & 0x7FFFFFu) != 0u ? 1u : 0u);
    scale_bits = ex;
    return __uint_as_float((254u - ex) << 23);  // 2^(127-(ex-127)), exact
  } else {
    scale_bits = __float_as_uint(r);
    return div_short(1.0f, r);
  }
}

__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -kFmax), kFmax); }

// int8: four codes (int8_code_bits: clamp to +-127, round with ties to even, code in the low
// byte), packed little-endian; v_perm_b32 gathers the low bytes (selector 0x0c: zero).
__device__ __forceinline__ uint32_t cvt4_i8(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_perm(int8_code_bits(b), int8_code_bits(a), 0x0c0c0400u);  // a, b
  const uint32_t hi = __builtin_amdgcn_perm(int8_code_bits(d), int8_code_bits(c), 0x0c0c0400u);  // c, d
  return lo | (hi << 16);
}

// 16 values times the multiplier, as 16 output codes (e4m3 after the clamp to +-448, or
// int8)
template <bool I8>
__device__ __forceinline__ u32x4 encode16(const float (&v)[16], float inv) {
  u32x4 w;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if constexpr (I8)
      w[q] = cvt4_i8(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
    else
      w[q] = cvt4(clamp448(v[4 * q] * inv), clamp448(v[4 * q + 1] * inv), clamp448(v[4 * q + 2] * inv),
                  clamp448(v[4 * q + 3] * inv));
  }
  return w;
}

// ------------------------------------------------------------------ row dispatch
// Masked dispatch: exclusive prefix sum of clamp(masked_m[e], 0, M) over experts into
// lds_pref[0..E] (lds_pref[E] = total), one block-wide scan over kThreads partials stored
// after it. Returns the number of valid rows. Every thread of the block must call it.
__device__ int64_t masked_prefix(const QuantParams& p, int32_t* lds_pref) {
  const int E = static_cast<int>(p.E);
  int32_t* part = lds_pref + E + 1;
  const int tid = threadIdx.x;
  if (E <= 64) {
    // one expert per lane of wave 0: an inclusive scan over the wave (6 shuffle steps),
    // then one barrier instead of the block-wide scan below
    if (tid < 64) {
      int32_t c = 0;
      if (tid < E) {
        c = p.masked_m[tid];
        c = c < 0 ? 0 : (c > p.M ? static_cast<int32_t>(p.M) : c);
      }
      int32_t inc = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t up = __shfl_up(inc, off, 64);
        if (tid >= off) inc += up;
      }
      if (tid < E) lds_pref[tid] = inc - c;
      if (tid == E - 1) lds_pref[E] = inc;
      if (E == 0 && tid == 0) lds_pref[0] = 0;
    }
    __syncthreads();
    return lds_pref[E];
  }
  const int per = (E + kThreads - 1) / kThreads;
  const int beg = min(tid * per, E), end = min(beg + per, E);
  int32_t local = 0;
  for (int i = beg; i < end; i++) {
    int32_t c = p.masked_m[i];
    c = c < 0 ? 0 : (c > p.M ? static_cast<int32_t>(p.M) : c);
    local += c;
  }
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int32_t add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int32_t run = part[tid] - local;  // exclusive start of this thread's slice
  for (int i = beg; i < end; i++) {
    lds_pref[i] = run;
    int32_t c = p.masked_m[i];
    c = c < 0 ? 0 : (c > p.M ? static_cast<int32_t>(p.M) : c);
    run += c;
  }
  if (tid == kThreads - 1) lds_pref[E] = part[kThreads - 1];
  __syncthreads();
  return lds_pref[E];
}

// (expert, row) of the row-th processed row: a binary search of the prefix when masked,
// else row-major over [E][M].
__device__ __forceinline__ void row_at(const QuantParams& p, const int32_t* lds_pref, bool masked, int64_t row,
                                       int64_t& e, int64_t& m) {
  if (masked) {
    int lo = 0, hi = static_cast<int>(p.E);  // lds_pref[lo] <= row < lds_pref[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (lds_pref[mid] <= row) lo = mid; else hi = mid;
    }
    e = lo;
    m = row - lds_pref[lo];
  } else {
    e = row / p.M;
    m = row - e * p.M;
  }
}

// ------------------------------------------------------------------ the group kernel
template <int DT, int G, int FMT, bool SILU, bool I8>
__global__ __launch_bounds__(kThreads) void group_quant_kernel(QuantParams p) {
  extern __shared__ int32_t lds_pref[];  // masked only: E+1 exclusive prefix + 256 partials
  constexpr int LANES = G / kPerLane;
  const int lane = threadIdx.x & 63;
  const bool masked = p.masked_m != nullptr;
  const int64_t total_rows = masked ? masked_prefix(p, lds_pref) : p.E * p.M;

  const int64_t items = total_rows * p.nseg;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_index(); t < items;
       t += nwaves) {
    const int64_t row = t / p.nseg;
    const int seg = static_cast<int>(t - row * p.nseg);
    int64_t e, m;
    row_at(p, lds_pref, masked, row, e, m);
    const int64_t xrow = e * p.x_se + m * p.x_sm;
    uint8_t* qrow = p.q + e * p.q_se + m * p.q_sm;
    const int64_t srow = e * p.s_se + m * p.s_sm;
    const int c0 = seg * p.chunks_per_seg;
    const int nc = min(p.chunks_per_seg, p.chunks_per_row - c0);  // wave-uniform

    // issue every load of the segment first
    Raw16<DT> ra[kMaxChunks];
    Raw16<DT> rb[SILU ? kMaxChunks : 1];
#pragma unroll
    for (int c = 0; c < kMaxChunks; c++) {
      zero_raw<DT>(ra[c]);
      if constexpr (SILU) zero_raw<DT>(rb[c]);
      if (c < nc) {
        const int64_t k = static_cast<int64_t>(c0 + c) * kChunk + lane * kPerLane;
        if (k < p.K) {
          load_raw<DT>(p.x, xrow + k, ra[c]);
          if constexpr (SILU) load_raw<DT>(p.x, xrow + p.K + k, rb[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kMaxChunks; c++) {
      if (c < nc) {
        const int64_t k = static_cast<int64_t>(c0 + c) * kChunk + lane * kPerLane;
        float v[16];
        widen<DT>(ra[c], v);
        if constexpr (SILU) {
          float u[16];
          widen<DT>(rb[c], u);
          silu_mul16(v, u);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; j++) amax = fmaxf(amax, fabsf(v[j]));
        amax = group_max<LANES>(amax);  // all lanes active here
        amax = fmaxf(amax, kEps);
        uint32_t sbits;
        const float inv = group_multiplier<FMT, I8>(amax, sbits);
        if (k < p.K) {
          // default cache policy: the codes stay in the Infinity Cache for the GEMM that
          // reads them next (quant + GEMM measured ~3% faster than with non-temporal stores)
          *reinterpret_cast<u32x4*>(qrow + k) = encode16<I8>(v, inv);
          if ((lane & (LANES - 1)) == 0) {
            const int64_t g = k / G;
            // packed: group g is byte g % 4 of word g / 4 (little-endian), strides in words
            const int64_t sidx = p.packed ? 4 * (srow + (g >> 2) * p.s_sg) + (g & 3) : srow + g * p.s_sg;
            if constexpr (FMT == FP8Q_SCALE_UE8M0)
              static_cast<uint8_t*>(p.s)[sidx] = static_cast<uint8_t>(sbits);
            else
              static_cast<uint32_t*>(p.s)[sidx] = sbits;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ flat, column-major UE8M0
// Same arithmetic as group_quant_kernel (one 1024-element chunk per wave), for flat problems
// whose UE8M0 scales are column-major bytes ([K/G][M], M % 4 == 0, 4-byte aligned strides):
// the 4 waves of a block take rows 4q .. 4q+3 of one chunk, so each group's 4 scale bytes are
// adjacent. The waves put them in LDS and one wave writes every group's 4 bytes as one word:
// a fourth of the scattered scale stores (each byte of a group lands in its own cache line).
template <int DT, int G, bool SILU>
__global__ __launch_bounds__(kThreads) void group_quant_rows4_kernel(QuantParams p) {
  constexpr int LANES = G / kPerLane;
  constexpr int kGroups = kChunk / G;  // groups per chunk
  __shared__ uint32_t words[2][kGroups];  // by iteration parity
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const int64_t blocks = (p.M >> 2) * p.nseg;  // (row quad, chunk) pairs
  int par = 0;
  for (int64_t bt = blockIdx.x; bt < blocks; bt += gridDim.x, par ^= 1) {
    const int64_t q4 = bt / p.nseg;
    const int seg = static_cast<int>(bt - q4 * p.nseg);
    const int64_t m = 4 * q4 + wave;
    const int64_t k = static_cast<int64_t>(seg) * kChunk + lane * kPerLane;
    Raw16<DT> ra, rb;
    zero_raw<DT>(ra);
    if constexpr (SILU) zero_raw<DT>(rb);
    if (k < p.K) {
      load_raw<DT>(p.x, m * p.x_sm + k, ra);
      if constexpr (SILU) load_raw<DT>(p.x, m * p.x_sm + p.K + k, rb);
    }
    float v[16];
    widen<DT>(ra, v);
    if constexpr (SILU) {
      float u[16];
      widen<DT>(rb, u);
      silu_mul16(v, u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; j++) amax = fmaxf(amax, fabsf(v[j]));
    amax = group_max<LANES>(amax);  // all lanes active here
    amax = fmaxf(amax, kEps);
    uint32_t sbits;
    const float inv = group_multiplier<FP8Q_SCALE_UE8M0, false>(amax, sbits);
    if (k < p.K) *reinterpret_cast<u32x4*>(p.q + m * p.q_sm + k) = encode16<false>(v, inv);
    if ((lane & (LANES - 1)) == 0)
      reinterpret_cast<uint8_t*>(words[par])[4 * (lane / LANES) + wave] = static_cast<uint8_t>(sbits);
    __syncthreads();
    // group g of rows 4q..4q+3: bytes g * s_sg + 4q .. +3; groups past K are not stored. The
    // other buffer is written next, and this one again only after the next barrier.
    if (wave == 0 && lane < kGroups) {
      const int64_t g = static_cast<int64_t>(seg) * kGroups + lane;
      if (g * G < p.K)
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p.s) + g * p.s_sg + 4 * q4) = words[par][lane];
    }
  }
}

// ------------------------------------------------------------------ the per-token kernel
// Max over all 64 lanes, returned wave-uniform: 8-lane DPP butterfly, row_mirror for 16
// lanes, then the four 16-lane rows through readlane.
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<8>(v);
  v = fmaxf(v, dpp<0x140>(v));  // row_mirror: lane i with lane 15 - i of its row
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// One wave per row, the whole row one group. The row is read in batches of kReg chunks
// (each lane: 16 elements per chunk). A row of at most kReg chunks stays in registers
// between the amax pass and the quantize pass; a longer row is read twice (the second
// read is normally served by the L2 / Infinity Cache). K % 16 == 0, so every lane's 16
// elements are either all inside the row or all outside.
template <int DT, int FMT, bool SILU, bool I8>
__global__ __launch_bounds__(kThreads) void token_quant_kernel(QuantParams p) {
  extern __shared__ int32_t lds_pref[];
  constexpr int kReg = (DT == FP8Q_DTYPE_F32 ? 4 : 8) / (SILU ? 2 : 1);
  const int lane = threadIdx.x & 63;
  const bool masked = p.masked_m != nullptr;
  const int64_t total_rows = masked ? masked_prefix(p, lds_pref) : p.E * p.M;
  const int nc = p.chunks_per_row;
  const bool resident = nc <= kReg;

  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_index(); row < total_rows;
       row += nwaves) {
    int64_t e, m;
    row_at(p, lds_pref, masked, row, e, m);
    const int64_t xrow = e * p.x_se + m * p.x_sm;
    uint8_t* qrow = p.q + e * p.q_se + m * p.q_sm;

    Raw16<DT> ra[kReg];
    Raw16<DT> rb[SILU ? kReg : 1];
    float keep[SILU ? kReg : 1][16];  // silu values of a resident row
    auto load_batch = [&](int c0) {
#pragma unroll
      for (int c = 0; c < kReg; c++) {
        zero_raw<DT>(ra[c]);
        if constexpr (SILU) zero_raw<DT>(rb[c]);
        const int64_t k = static_cast<int64_t>(c0 + c) * kChunk + lane * kPerLane;
        if (c0 + c < nc && k < p.K) {
          load_raw<DT>(p.x, xrow + k, ra[c]);
          if constexpr (SILU) load_raw<DT>(p.x, xrow + p.K + k, rb[c]);
        }
      }
    };
    auto values = [&](int c, float (&v)[16]) {
      widen<DT>(ra[c], v);
      if constexpr (SILU) {
        float u[16];
        widen<DT>(rb[c], u);
        silu_mul16(v, u);
      }
    };

    // pass 1: row amax (lanes past K hold zeros)
    float amax = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += kReg) {
      load_batch(c0);
#pragma unroll
      for (int c = 0; c < kReg; c++) {
        if (c0 + c < nc) {
          float v[16];
          values(c, v);
#pragma unroll
          for (int j = 0; j < 16; j++) amax = fmaxf(amax, fabsf(v[j]));
          if constexpr (SILU) {
#pragma unroll
            for (int j = 0; j < 16; j++) keep[c][j] = v[j];
          }
        }
      }
    }
    amax = fmaxf(wave_max(amax), kEps);
    uint32_t sbits;
    const float inv = group_multiplier<FMT, I8>(amax, sbits);
    if (lane == 0) {
      const int64_t sidx = e * p.s_se + m * p.s_sm;
      if constexpr (FMT == FP8Q_SCALE_UE8M0)
        static_cast<uint8_t*>(p.s)[sidx] = static_cast<uint8_t>(sbits);
      else
        static_cast<uint32_t*>(p.s)[sidx] = sbits;
    }

    // pass 2: quantize (a resident row reuses its registers)
    for (int c0 = 0; c0 < nc; c0 += kReg) {
      if (!resident) load_batch(c0);
#pragma unroll
      for (int c = 0; c < kReg; c++) {
        const int64_t k = static_cast<int64_t>(c0 + c) * kChunk + lane * kPerLane;
        if (c0 + c < nc && k < p.K) {
          float v[16];
          if constexpr (SILU) {
            if (resident) {
#pragma unroll
              for (int j = 0; j < 16; j++) v[j] = keep[c][j];
            } else {
              values(c, v);
            }
          } else {
            values(c, v);
          }
          *reinterpret_cast<u32x4*>(qrow + k) = encode16<I8>(v, inv);
        }
      }
    }
  }
}

// Per-token, one block per row: wave w of the block takes chunks w and w + 4 of the row (held
// in registers), the four waves' maxima meet in LDS, and every wave then quantizes its own
// chunks. A launch has four times the waves of the one-wave kernel above, so the loads of
// some rows overlap the stores of others. Rows of at most 4 * kTokenRegB chunks (8192
// elements); the one-wave kernel takes longer rows. (Sized for more chunks per wave, the
// kernel would hold their registers for every row and lose occupancy.)
template <int DT, int FMT, bool SILU, bool I8>
__global__ __launch_bounds__(kThreads) void token_quant_block_kernel(QuantParams p) {
  extern __shared__ int32_t lds_pref[];
  __shared__ float wave_amax[2][kWavesPerBlock];  // by iteration parity
  constexpr int kRegB = kTokenRegB;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const bool masked = p.masked_m != nullptr;
  const int64_t total_rows = masked ? masked_prefix(p, lds_pref) : p.E * p.M;
  const int nc = p.chunks_per_row;
  int par = 0;
  for (int64_t row = blockIdx.x; row < total_rows; row += gridDim.x, par ^= 1) {
    int64_t e, m;
    row_at(p, lds_pref, masked, row, e, m);
    const int64_t xrow = e * p.x_se + m * p.x_sm;
    uint8_t* qrow = p.q + e * p.q_se + m * p.q_sm;
    Raw16<DT> ra[kRegB];
    Raw16<DT> rb[SILU ? kRegB : 1];
#pragma unroll
    for (int i = 0; i < kRegB; i++) {
      zero_raw<DT>(ra[i]);
      if constexpr (SILU) zero_raw<DT>(rb[i]);
      const int c = wave + kWavesPerBlock * i;
      const int64_t k = static_cast<int64_t>(c) * kChunk + lane * kPerLane;
      if (c < nc && k < p.K) {
        load_raw<DT>(p.x, xrow + k, ra[i]);
        if constexpr (SILU) load_raw<DT>(p.x, xrow + p.K + k, rb[i]);
      }
    }
    // pass 1: this wave's share of the row amax (lanes past K hold zeros); silu values kept
    float keep[SILU ? kRegB : 1][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kRegB; i++) {
      if (wave + kWavesPerBlock * i < nc) {
        float v[16];
        widen<DT>(ra[i], v);
        if constexpr (SILU) {
          float u[16];
          widen<DT>(rb[i], u);
          silu_mul16(v, u);
#pragma unroll
          for (int j = 0; j < 16; j++) keep[i][j] = v[j];
        }
#pragma unroll
        for (int j = 0; j < 16; j++) amax = fmaxf(amax, fabsf(v[j]));
      }
    }
    amax = wave_max(amax);
    if (lane == 0) wave_amax[par][wave] = amax;
    __syncthreads();  // the other buffer is written next, this one again after the next barrier
    amax = fmaxf(fmaxf(wave_amax[par][0], wave_amax[par][1]), fmaxf(wave_amax[par][2], wave_amax[par][3]));
    amax = fmaxf(amax, kEps);
    uint32_t sbits;
    const float inv = group_multiplier<FMT, I8>(amax, sbits);
    if (wave == 0 && lane == 0) {
      const int64_t sidx = e * p.s_se + m * p.s_sm;
      if constexpr (FMT == FP8Q_SCALE_UE8M0)
        static_cast<uint8_t*>(p.s)[sidx] = static_cast<uint8_t>(sbits);
      else
        static_cast<uint32_t*>(p.s)[sidx] = sbits;
    }
    // pass 2: quantize this wave's chunks
#pragma unroll
    for (int i = 0; i < kRegB; i++) {
      const int c = wave + kWavesPerBlock * i;
      const int64_t k = static_cast<int64_t>(c) * kChunk + lane * kPerLane;
      if (c < nc && k < p.K) {
        float v[16];
        if constexpr (SILU) {
#pragma unroll
          for (int j = 0; j < 16; j++) v[j] = keep[i][j];
        } else {
          widen<DT>(ra[i], v);
        }
        *reinterpret_cast<u32x4*>(qrow + k) = encode16<I8>(v, inv);
      }
    }
  }
}

// Whether a per-token row goes to token_quant_block_kernel (one block per row): its chunks
// fit the four waves' registers.
constexpr bool token_rows_per_block(int chunks_per_row) { return chunks_per_row <= kWavesPerBlock * kTokenRegB; }

// Instantiated combinations: e4m3 output with fp32 or UE8M0 scales, with or without silu;
// int8 output with fp32 scales, without silu. G == 0 selects the per-token kernel.
template <int DT, int G, int FMT, bool SILU, bool I8>
void launch_one(const QuantParams& p, int grid, size_t lds, hipStream_t stream) {
  if constexpr (G == 0) {
    if (token_rows_per_block(p.chunks_per_row))  // the grid is then one block per row
      hipLaunchKernelGGL((token_quant_block_kernel<DT, FMT, SILU, I8>), dim3(grid), dim3(kThreads), lds, stream, p);
    else
      hipLaunchKernelGGL((token_quant_kernel<DT, FMT, SILU, I8>), dim3(grid), dim3(kThreads), lds, stream, p);
  }
  else
    hipLaunchKernelGGL((group_quant_kernel<DT, G, FMT, SILU, I8>), dim3(grid), dim3(kThreads), lds, stream, p);
}

template <int DT, int G>
void launch_variant(int fmt, bool silu, bool i8, const QuantParams& p, int grid, size_t lds, hipStream_t s) {
  if (i8) launch_one<DT, G, FP8Q_SCALE_F32, false, true>(p, grid, lds, s);
  else if (fmt == FP8Q_SCALE_UE8M0 && silu) launch_one<DT, G, FP8Q_SCALE_UE8M0, true, false>(p, grid, lds, s);
  else if (fmt == FP8Q_SCALE_UE8M0) launch_one<DT, G, FP8Q_SCALE_UE8M0, false, false>(p, grid, lds, s);
  else if (silu) launch_one<DT, G, FP8Q_SCALE_F32, true, false>(p, grid, lds, s);
  else launch_one<DT, G, FP8Q_SCALE_F32, false, false>(p, grid, lds, s);
}

template <int DT, int G>
void launch_rows4(bool silu, const QuantParams& p, int grid, hipStream_t s) {
  if (silu)
    hipLaunchKernelGGL((group_quant_rows4_kernel<DT, G, true>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((group_quant_rows4_kernel<DT, G, false>), dim3(grid), dim3(kThreads), 0, s, p);
}

template <int DT>
void launch_rows4_g(int g, bool silu, const QuantParams& p, int grid, hipStream_t s) {
  if (g == 32) launch_rows4<DT, 32>(silu, p, grid, s);
  else if (g == 64) launch_rows4<DT, 64>(silu, p, grid, s);
  else launch_rows4<DT, 128>(silu, p, grid, s);
}

template <int DT>
void launch_g(int g, int fmt, bool silu, bool i8, const QuantParams& p, int grid, size_t lds, hipStream_t s) {
  if (g == 32) launch_variant<DT, 32>(fmt, silu, i8, p, grid, lds, s);
  else if (g == 64) launch_variant<DT, 64>(fmt, silu, i8, p, grid, lds, s);
  else if (g == 128) launch_variant<DT, 128>(fmt, silu, i8, p, grid, lds, s);
  else launch_variant<DT, 0>(fmt, silu, i8, p, grid, lds, s);
}

}  // namespace

// Picks the segment length and the grid, then launches. Measured on MI355X: one chunk per
// wave item and one wave per item (as many waves as the problem has chunks) streams best;
// the hardware's own wave scheduling keeps HBM busier than longer per-wave segments.
// group_size 32/64/128 runs the group kernel (or, for flat column-major UE8M0 scales, the
// row-quad kernel); any other value is G = K (per-token), run with one block per row up to
// 8192 elements and one wave per row beyond.
int launch_group_quant(int in_dtype, int scale_fmt, int group_size, bool silu, bool i8, QuantParams p,
                       int64_t expected_m, hipStream_t stream) {
  const bool per_token = group_size != 32 && group_size != 64 && group_size != 128;
  const int chunks = static_cast<int>((p.K + kChunk - 1) / kChunk);
  int64_t rows_est = p.E * p.M;
  if (p.masked_m) rows_est = p.E * (expected_m > 0 ? std::min<int64_t>(expected_m, p.M) : p.M);
  if (rows_est < 1) rows_est = 1;
  p.chunks_per_seg = per_token ? chunks : 1;
  p.chunks_per_row = chunks;
  p.nseg = per_token ? 1 : chunks;
  const int64_t items = rows_est * p.nseg;
  int64_t grid = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (per_token && token_rows_per_block(chunks)) grid = rows_est;  // one block per row
  // masked launches rebuild the expert prefix sum in every block: cap the grid there so each
  // wave walks several rows instead
  grid = std::max<int64_t>(1, std::min<int64_t>(grid, p.masked_m ? 4096 : 65535));
  const size_t lds = p.masked_m ? static_cast<size_t>(p.E + 1 + kThreads) * sizeof(int32_t) : 0;
  const int g = per_token ? 0 : group_size;
  // flat problems with column-major UE8M0 bytes, rows a multiple of 4 and word-aligned scale
  // columns: the row-quad kernel, which writes each group's scales 4 rows at a time. Measured
  // on dense M=4096 x 7168: 17.8-18.6 us against 18.9-19.0 (outputs identical).
  const bool rows4 = !per_token && !p.masked_m && p.E == 1 && scale_fmt == FP8Q_SCALE_UE8M0 && !i8 && !p.packed &&
                     p.s_sm == 1 && p.M % 4 == 0 && p.s_sg % 4 == 0 && (reinterpret_cast<uintptr_t>(p.s) & 3) == 0;
  if (rows4) {
    const int64_t blocks = (p.M / 4) * p.nseg;
    const int rgrid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(blocks, 65535)));
    switch (in_dtype) {
      case FP8Q_DTYPE_BF16: launch_rows4_g<FP8Q_DTYPE_BF16>(g, silu, p, rgrid, stream); break;
      case FP8Q_DTYPE_F16: launch_rows4_g<FP8Q_DTYPE_F16>(g, silu, p, rgrid, stream); break;
      default: launch_rows4_g<FP8Q_DTYPE_F32>(g, silu, p, rgrid, stream); break;
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(FP8Q_ELAUNCH, std::string("group quant launch: ") + hipGetErrorString(err));
    return FP8Q_OK;
  }
  switch (in_dtype) {
    case FP8Q_DTYPE_BF16: launch_g<FP8Q_DTYPE_BF16>(g, scale_fmt, silu, i8, p, (int)grid, lds, stream); break;
    case FP8Q_DTYPE_F16: launch_g<FP8Q_DTYPE_F16>(g, scale_fmt, silu, i8, p, (int)grid, lds, stream); break;
    default: launch_g<FP8Q_DTYPE_F32>(g, scale_fmt, silu, i8, p, (int)grid, lds, stream); break;
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(FP8Q_ELAUNCH, std::string("group quant launch: ") + hipGetErrorString(err));
  return FP8Q_OK;
}

}  // namespace fp8q

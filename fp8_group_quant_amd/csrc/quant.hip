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
// Mapping to CDNA4:
//   - one wavefront (64 lanes) streams a segment of one row; each lane owns 8
//     consecutive elements of every 512-element chunk, so every load is a 16-byte
//     (bf16/f16) or 2x16-byte (f32) vector load and the wave reads 1 KB contiguous per
//     chunk. All chunk loads of a segment are issued before any arithmetic.
//   - a group of G elements lives in G/8 adjacent lanes; its amax is a 2-4 step DPP
//     butterfly (quad_perm, row_half_mirror, row_mirror) inside one 16-lane DPP row.
//   - fp32 -> e4m3fn uses the hardware v_cvt_pk_fp8_f32 (round to nearest even), after
//     the explicit clamp to +-448, so saturation never depends on the instruction.
//   - masked (EP-MoE) dispatch: each block turns masked_m into a prefix sum in LDS and
//     the waves walk the flattened list of valid rows only, so the launch scales with
//     the number of valid rows, never with the capacity.
//
// Floating point: this file must be compiled without contraction (-ffp-contract=off) and
// with correctly rounded fp32 division; the arithmetic sequence is part of the contract
// (bit-exact results), see fp8q.h.
#include "fp8q_internal.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 64 * kWavesPerBlock;
constexpr int kChunk = 512;     // elements per wave-wide chunk: 64 lanes x 8
constexpr int kMaxChunks = 8;   // chunks per segment (unrolled)
constexpr float kFmax = 448.0f;
constexpr float kEps = 0x1.b7cdfep-34f;  // 1e-10f, the amax floor

// ------------------------------------------------------------------ wave helpers
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}

// Max over the LANES (4, 8 or 16) adjacent lanes holding one group; every lane of the
// group receives the result. All 64 lanes must be active.
template <int LANES>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));                    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));                    // quad_perm [2,3,0,1]
  if constexpr (LANES >= 8) v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
  if constexpr (LANES >= 16) v = fmaxf(v, dpp<0x140>(v));  // row_mirror
  return v;
}

// ------------------------------------------------------------------ element loads
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Raw storage of 8 consecutive input elements of one lane.
template <int DT>
struct Raw8;
template <>
struct Raw8<FP8Q_DTYPE_BF16> { u32x4 w; };
template <>
struct Raw8<FP8Q_DTYPE_F16> { u32x4 w; };
template <>
struct Raw8<FP8Q_DTYPE_F32> { f32x4 lo, hi; };

// Inputs are streamed once: non-temporal 16-byte loads.
template <int DT>
__device__ __forceinline__ void load_raw(const void* base, int64_t idx, Raw8<DT>& r) {
  if constexpr (DT == FP8Q_DTYPE_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
    r.lo = __builtin_nontemporal_load(p);
    r.hi = __builtin_nontemporal_load(p + 1);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
    r.w = __builtin_nontemporal_load(p);
  }
}

template <int DT>
__device__ __forceinline__ void zero_raw(Raw8<DT>& r) {
  if constexpr (DT == FP8Q_DTYPE_F32) {
    r.lo = f32x4{0.f, 0.f, 0.f, 0.f};
    r.hi = r.lo;
  } else {
    r.w = u32x4{0u, 0u, 0u, 0u};
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
__device__ __forceinline__ void widen(const Raw8<DT>& r, float (&v)[8]) {
  if constexpr (DT == FP8Q_DTYPE_F32) {
    v[0] = r.lo.x; v[1] = r.lo.y; v[2] = r.lo.z; v[3] = r.lo.w;
    v[4] = r.hi.x; v[5] = r.hi.y; v[6] = r.hi.z; v[7] = r.hi.w;
  } else if constexpr (DT == FP8Q_DTYPE_BF16) {
    v[0] = bf16_lo(r.w.x); v[1] = bf16_hi(r.w.x); v[2] = bf16_lo(r.w.y); v[3] = bf16_hi(r.w.y);
    v[4] = bf16_lo(r.w.z); v[5] = bf16_hi(r.w.z); v[6] = bf16_lo(r.w.w); v[7] = bf16_hi(r.w.w);
  } else {
    v[0] = f16_lo(r.w.x); v[1] = f16_hi(r.w.x); v[2] = f16_lo(r.w.y); v[3] = f16_hi(r.w.y);
    v[4] = f16_lo(r.w.z); v[5] = f16_hi(r.w.z); v[6] = f16_lo(r.w.w); v[7] = f16_hi(r.w.w);
  }
}

// ------------------------------------------------------------------ silu(g) * u
// exp(t) as a fixed fp32 sequence: Cody-Waite reduction by ln 2 (two-part constant, fma),
// degree-7 Taylor polynomial in Horner form (fma), scaling by 2^n built from its bits.
// Constants are the fp32 values nearest to log2(e), ln 2, the remainder of ln 2, and 1/k!.
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
  const float two_n = __uint_as_float(static_cast<uint32_t>(static_cast<int>(n) + 127) << 23);
  return p * two_n;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  const float d = 1.0f + exp_fixed(-g);
  const float s = g / d;  // correctly rounded division
  return s * u;
}

// ------------------------------------------------------------------ scale rules
template <int FMT>
__device__ __forceinline__ float group_multiplier(float amax, uint32_t& scale_bits) {
  const float r = amax / kFmax;  // correctly rounded
  if constexpr (FMT == FP8Q_SCALE_UE8M0) {
    const uint32_t bits = __float_as_uint(r);
    const uint32_t ex = ((bits >> 23) & 0xFFu) + ((bits & 0x7FFFFFu) != 0u ? 1u : 0u);
    scale_bits = ex;
    return __uint_as_float((254u - ex) << 23);  // 2^(127-(ex-127)), exact
  } else {
    scale_bits = __float_as_uint(r);
    return 1.0f / r;  // correctly rounded
  }
}

__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -kFmax), kFmax); }

// ------------------------------------------------------------------ the kernel
template <int DT, int G, int FMT, bool SILU>
__global__ __launch_bounds__(kThreads) void group_quant_kernel(QuantParams p) {
  extern __shared__ int32_t lds_pref[];  // masked only: E+1 exclusive prefix + 256 partials
  constexpr int LANES = G / 8;
  const int lane = threadIdx.x & 63;
  const bool masked = p.masked_m != nullptr;

  int64_t total_rows;
  if (masked) {
    // prefix sum of clamp(masked_m[e], 0, M) over experts, one block-wide scan
    const int E = static_cast<int>(p.E);
    int32_t* part = lds_pref + E + 1;
    const int tid = threadIdx.x;
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
    total_rows = lds_pref[E];
  } else {
    total_rows = p.E * p.M;
  }

  const int64_t items = total_rows * p.nseg;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6); t < items;
       t += nwaves) {
    const int64_t row = t / p.nseg;
    const int seg = static_cast<int>(t - row * p.nseg);
    int64_t e, m;
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
    const int64_t xrow = e * p.x_se + m * p.x_sm;
    uint8_t* qrow = p.q + e * p.q_se + m * p.q_sm;
    const int64_t srow = e * p.s_se + m * p.s_sm;
    const int c0 = seg * p.chunks_per_seg;
    const int nc = min(p.chunks_per_seg, p.chunks_per_row - c0);  // wave-uniform

    // issue every load of the segment first
    Raw8<DT> ra[kMaxChunks];
    Raw8<DT> rb[SILU ? kMaxChunks : 1];
#pragma unroll
    for (int c = 0; c < kMaxChunks; c++) {
      zero_raw<DT>(ra[c]);
      if constexpr (SILU) zero_raw<DT>(rb[c]);
      if (c < nc) {
        const int64_t k = static_cast<int64_t>(c0 + c) * kChunk + lane * 8;
        if (k < p.K) {
          load_raw<DT>(p.x, xrow + k, ra[c]);
          if constexpr (SILU) load_raw<DT>(p.x, xrow + p.K + k, rb[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kMaxChunks; c++) {
      if (c < nc) {
        const int64_t k = static_cast<int64_t>(c0 + c) * kChunk + lane * 8;
        float v[8];
        widen<DT>(ra[c], v);
        if constexpr (SILU) {
          float u[8];
          widen<DT>(rb[c], u);
#pragma unroll
          for (int j = 0; j < 8; j++) v[j] = silu_mul(v[j], u[j]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) amax = fmaxf(amax, fabsf(v[j]));
        amax = group_max<LANES>(amax);  // all lanes active here
        amax = fmaxf(amax, kEps);
        uint32_t sbits;
        const float inv = group_multiplier<FMT>(amax, sbits);
        if (k < p.K) {
          const uint32_t w0 = cvt4(clamp448(v[0] * inv), clamp448(v[1] * inv),
                                   clamp448(v[2] * inv), clamp448(v[3] * inv));
          const uint32_t w1 = cvt4(clamp448(v[4] * inv), clamp448(v[5] * inv),
                                   clamp448(v[6] * inv), clamp448(v[7] * inv));
          *reinterpret_cast<uint2*>(qrow + k) = make_uint2(w0, w1);
          if ((lane & (LANES - 1)) == 0) {
            const int64_t sidx = srow + (k / G) * p.s_sg;
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

template <int DT, int G, int FMT, bool SILU>
void launch_one(const QuantParams& p, int grid, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((group_quant_kernel<DT, G, FMT, SILU>), dim3(grid), dim3(kThreads), lds, stream, p);
}

template <int DT, int G, int FMT>
void launch_silu(bool silu, const QuantParams& p, int grid, size_t lds, hipStream_t s) {
  if (silu) launch_one<DT, G, FMT, true>(p, grid, lds, s);
  else launch_one<DT, G, FMT, false>(p, grid, lds, s);
}

template <int DT, int G>
void launch_fmt(int fmt, bool silu, const QuantParams& p, int grid, size_t lds, hipStream_t s) {
  if (fmt == FP8Q_SCALE_UE8M0) launch_silu<DT, G, FP8Q_SCALE_UE8M0>(silu, p, grid, lds, s);
  else launch_silu<DT, G, FP8Q_SCALE_F32>(silu, p, grid, lds, s);
}

template <int DT>
void launch_g(int g, int fmt, bool silu, const QuantParams& p, int grid, size_t lds, hipStream_t s) {
  if (g == 32) launch_fmt<DT, 32>(fmt, silu, p, grid, lds, s);
  else if (g == 64) launch_fmt<DT, 64>(fmt, silu, p, grid, lds, s);
  else launch_fmt<DT, 128>(fmt, silu, p, grid, lds, s);
}

}  // namespace

// Picks the segment length (chunks per wave item) and the grid, then launches.
// Rows are cut into segments of U chunks (U <= 8) with no partial segment when
// possible; U shrinks when there are too few rows to give every wave slot work.
int launch_group_quant(int in_dtype, int scale_fmt, int group_size, bool silu, QuantParams p,
                       int64_t expected_m, hipStream_t stream) {
  const int chunks = static_cast<int>((p.K + kChunk - 1) / kChunk);
  int64_t rows_est = p.E * p.M;
  if (p.masked_m) rows_est = p.E * (expected_m > 0 ? std::min<int64_t>(expected_m, p.M) : p.M);
  if (rows_est < 1) rows_est = 1;
  constexpr int64_t kTargetItems = 8192;  // wave slots on 256 CUs at 32 waves each
  int U = 1;
  for (int u = kMaxChunks; u >= 1; u--) {
    if (chunks % u != 0 && u < chunks) continue;  // avoid partial segments
    if (rows_est * ((chunks + u - 1) / u) >= kTargetItems || u == 1) { U = u; break; }
  }
  if (U > chunks) U = chunks;
  p.chunks_per_seg = U;
  p.chunks_per_row = chunks;
  p.nseg = (chunks + U - 1) / U;
  const int64_t items = rows_est * p.nseg;
  int64_t grid = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  grid = std::max<int64_t>(1, std::min<int64_t>(grid, 2048));
  const size_t lds = p.masked_m ? static_cast<size_t>(p.E + 1 + kThreads) * sizeof(int32_t) : 0;
  switch (in_dtype) {
    case FP8Q_DTYPE_BF16: launch_g<FP8Q_DTYPE_BF16>(group_size, scale_fmt, silu, p, (int)grid, lds, stream); break;
    case FP8Q_DTYPE_F16: launch_g<FP8Q_DTYPE_F16>(group_size, scale_fmt, silu, p, (int)grid, lds, stream); break;
    default: launch_g<FP8Q_DTYPE_F32>(group_size, scale_fmt, silu, p, (int)grid, lds, stream); break;
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(FP8Q_ELAUNCH, std::string("group quant launch: ") + hipGetErrorString(err));
  return FP8Q_OK;
}

}  // namespace fp8q

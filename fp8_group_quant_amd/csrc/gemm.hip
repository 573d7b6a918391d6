// gemm.hip — block-scaled FP8 GEMMs for gfx950: the 1x128 x 128x128 groupwise GEMM (dense
// and masked grouped per expert) and the MXFP8 GEMM with 1x32 E8M0 scales.
//
// What is computed follows "FlashInfer GEMM 学习笔记", section 6 (block-scaled FP8 and
// MXFP8 with block size 32, plain 2D scale tensors) and section 7 (DeepGEMM's NT groupwise
// GEMM, grouped masked with expected_m + masked_m), with the activation-side scales that
// the per-token-group quantizer produces (sglang PR #30924 report, prhub, "实现拆解"):
//   BLOCK128: Y[m][n] = bf16( sum_kb sa(m,kb) * sb(n/128,kb) * sum_{k in kb} A[m][k] B[n][k] )
//   MX32:     Y[m][n] = bf16( sum_k 2^(ea(m,k/32)-127) A[m][k] * 2^(eb(n,k/32)-127) B[n][k] )
//
// Mapping to CDNA4:
//   - v_mfma_f32_16x16x128_f8f6f4 consumes exactly one 128-wide K block per instruction.
//     The operands are swapped (MFMA "A" = 16 rows of B, MFMA "B" = 16 rows of A), so the
//     16x16 result of one instruction is Y^T and each lane holds four consecutive n of one
//     m: the per-block scale factor sa(m,kb)*sb(nb,kb) is a single value per lane, and the
//     fold is one fma per accumulator per K block, in fp32 registers.
//   - MX32 uses the scaled form of the same instruction: the E8M0 bytes of each 16-row
//     slice and 32-wide K block are applied by the matrix core, and accumulation runs
//     across the whole K loop inside the MFMA with no fold.
//   - K layout inside a lane (measured on gfx950): lane l of a 16x16x128 operand holds row
//     l%16 and two 16-byte runs of K, at 16*(l/16) and 64 + 16*(l/16); the E8M0 scale for
//     (row i, 32-wide block b) comes from lane i + 16*b.
//   - tiles of 128x128 outputs, 4 wavefronts of 64x64, K step 128, double-buffered LDS with
//     a 144-byte row pitch (16 bytes of padding keep the 16-lane 16-byte fragment reads on
//     distinct banks), global loads for step k+1 in flight while step k computes.
//   - persistent workgroups; the tile list is split into 8 contiguous ranges, one per XCD
//     (workgroup w runs on XCD w % 8), so tiles that share operand rows run on the same
//     L2. Masked grouped launches build the tile list on device from masked_m, so the work
//     scales with the valid rows, never with the capacity.
#include "fp8q_internal.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;  // rows of A (m) per tile
constexpr int BN = 128;  // rows of B (n) per tile
constexpr int BK = 128;  // K per step (= one scale block)
constexpr int kThreads = 256;
constexpr int kPitch = BK + 16;  // LDS row pitch in bytes
constexpr int kXcds = 8;

struct Smem {
  alignas(16) uint8_t a[2][BM * kPitch];
  alignas(16) uint8_t b[2][BN * kPitch];
  float sa[2][BM];        // BLOCK128: activation scale per row for the step
  float sb[2];            // BLOCK128: weight scale of the tile's N block for the step
  uint32_t ea[2][BM];     // MX32: 4 E8M0 bytes (K blocks 4kb..4kb+3) per row of A
  uint32_t eb[2][BN];     // MX32: same for B
};

// value of a scale element as float: fp32, or UE8M0 byte b -> 2^(b-127)
template <int FMT>
__device__ __forceinline__ float scale_at(const void* s, int64_t idx) {
  if constexpr (FMT == FP8Q_SCALE_F32) {
    return static_cast<const float*>(s)[idx];
  } else {
    const uint32_t e = static_cast<const uint8_t*>(s)[idx];
    if (e == 0u) return __uint_as_float(0x00400000u);  // 2^-127 (subnormal)
    if (e == 255u) return __uint_as_float(0x7FC00000u);
    return __uint_as_float(e << 23);
  }
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // inputs are finite
}

// 4 E8M0 bytes (K blocks 4kb .. 4kb+3) of one row
__device__ __forceinline__ uint32_t load_e4(const uint8_t* s, int64_t row_off, int64_t sk, int kb) {
  if (sk == 1) {
    // row_off + 4kb is a multiple of 4 when the row stride is (checked by the launcher)
    return *reinterpret_cast<const uint32_t*>(s + row_off + 4 * kb);
  }
  const int64_t k0 = static_cast<int64_t>(4 * kb) * sk;
  return static_cast<uint32_t>(s[row_off + k0]) | (static_cast<uint32_t>(s[row_off + k0 + sk]) << 8) |
         (static_cast<uint32_t>(s[row_off + k0 + 2 * sk]) << 16) |
         (static_cast<uint32_t>(s[row_off + k0 + 3 * sk]) << 24);
}

struct Tile {
  int64_t e, tm, tn;
  int64_t rows;  // valid rows of A for this expert (M, or clamped masked_m[e])
};

// Global -> register staging of one K step: 4 chunks of A and 4 of B per thread, plus
// the step's scales.
template <bool MX, int SA_FMT, int SB_FMT>
struct Stage {
  u32x4 a[4], b[4];
  float sa;
  float sb;
  uint32_t ea, eb;

  __device__ __forceinline__ void load(const GemmParams& p, const uint8_t* A, const uint8_t* B,
                                       const void* SA, const void* SB, int64_t m0, int64_t n0,
                                       int64_t mrows, int64_t N, int kb, int tid) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int i = tid + kThreads * j;
      const int r = i >> 3, c = i & 7;
      const int64_t ma = min(m0 + r, mrows - 1);
      const int64_t nb = min(n0 + r, N - 1);
      a[j] = *reinterpret_cast<const u32x4*>(A + ma * p.lda + kb * BK + c * 16);
      b[j] = *reinterpret_cast<const u32x4*>(B + nb * p.ldb + kb * BK + c * 16);
    }
    if constexpr (MX) {
      if (tid < BM) {
        const int64_t ma = min(m0 + tid, mrows - 1);
        ea = load_e4(static_cast<const uint8_t*>(SA), ma * p.sa_sm, p.sa_sk, kb);
      } else {
        const int64_t nb = min(n0 + (tid - BM), N - 1);
        eb = load_e4(static_cast<const uint8_t*>(SB), nb * p.sb_sn, p.sb_sk, kb);
      }
    } else {
      if (tid < BM) {
        const int64_t ma = min(m0 + tid, mrows - 1);
        sa = scale_at<SA_FMT>(SA, ma * p.sa_sm + kb * p.sa_sk);
      } else if (tid == BM) {
        sb = scale_at<SB_FMT>(SB, (n0 / 128) * p.sb_sn + kb * p.sb_sk);
      }
    }
  }

  __device__ __forceinline__ void store(Smem& sm, int buf, int tid) const {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int i = tid + kThreads * j;
      const int r = i >> 3, c = i & 7;
      *reinterpret_cast<u32x4*>(&sm.a[buf][r * kPitch + c * 16]) = a[j];
      *reinterpret_cast<u32x4*>(&sm.b[buf][r * kPitch + c * 16]) = b[j];
    }
    if constexpr (MX) {
      if (tid < BM) sm.ea[buf][tid] = ea;
      else sm.eb[buf][tid - BM] = eb;
    } else {
      if (tid < BM) sm.sa[buf][tid] = sa;
      else if (tid == BM) sm.sb[buf] = sb;
    }
  }
};

__device__ __forceinline__ v8i frag(const uint8_t* tile, int row, int lane) {
  const uint8_t* p = tile + row * kPitch + (lane >> 4) * 16;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 64);
  v8i v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// Computes one 128x128 output tile (4 waves x 64x64) and stores it.
template <bool MX, int SA_FMT, int SB_FMT>
__device__ void run_tile(const GemmParams& p, Smem& sm, const Tile& t) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const uint8_t* A = p.a + t.e * p.a_se;
  const uint8_t* B = p.b + t.e * p.b_se;
  const void* SA = MX || SA_FMT == FP8Q_SCALE_UE8M0
                       ? static_cast<const void*>(static_cast<const uint8_t*>(p.sa) + t.e * p.sa_se)
                       : static_cast<const void*>(static_cast<const float*>(p.sa) + t.e * p.sa_se);
  const void* SB = MX || SB_FMT == FP8Q_SCALE_UE8M0
                       ? static_cast<const void*>(static_cast<const uint8_t*>(p.sb) + t.e * p.sb_se)
                       : static_cast<const void*>(static_cast<const float*>(p.sb) + t.e * p.sb_se);
  const int64_t m0 = t.tm * BM, n0 = t.tn * BN;
  const int nkb = static_cast<int>(p.K / BK);

  v4f acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int i = 0; i < 4; i++) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

  Stage<MX, SA_FMT, SB_FMT> st;
  st.load(p, A, B, SA, SB, m0, n0, t.rows, p.N, 0, tid);
  st.store(sm, 0, tid);
  __syncthreads();

  for (int kb = 0; kb < nkb; kb++) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) st.load(p, A, B, SA, SB, m0, n0, t.rows, p.N, kb + 1, tid);

    v8i fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) fb[i] = frag(sm.a[cur], wm * 64 + i * 16 + (lane & 15), lane);
#pragma unroll
    for (int j = 0; j < 4; j++) fa[j] = frag(sm.b[cur], wn * 64 + j * 16 + (lane & 15), lane);

    if constexpr (MX) {
      uint32_t sca[4], scb[4];  // this lane's E8M0 byte in bits 0..7
#pragma unroll
      for (int i = 0; i < 4; i++) sca[i] = sm.ea[cur][wm * 64 + i * 16 + (lane & 15)] >> (8 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < 4; j++) scb[j] = sm.eb[cur][wn * 64 + j * 16 + (lane & 15)] >> (8 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int i = 0; i < 4; i++)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[j], fb[i], acc[j][i], 0, 0, 0,
                                                                       static_cast<int>(scb[j]), 0,
                                                                       static_cast<int>(sca[i]));
    } else {
      const float sbv = sm.sb[cur];
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; i++) s[i] = sm.sa[cur][wm * 64 + i * 16 + (lane & 15)] * sbv;
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[j], fb[i], z, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; r++) acc[j][i][r] = fmaf(pr[r], s[i], acc[j][i][r]);
        }
    }

    if (kb + 1 < nkb) st.store(sm, cur ^ 1, tid);
    __syncthreads();
  }

  // epilogue: lane holds Y[m][n..n+3] for m = m0+wm*64+i*16+(lane&15), n = n0+wn*64+j*16+4*(lane>>4)
  uint16_t* Y = p.y + t.e * p.y_se;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t m = m0 + wm * 64 + i * 16 + (lane & 15);
    if (m >= t.rows) continue;
    uint16_t* yrow = Y + m * p.ldy;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t n = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
      const uint32_t h0 = bf16_rne(acc[j][i][0]), h1 = bf16_rne(acc[j][i][1]);
      const uint32_t h2 = bf16_rne(acc[j][i][2]), h3 = bf16_rne(acc[j][i][3]);
      if (n + 3 < p.N) {
        *reinterpret_cast<uint32_t*>(yrow + n) = h0 | (h1 << 16);
        *reinterpret_cast<uint32_t*>(yrow + n + 2) = h2 | (h3 << 16);
      } else {
        if (n < p.N) yrow[n] = static_cast<uint16_t>(h0);
        if (n + 1 < p.N) yrow[n + 1] = static_cast<uint16_t>(h1);
        if (n + 2 < p.N) yrow[n + 2] = static_cast<uint16_t>(h2);
      }
    }
  }
}

template <bool MX, int SA_FMT, int SB_FMT>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmParams p) {
  __shared__ Smem sm;
  __shared__ int32_t part[kThreads];
  extern __shared__ int32_t pref[];  // masked only, E + 1 entries: exclusive prefix of tiles
  const int tid = threadIdx.x;
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const bool masked = p.masked_m != nullptr;

  int64_t T;
  if (masked) {
    const int E = static_cast<int>(p.E);
    const int per = (E + kThreads - 1) / kThreads;
    const int beg = min(tid * per, E), end = min(beg + per, E);
    int32_t local = 0;
    for (int i = beg; i < end; i++) {
      int64_t r = p.masked_m[i];
      r = r < 0 ? 0 : (r > p.M ? p.M : r);
      local += static_cast<int32_t>(((r + BM - 1) / BM) * tiles_n);
    }
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int32_t add = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    int32_t run = part[tid] - local;
    for (int i = beg; i < end; i++) {
      pref[i] = run;
      int64_t r = p.masked_m[i];
      r = r < 0 ? 0 : (r > p.M ? p.M : r);
      run += static_cast<int32_t>(((r + BM - 1) / BM) * tiles_n);
    }
    if (tid == kThreads - 1) pref[E] = part[kThreads - 1];
    __syncthreads();
    T = pref[E];
  } else {
    T = ((p.M + BM - 1) / BM) * tiles_n;
  }

  // XCD-contiguous split of the tile list: workgroup w runs on XCD w % 8.
  const int64_t G = gridDim.x;  // a multiple of 8
  const int64_t xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, nslots = G / kXcds;
  const int64_t t_beg = (xcd * T) / kXcds, t_end = ((xcd + 1) * T) / kXcds;
  const int64_t tiles_m = (p.M + BM - 1) / BM;

  for (int64_t t = t_beg + slot; t < t_end; t += nslots) {
    Tile tile;
    if (masked) {
      int lo = 0, hi = static_cast<int>(p.E);  // pref[lo] <= t < pref[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] <= t) lo = mid; else hi = mid;
      }
      int64_t r = p.masked_m[lo];
      r = r < 0 ? 0 : (r > p.M ? p.M : r);
      const int64_t tm_e = (r + BM - 1) / BM;
      const int64_t local = t - pref[lo];
      tile.e = lo;
      tile.tm = local % tm_e;  // m tiles of one (expert, n tile) are adjacent
      tile.tn = local / tm_e;
      tile.rows = r;
    } else {
      // grouped order: 8 m tiles share each sweep over n, so B rows are reused from L2
      constexpr int64_t kGroupM = 8;
      const int64_t in_group = kGroupM * tiles_n;
      const int64_t g = t / in_group;
      const int64_t first_m = g * kGroupM;
      const int64_t gm = min(tiles_m - first_m, kGroupM);
      tile.e = 0;
      tile.tm = first_m + (t % in_group) % gm;
      tile.tn = (t % in_group) / gm;
      tile.rows = p.M;
    }
    run_tile<MX, SA_FMT, SB_FMT>(p, sm, tile);
  }
}

template <bool MX, int SA_FMT, int SB_FMT>
void launch(const GemmParams& p, int grid, hipStream_t s) {
  const size_t lds = p.masked_m ? static_cast<size_t>(p.E + 1) * sizeof(int32_t) : 0;
  hipLaunchKernelGGL((gemm_kernel<MX, SA_FMT, SB_FMT>), dim3(grid), dim3(kThreads), lds, s, p);
}

int grid_for(int64_t tiles) {
  constexpr int64_t kMaxGrid = 256 * 2;  // 2 resident workgroups per CU
  int64_t g = std::min<int64_t>(tiles, kMaxGrid);
  g = ((g + kXcds - 1) / kXcds) * kXcds;
  return static_cast<int>(std::max<int64_t>(g, kXcds));
}

int finish(const char* what) {
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(FP8Q_ELAUNCH, std::string(what) + ": " + hipGetErrorString(err));
  return FP8Q_OK;
}

}  // namespace

int launch_gemm_block128(const GemmParams& p, int64_t expected_m, hipStream_t stream) {
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  int64_t tiles;
  if (p.masked_m) {
    const int64_t rows = expected_m > 0 ? std::min<int64_t>(expected_m, p.M) : p.M;
    tiles = p.E * ((rows + BM - 1) / BM) * tiles_n;
  } else {
    tiles = ((p.M + BM - 1) / BM) * tiles_n;
  }
  const int grid = grid_for(tiles);
  const bool a8 = p.sa_fmt == FP8Q_SCALE_UE8M0, b8 = p.sb_fmt == FP8Q_SCALE_UE8M0;
  if (a8 && b8) launch<false, FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, grid, stream);
  else if (a8) launch<false, FP8Q_SCALE_UE8M0, FP8Q_SCALE_F32>(p, grid, stream);
  else if (b8) launch<false, FP8Q_SCALE_F32, FP8Q_SCALE_UE8M0>(p, grid, stream);
  else launch<false, FP8Q_SCALE_F32, FP8Q_SCALE_F32>(p, grid, stream);
  return finish("block-scaled GEMM launch");
}

int launch_gemm_mx32(const GemmParams& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  launch<true, FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, grid_for(tiles), stream);
  return finish("MXFP8 GEMM launch");
}

}  // namespace fp8q

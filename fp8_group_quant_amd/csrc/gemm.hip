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
//     m: the per-block factor sa(m,kb)*sb(nb,kb) is a single value per lane, and the fold
//     is one fma per accumulator per K block, in fp32 registers.
//   - MX32 uses the scaled form of the same instruction: the E8M0 bytes of each 16-row
//     slice and 32-wide K block are applied by the matrix core, and accumulation runs
//     across the whole K loop inside the MFMA with no fold.
//   - K layout inside a lane (measured on gfx950): lane l of a 16x16x128 operand holds row
//     l%16 and two 16-byte runs of K, at 16*(l/16) and 64 + 16*(l/16); the E8M0 scale for
//     (row i, 32-wide block b) comes from lane i + 16*b.
//   - 256x256 output tiles, 8 wavefronts of 128(m) x 64(n), K step 128. Operand tiles move
//     global -> LDS with global_load_lds_dwordx4 (no register staging), two LDS stages, the
//     loads of step k+1 in flight while step k computes, one barrier per step. LDS rows are
//     128 bytes with the 16-byte chunk index XOR-swizzled by (row/2)%8, which keeps the
//     16 rows read by one fragment load on distinct banks without padding.
//   - per-step scales are read straight from global memory into registers one step ahead.
//   - persistent workgroups (one per CU); the tile list is split into 8 contiguous ranges,
//     one per XCD (workgroup w runs on XCD w % 8), and dense tiles are ordered in groups of
//     4 m-tiles so one XCD's tiles share operand rows in its L2. Masked grouped launches
//     build the tile list on device from masked_m, so the work scales with the valid rows.
#include "fp8q_internal.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 128;   // K per step (= one BLOCK128 scale block)
constexpr int kXcds = 8;
constexpr int kCUs = 256;

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int GROUP_M_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
  static constexpr int SM = WTM / 16, SN = WTN / 16;            // 16x16 subtiles per wave
  static constexpr int kRowBlocksA = BM / 8, kRowBlocksB = BN / 8;  // 8 rows (1 KB) per wave load
  static constexpr int kLoadsA = kRowBlocksA / kWaves, kLoadsB = kRowBlocksB / kWaves;
  static_assert(kLoadsA * kWaves == kRowBlocksA && kLoadsB * kWaves == kRowBlocksB, "load split");
  static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's n range must stay inside one 128-block");
};

using Large = TileCfg<256, 256, 2, 4, 4>;

// LDS: two stages of both operand tiles and of the per-step scales. Scales are stored in
// the order the lanes read them: BLOCK128 sa as [wave row][lane%16][subtile] floats;
// MX32 E8M0 bytes as [wave row][lane%16][K block][subtile].
template <class C>
struct Smem {
  alignas(16) uint8_t a[2][C::BM * BK];
  alignas(16) uint8_t b[2][C::BN * BK];
  alignas(16) float sa[2][C::BM];
  float sb[2][C::BN / 128 > 0 ? C::BN / 128 : 1];
  alignas(16) uint8_t ea[2][C::BM * 4];
  alignas(16) uint8_t eb[2][C::BN * 4];
};

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

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

struct Tile {
  int64_t e, tm, tn;
  int64_t rows;  // valid rows of A for this expert (M, or clamped masked_m[e])
};

// Direct global -> LDS copy of one K step of a BM/BN-row operand tile. Wave w, load i
// fills row block rb = w*kLoads + i (8 rows, 1 KB): lane l writes LDS slot l of the block,
// which holds physical chunk l%8 of row rb*8 + l/8, i.e. logical chunk (l%8) ^ swz(row).
template <int kLoads>
__device__ __forceinline__ void load_stage(uint8_t* lds, const uint8_t* g, int64_t ld, int64_t r0,
                                           int64_t rmax, int kb, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kLoads; i++) {
    const int rb = wave * kLoads + i;
    const int row = rb * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    const int64_t grow = min(r0 + row, rmax);
    const uint8_t* src = g + grow * ld + kb * BK + chunk * 16;
    // (address-space conversions need C-style casts)
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(lds + rb * 1024), 16, 0, 0);
  }
}

// MFMA operand fragment of 16 rows starting at row r (lane l: row r + l%16, K runs at
// 16*(l/16) and 64 + 16*(l/16)).
__device__ __forceinline__ v8i frag(const uint8_t* tile, int r, int lane) {
  const int row = r + (lane & 15);
  const int c = lane >> 4;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + row * BK + ((c ^ swz(row)) << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + row * BK + (((c + 4) ^ swz(row)) << 4));
  v8i v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Scale staging for one K step: thread t < BM fetches the scale(s) of tile row t of A;
// thread BM + u fetches those of B (MX32: row u of the tile; BLOCK128: N block u). The
// value is held in one register from the top of a step to its end, then stored to LDS.
template <class C, bool MX, int SA_FMT, int SB_FMT>
struct ScaleStage {
  uint32_t v;

  __device__ __forceinline__ void load(const GemmParams& p, const void* SA, const void* SB, int64_t m0,
                                       int64_t n0, int64_t rmax, int kb) {
    const int tid = threadIdx.x;
    v = 0;
    if constexpr (MX) {
      const uint8_t* s8;
      int64_t off, sk;
      if (tid < C::BM) {
        s8 = static_cast<const uint8_t*>(SA);
        off = min(m0 + tid, rmax) * p.sa_sm;
        sk = p.sa_sk;
      } else if (tid < C::BM + C::BN) {
        s8 = static_cast<const uint8_t*>(SB);
        off = min(n0 + (tid - C::BM), p.N - 1) * p.sb_sn;
        sk = p.sb_sk;
      } else {
        return;
      }
      const int64_t k0 = static_cast<int64_t>(4 * kb) * sk;
      v = static_cast<uint32_t>(s8[off + k0]) | (static_cast<uint32_t>(s8[off + k0 + sk]) << 8) |
          (static_cast<uint32_t>(s8[off + k0 + 2 * sk]) << 16) | (static_cast<uint32_t>(s8[off + k0 + 3 * sk]) << 24);
    } else {
      if (tid < C::BM) {
        v = __float_as_uint(scale_at<SA_FMT>(SA, min(m0 + tid, rmax) * p.sa_sm + kb * p.sa_sk));
      } else if (tid < C::BM + C::BN / 128) {
        const int64_t nb = min(n0 / 128 + (tid - C::BM), (p.N - 1) / 128);
        v = __float_as_uint(scale_at<SB_FMT>(SB, nb * p.sb_sn + kb * p.sb_sk));
      }
    }
  }

  __device__ __forceinline__ void store(Smem<C>& sm, int st) const {
    const int tid = threadIdx.x;
    if constexpr (MX) {
      if (tid < C::BM + C::BN) {
        const bool is_a = tid < C::BM;
        const int r = is_a ? tid : tid - C::BM;
        const int wt = is_a ? C::WTM : C::WTN, nsub = wt / 16;
        const int w = r / wt, i = (r % wt) / 16, l16 = r % 16;
        uint8_t* dst = is_a ? sm.ea[st] : sm.eb[st];
#pragma unroll
        for (int b = 0; b < 4; b++) dst[((w * 16 + l16) * 4 + b) * nsub + i] = static_cast<uint8_t>(v >> (8 * b));
      }
    } else {
      if (tid < C::BM) {
        const int w = tid / C::WTM, i = (tid % C::WTM) / 16, l16 = tid % 16;
        sm.sa[st][(w * 16 + l16) * C::SM + i] = __uint_as_float(v);
      } else if (tid < C::BM + C::BN / 128) {
        sm.sb[st][tid - C::BM] = __uint_as_float(v);
      }
    }
  }
};

// Computes one BM x BN output tile and stores it.
template <class C, bool MX, int SA_FMT, int SB_FMT>
__device__ void run_tile(const GemmParams& p, Smem<C>& sm, const Tile& t) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const uint8_t* A = p.a + t.e * p.a_se;
  const uint8_t* B = p.b + t.e * p.b_se;
  const int sa_w = (MX || SA_FMT == FP8Q_SCALE_UE8M0) ? 1 : 4;
  const int sb_w = (MX || SB_FMT == FP8Q_SCALE_UE8M0) ? 1 : 4;
  const void* SA = static_cast<const uint8_t*>(p.sa) + t.e * p.sa_se * sa_w;
  const void* SB = static_cast<const uint8_t*>(p.sb) + t.e * p.sb_se * sb_w;
  const int64_t m0 = t.tm * C::BM, n0 = t.tn * C::BN;
  const int64_t rmax = t.rows - 1, nmax = p.N - 1;
  const int nkb = static_cast<int>(p.K / BK);

  v4f acc[C::SM][C::SN];
#pragma unroll
  for (int i = 0; i < C::SM; i++)
#pragma unroll
    for (int j = 0; j < C::SN; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  ScaleStage<C, MX, SA_FMT, SB_FMT> ss;
  load_stage<C::kLoadsA>(sm.a[0], A, p.lda, m0, rmax, 0, wave, lane);
  load_stage<C::kLoadsB>(sm.b[0], B, p.ldb, n0, nmax, 0, wave, lane);
  ss.load(p, SA, SB, m0, n0, rmax, 0);
  ss.store(sm, 0);

  for (int kb = 0; kb < nkb; kb++) {
    const int st = kb & 1;
    wait_vm();         // this thread's loads of stage kb have landed
    __syncthreads();   // ... everyone's; and nobody still reads stage st^1
    const bool more = kb + 1 < nkb;
    if (more) {
      load_stage<C::kLoadsA>(sm.a[st ^ 1], A, p.lda, m0, rmax, kb + 1, wave, lane);
      load_stage<C::kLoadsB>(sm.b[st ^ 1], B, p.ldb, n0, nmax, kb + 1, wave, lane);
      ss.load(p, SA, SB, m0, n0, rmax, kb + 1);
    }
    const uint8_t* ta = sm.a[st];
    const uint8_t* tb = sm.b[st];
    v8i wf[C::SN];
#pragma unroll
    for (int j = 0; j < C::SN; j++) wf[j] = frag(tb, wn * C::WTN + j * 16, lane);
    if constexpr (MX) {
      // this lane's E8M0 bytes: A rows (subtile i) and B rows (subtile j), K block 4kb + lane/16
      uint32_t ea_w[(C::SM + 3) / 4], eb_w[(C::SN + 3) / 4];
      const uint8_t* pea = sm.ea[st] + ((wm * 16 + (lane & 15)) * 4 + (lane >> 4)) * C::SM;
      const uint8_t* peb = sm.eb[st] + ((wn * 16 + (lane & 15)) * 4 + (lane >> 4)) * C::SN;
#pragma unroll
      for (int q = 0; q < (C::SM + 3) / 4; q++) ea_w[q] = reinterpret_cast<const uint32_t*>(pea)[q];
#pragma unroll
      for (int q = 0; q < (C::SN + 3) / 4; q++) eb_w[q] = reinterpret_cast<const uint32_t*>(peb)[q];
      // one m subtile at a time: its fragment is read one subtile ahead, and the scheduling
      // barrier keeps later subtiles' loads and MFMAs from being hoisted (register pressure)
      v8i xf = frag(ta, wm * C::WTM, lane);
#pragma unroll
      for (int i = 0; i < C::SM; i++) {
        const v8i xn = i + 1 < C::SM ? frag(ta, wm * C::WTM + (i + 1) * 16, lane) : xf;
        const int sa_i = static_cast<int>(ea_w[i / 4] >> (8 * (i % 4)));
#pragma unroll
        for (int j = 0; j < C::SN; j++) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[j], xf, acc[i][j], 0, 0, 0, static_cast<int>(eb_w[j / 4] >> (8 * (j % 4))), 0, sa_i);
          asm volatile("" : "+v"(acc[i][j]));  // keeps the subtile order (register pressure)
        }
        xf = xn;
      }
    } else {
      const float sbv = sm.sb[st][(wn * C::WTN) / 128];
      const float* psa = sm.sa[st] + (wm * 16 + (lane & 15)) * C::SM;
      // software-pipelined fold: the MFMAs of subtile i are issued before the fold of
      // subtile i-1, so each fold reads results that are already complete
      v8i xf = frag(ta, wm * C::WTM, lane);
      v4f prev[C::SN];
      float s_prev = 0.f;
#pragma unroll
      for (int i = 0; i < C::SM; i++) {
        const v8i xn = i + 1 < C::SM ? frag(ta, wm * C::WTM + (i + 1) * 16, lane) : xf;
        const float s = psa[i] * sbv;
        v4f pr[C::SN];
#pragma unroll
        for (int j = 0; j < C::SN; j++) {
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          pr[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf, z, 0, 0, 0, 0, 0, 0);
        }
        if (i > 0) {
#pragma unroll
          for (int j = 0; j < C::SN; j++) {
#pragma unroll
            for (int r = 0; r < 4; r++) acc[i - 1][j][r] = fmaf(prev[j][r], s_prev, acc[i - 1][j][r]);
            // keeps the folds in subtile order: otherwise they sink below every MFMA of the
            // step and all MFMA results stay live at once (register spills)
            asm volatile("" : "+v"(acc[i - 1][j]));
          }
        }
#pragma unroll
        for (int j = 0; j < C::SN; j++) prev[j] = pr[j];
        s_prev = s;
        xf = xn;
      }
#pragma unroll
      for (int j = 0; j < C::SN; j++) {
#pragma unroll
        for (int r = 0; r < 4; r++) acc[C::SM - 1][j][r] = fmaf(prev[j][r], s_prev, acc[C::SM - 1][j][r]);
        asm volatile("" : "+v"(acc[C::SM - 1][j]));
      }
    }
    if (more) ss.store(sm, st ^ 1);
  }
  __syncthreads();  // the next tile's first loads overwrite stage 0

  // epilogue: lane holds Y[m][n..n+3], m = m0+wm*WTM+i*16+lane%16, n = n0+wn*WTN+j*16+4*(lane/16)
  uint16_t* Y = p.y + t.e * p.y_se;
#pragma unroll
  for (int i = 0; i < C::SM; i++) {
    const int64_t m = m0 + wm * C::WTM + i * 16 + (lane & 15);
    if (m >= t.rows) continue;
    uint16_t* yrow = Y + m * p.ldy;
#pragma unroll
    for (int j = 0; j < C::SN; j++) {
      const int64_t n = n0 + wn * C::WTN + j * 16 + 4 * (lane >> 4);
      const uint32_t h0 = bf16_rne(acc[i][j][0]), h1 = bf16_rne(acc[i][j][1]);
      const uint32_t h2 = bf16_rne(acc[i][j][2]), h3 = bf16_rne(acc[i][j][3]);
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

template <class C, bool MX, int SA_FMT, int SB_FMT>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_kernel(GemmParams p) {
  __shared__ Smem<C> sm;
  __shared__ int32_t part[C::kThreads];
  extern __shared__ int32_t pref[];  // masked only, E + 1 entries: exclusive prefix of tiles
  const int tid = threadIdx.x;
  const int64_t tiles_n = (p.N + C::BN - 1) / C::BN;
  const bool masked = p.masked_m != nullptr;

  int64_t T;
  if (masked) {
    const int E = static_cast<int>(p.E);
    const int per = (E + C::kThreads - 1) / C::kThreads;
    const int beg = min(tid * per, E), end = min(beg + per, E);
    int32_t local = 0;
    for (int i = beg; i < end; i++) {
      int64_t r = p.masked_m[i];
      r = r < 0 ? 0 : (r > p.M ? p.M : r);
      local += static_cast<int32_t>(((r + C::BM - 1) / C::BM) * tiles_n);
    }
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < C::kThreads; off <<= 1) {
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
      run += static_cast<int32_t>(((r + C::BM - 1) / C::BM) * tiles_n);
    }
    if (tid == C::kThreads - 1) pref[E] = part[C::kThreads - 1];
    __syncthreads();
    T = pref[E];
  } else {
    T = ((p.M + C::BM - 1) / C::BM) * tiles_n;
  }

  // XCD-contiguous split of the tile list: workgroup w runs on XCD w % 8.
  const int64_t G = gridDim.x;  // a multiple of 8
  const int64_t xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, nslots = G / kXcds;
  const int64_t t_beg = (xcd * T) / kXcds, t_end = ((xcd + 1) * T) / kXcds;
  const int64_t tiles_m = (p.M + C::BM - 1) / C::BM;

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
      const int64_t tm_e = (r + C::BM - 1) / C::BM;
      const int64_t local = t - pref[lo];
      tile.e = lo;
      tile.tm = local % tm_e;  // m tiles of one (expert, n tile) are adjacent
      tile.tn = local / tm_e;
      tile.rows = r;
    } else {
      // grouped order: GROUP_M m tiles share each sweep over n, so rows are reused from L2
      const int64_t in_group = C::GROUP_M * tiles_n;
      const int64_t g = t / in_group;
      const int64_t first_m = g * C::GROUP_M;
      const int64_t gm = min(tiles_m - first_m, static_cast<int64_t>(C::GROUP_M));
      tile.e = 0;
      tile.tm = first_m + (t % in_group) % gm;
      tile.tn = (t % in_group) / gm;
      tile.rows = p.M;
    }
    run_tile<C, MX, SA_FMT, SB_FMT>(p, sm, tile);
  }
}

template <class C, bool MX, int SA_FMT, int SB_FMT>
void launch(const GemmParams& p, int grid, hipStream_t s) {
  const size_t lds = p.masked_m ? static_cast<size_t>(p.E + 1) * sizeof(int32_t) : 0;
  hipLaunchKernelGGL((gemm_kernel<C, MX, SA_FMT, SB_FMT>), dim3(grid), dim3(C::kThreads), lds, s, p);
}

int grid_for(int64_t tiles) {
  int64_t g = std::min<int64_t>(tiles, kCUs);  // one resident workgroup per CU
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
  using C = Large;
  const int64_t tiles_n = (p.N + C::BN - 1) / C::BN;
  int64_t tiles;
  if (p.masked_m) {
    const int64_t rows = expected_m > 0 ? std::min<int64_t>(expected_m, p.M) : p.M;
    tiles = p.E * ((rows + C::BM - 1) / C::BM) * tiles_n;
  } else {
    tiles = ((p.M + C::BM - 1) / C::BM) * tiles_n;
  }
  const int grid = grid_for(tiles);
  const bool a8 = p.sa_fmt == FP8Q_SCALE_UE8M0, b8 = p.sb_fmt == FP8Q_SCALE_UE8M0;
  if (a8 && b8) launch<C, false, FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, grid, stream);
  else if (a8) launch<C, false, FP8Q_SCALE_UE8M0, FP8Q_SCALE_F32>(p, grid, stream);
  else if (b8) launch<C, false, FP8Q_SCALE_F32, FP8Q_SCALE_UE8M0>(p, grid, stream);
  else launch<C, false, FP8Q_SCALE_F32, FP8Q_SCALE_F32>(p, grid, stream);
  return finish("block-scaled GEMM launch");
}

int launch_gemm_mx32(const GemmParams& p, hipStream_t stream) {
  using C = Large;
  const int64_t tiles = ((p.M + C::BM - 1) / C::BM) * ((p.N + C::BN - 1) / C::BN);
  launch<C, true, FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, grid_for(tiles), stream);
  return finish("MXFP8 GEMM launch");
}

}  // namespace fp8q

// gemm.hip — block-scaled FP8 GEMMs for gfx950: the 1x128 x 128x128 groupwise GEMM (dense,
// masked grouped per expert, and grouped over packed rows by segments or by m_indices) and
// the MXFP8 GEMM with 1x32 E8M0 scales.
//
// What is computed follows "FlashInfer GEMM 学习笔记", section 6 (block-scaled FP8 and
// MXFP8 with block size 32, plain 2D scale tensors) and section 7 (DeepGEMM's NT groupwise
// GEMM: grouped masked with expected_m + masked_m, grouped contiguous with m_indices, and
// SegmentGEMM over seg_indptr), with the activation-side scales that the per-token-group
// quantizer produces (sglang PR #30924 report, prhub, "实现拆解"):
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
//     across the whole K loop inside the MFMA with no fold. BLOCK128 with UE8M0 activation
//     scales uses it too, for the activation side only: the fold then multiplies by the
//     fp32 weight-block scale, one value per wavefront. With UE8M0 weight-block scales
//     as well, both sides go to the matrix core and BLOCK128 needs no fold either.
//   - K layout inside a lane (measured on gfx950): lane l of a 16x16x128 operand holds row
//     l%16 and two 16-byte runs of K, at 16*(l/16) and 64 + 16*(l/16); the E8M0 scale for
//     (row i, 32-wide block b) comes from lane i + 16*b.
//   - Tile shapes, all with 8 wavefronts and K steps of 128: 256x256 (wave tiles 128x64,
//     two LDS stages) for large flat problems and MXFP8; 128x256 (wave tiles 64x64, three
//     stages) for grouped launches, whose groups pad rows to 128, and for the columns that
//     fill a flat problem's last round of tiles; 256x128 otherwise. LDS rows are 128 bytes
//     with the 16-byte chunk index XOR-swizzled by (row/2)%8, which keeps the 16 rows read
//     by one fragment load on distinct banks without padding.
//   - Two ways to fill LDS. The main kernel loads operand tiles and scales straight into
//     LDS (global_load_lds), one barrier per step, loads issued one or two steps ahead and
//     the next step's first operands read during the current step's last row (see
//     "direct-to-LDS pipeline" below). Scale layouts it cannot move in aligned 4-byte
//     pieces go to a register-staged kernel: loads issued two steps ahead into one of two
//     register sets, written to one of two LDS stages. (UE8M0 row-major activation rows of
//     whole 4-byte words are read as packed words, so they stay on the main kernel.)
//   - BLOCK128 fold pipeline: each MFMA product goes to a four-slot register ring and is
//     folded three MFMAs later, so no fold waits on the MFMA it consumes and the fold's
//     VALU work co-issues with the matrix core.
//   - persistent workgroups (one per CU); the tile list is split into 8 contiguous ranges,
//     one per XCD (workgroup w runs on XCD w % 8), and dense tiles are ordered in groups of
//     4 m-tiles so one XCD's tiles share operand rows in its L2. Grouped launches build the
//     tile list on device (from masked_m or seg_indptr; m_indices per 128-row block), so
//     the work scales with the valid rows.
//   - M <= 128: a split-K kernel streams 16 rows of B per workgroup through LDS.
#include "fp8q_internal.h"

#include <utility>

#pragma clang fp contract(off)

namespace fp8q {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 128;   // K per step (= one BLOCK128 scale block)

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

using Large = TileCfg<256, 128, 4, 2, 4>;

// One LDS stage: both operand tiles of one K step and the step's scales. Scales are
// stored in the order the lanes read them: BLOCK128 sa as [wave row][lane%16][subtile]
// floats; MX32 E8M0 bytes as [wave row][lane%16][K block][subtile].
template <class C>
struct Stage {
  alignas(16) uint8_t a[C::BM * BK];
  alignas(16) uint8_t b[C::BN * BK];
  alignas(16) float sa[C::BM];
  float sb[C::BN / 128 > 0 ? C::BN / 128 : 1];
  alignas(16) uint8_t ea[C::BM * 4];
  alignas(16) uint8_t eb[C::BN * 4];
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
  int64_t e, tm, tn;  // e: expert of A, its scales and Y (masked), else 0
  int64_t rows;  // valid rows from row0 (M, clamped masked_m[e], or the segment's length)
  int64_t row0;  // first row of the segment in A, its scales and Y (else 0)
  int64_t we;    // weight (B, sb): the expert, the segment's weight, or the block's m_indices
  bool skip;     // nothing to compute (weight index outside [0, W), or a padding block)
};

// rows of group g: masked experts (clamped masked_m[g]) or segments (clamped seg_indptr)
__device__ __forceinline__ int64_t seg_begin(const GemmParams& p, int64_t g) {
  const int64_t b = p.seg_indptr[g];
  return b < 0 ? 0 : (b > p.M ? p.M : b);
}
__device__ __forceinline__ int64_t group_rows(const GemmParams& p, int64_t g) {
  if (p.masked_m) {
    const int64_t r = p.masked_m[g];
    return r < 0 ? 0 : (r > p.M ? p.M : r);
  }
  const int64_t b = seg_begin(p, g), e = p.seg_indptr[g + 1];
  return e < b ? 0 : (e > p.M ? p.M : e) - b;
}

// Global -> register staging of one K step of both operand tiles. Chunk i (16 bytes) of
// a tile is row i/8, logical chunk i%8; consecutive threads read consecutive chunks of a
// row (one 128-byte line per 8 threads). The chunk is stored to LDS at its swizzled slot.
template <class C>
struct TileRegs {
  static constexpr int kChA = C::BM * 8 / C::kThreads, kChB = C::BN * 8 / C::kThreads;
  static_assert(kChA * C::kThreads == C::BM * 8 && kChB * C::kThreads == C::BN * 8, "chunk split");
  u32x4 a[kChA], b[kChB];

  __device__ __forceinline__ void load(const uint8_t* A, int64_t lda, int64_t m0, int64_t rmax,
                                       const uint8_t* B, int64_t ldb, int64_t n0, int64_t nmax, int kb) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kChA; j++) {
      const int i = tid + C::kThreads * j, r = i >> 3, c = i & 7;
      a[j] = *reinterpret_cast<const u32x4*>(A + min(m0 + r, rmax) * lda + kb * BK + c * 16);
    }
#pragma unroll
    for (int j = 0; j < kChB; j++) {
      const int i = tid + C::kThreads * j, r = i >> 3, c = i & 7;
      b[j] = *reinterpret_cast<const u32x4*>(B + min(n0 + r, nmax) * ldb + kb * BK + c * 16);
    }
  }

  __device__ __forceinline__ void store(uint8_t* ta, uint8_t* tb) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kChA; j++) {
      const int i = tid + C::kThreads * j, r = i >> 3, c = i & 7;
      *reinterpret_cast<u32x4*>(ta + r * BK + ((c ^ swz(r)) << 4)) = a[j];
    }
#pragma unroll
    for (int j = 0; j < kChB; j++) {
      const int i = tid + C::kThreads * j, r = i >> 3, c = i & 7;
      *reinterpret_cast<u32x4*>(tb + r * BK + ((c ^ swz(r)) << 4)) = b[j];
    }
  }
};

// MFMA operand fragment of 16 rows starting at row r (lane l: row r + l%16, K runs at
// 16*(l/16) and 64 + 16*(l/16)).
// r is a multiple of 16, so swz(r + lane%16) = swz(lane%16): the lane part of the address
// is the same for every fragment of a tile and r*BK can go into the instruction's offset.
__device__ __forceinline__ v8i frag(const uint8_t* tile, int r, int lane) {
  const int l = lane & 15, c = lane >> 4;
  const uint8_t* rp = tile + r * BK;
  const int lo_off = l * BK + ((c ^ swz(l)) << 4), hi_off = l * BK + (((c + 4) ^ swz(l)) << 4);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(rp + lo_off);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(rp + hi_off);
  v8i v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// float value of a raw scale word: fp32 bits, or a UE8M0 byte b -> 2^(b-127)
template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t raw) {
  if constexpr (FMT == FP8Q_SCALE_F32) {
    return __uint_as_float(raw);
  } else {
    uint32_t bits = raw << 23;
    bits = raw == 0u ? 0x00400000u : bits;    // 2^-127 (subnormal)
    bits = raw == 255u ? 0x7FC00000u : bits;  // NaN
    return __uint_as_float(bits);
  }
}

// Element index of activation scale (m, kb) from sa: packed UE8M0 words hold K blocks
// 4j..4j+3 of a row in bytes 0..3 (strides in words), other layouts one element per (m, kb).
__device__ __forceinline__ int64_t sa_index(const GemmParams& p, int64_t m, int kb) {
  return p.sa_packed ? 4 * (m * p.sa_sm + (kb >> 2) * p.sa_sk) + (kb & 3) : m * p.sa_sm + kb * p.sa_sk;
}

// Scale staging for one K step: thread t < BM fetches the scale(s) of tile row t of A;
// thread BM + u fetches those of B (MX32: row u of the tile; BLOCK128: N block u). The
// raw word is held in one register from the top of a step to its end (no use before
// then, so the load never stalls the step), then converted and stored to LDS.
template <class C, bool MX, int SA_FMT, int SB_FMT>
struct ScaleStage {
  uint32_t v;

  __device__ __forceinline__ void load(const GemmParams& p, const void* SA, const void* SB, int64_t m0,
                                       int64_t n0, int64_t rmax, int kb) {
    const int tid = threadIdx.x;
    // (threads that fetch no scale leave v untouched: store() never reads it for them, and
    // writing it would wait for the load still landing in it)
    if constexpr (MX) {
      const uint8_t* s8;
      int64_t off, sk;
      bool packed;
      if (tid < C::BM) {
        s8 = static_cast<const uint8_t*>(SA);
        off = min(m0 + tid, rmax) * p.sa_sm;
        sk = p.sa_sk;
        packed = p.sa_packed;
      } else if (tid < C::BM + C::BN) {
        s8 = static_cast<const uint8_t*>(SB);
        off = min(n0 + (tid - C::BM), p.N - 1) * p.sb_sn;
        sk = p.sb_sk;
        packed = p.sb_packed;
      } else {
        return;
      }
      if (packed) {  // word (row, kb): the E8M0 bytes of K blocks 4kb..4kb+3, strides in words
        v = reinterpret_cast<const uint32_t*>(s8)[off + static_cast<int64_t>(kb) * sk];
        return;
      }
      const int64_t k0 = static_cast<int64_t>(4 * kb) * sk;
      if (sk == 1 && ((reinterpret_cast<uintptr_t>(s8) + off + k0) & 3) == 0) {
        v = *reinterpret_cast<const uint32_t*>(s8 + off + k0);  // the 4 bytes of K blocks 4kb..4kb+3
      } else {
        v = static_cast<uint32_t>(s8[off + k0]) | (static_cast<uint32_t>(s8[off + k0 + sk]) << 8) |
            (static_cast<uint32_t>(s8[off + k0 + 2 * sk]) << 16) |
            (static_cast<uint32_t>(s8[off + k0 + 3 * sk]) << 24);
      }
    } else {
      if (tid < C::BM) {
        const int64_t idx = sa_index(p, min(m0 + tid, rmax), kb);
        v = SA_FMT == FP8Q_SCALE_F32 ? static_cast<const uint32_t*>(SA)[idx] : static_cast<const uint8_t*>(SA)[idx];
      } else if (tid < C::BM + C::BN / 128) {
        const int64_t nb = min(n0 / 128 + (tid - C::BM), (p.N - 1) / 128);
        const int64_t idx = nb * p.sb_sn + kb * p.sb_sk;
        v = SB_FMT == FP8Q_SCALE_F32 ? static_cast<const uint32_t*>(SB)[idx] : static_cast<const uint8_t*>(SB)[idx];
      }
    }
  }

  __device__ __forceinline__ void store(Stage<C>& sg) const {
    const int tid = threadIdx.x;
    if constexpr (MX) {
      if (tid < C::BM + C::BN) {
        const bool is_a = tid < C::BM;
        const int r = is_a ? tid : tid - C::BM;
        const int wt = is_a ? C::WTM : C::WTN, nsub = wt / 16;
        const int w = r / wt, i = (r % wt) / 16, l16 = r % 16;
        uint8_t* dst = is_a ? sg.ea : sg.eb;
#pragma unroll
        for (int b = 0; b < 4; b++) dst[((w * 16 + l16) * 4 + b) * nsub + i] = static_cast<uint8_t>(v >> (8 * b));
      }
    } else {
      if (tid < C::BM) {
        const int w = tid / C::WTM, i = (tid % C::WTM) / 16, l16 = tid % 16;
        sg.sa[(w * 16 + l16) * C::SM + i] = scale_value<SA_FMT>(v);
      } else if (tid < C::BM + C::BN / 128) {
        sg.sb[tid - C::BM] = scale_value<SB_FMT>(v);
      }
    }
  }
};

// Per-tile loop state shared by the K steps.
template <class C, bool MX, int SA_FMT, int SB_FMT>
struct TileRun {
  const GemmParams& p;
  const uint8_t* A;
  const uint8_t* B;
  const void* SA;
  const void* SB;
  int64_t m0, n0, rmax, nmax;
  int nkb, wave, lane, wm, wn;
  // two register sets: set q holds the tiles and scales of a step two steps ahead
  ScaleStage<C, MX, SA_FMT, SB_FMT> ss[2];
  TileRegs<C> tr[2];
  v4f acc[C::SM][C::SN];
  // BLOCK128 fold pipeline: products of the two most recent subtile rows (row i in pr[i%2])
  // and the factor of the last row of the previous step, whose fold is still pending.
  v4f pr[2][C::SN];
  float pend_s;

  __device__ __forceinline__ void issue(int q, int kb) {
    tr[q].load(A, p.lda, m0, rmax, B, p.ldb, n0, nmax, kb);
    ss[q].load(p, SA, SB, m0, n0, rmax, kb);
  }

  __device__ __forceinline__ void commit(int q, Stage<C>& nx) {
    tr[q].store(nx.a, nx.b);
    ss[q].store(nx);
  }

  // One K step (parity Q = kb % 2): compute from stage cu = stage Q; fetch step kb + 2 into
  // register set Q; write register set 1-Q (step kb + 1, fetched one step earlier) into
  // stage nx. Q is a compile-time constant so every register set and stage is fixed.
  template <int Q>
  __device__ __forceinline__ void step(Stage<C>& cu, Stage<C>& nx, int kb) {
    // every thread's stage-kb writes are in LDS, and nobody reads stage nx any more
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(Q, min(kb + 2, nkb - 1));  // the index is clamped so every step issues the same loads

    v8i wf[C::SN];
#pragma unroll
    for (int j = 0; j < C::SN; j++) wf[j] = frag(cu.b, wn * C::WTN + j * 16, lane);
    if constexpr (MX) {
      // this lane's E8M0 bytes: A rows (subtile i) and B rows (subtile j), K block 4kb + lane/16
      uint32_t ea_w[(C::SM + 3) / 4], eb_w[(C::SN + 3) / 4];
      const uint8_t* pea = cu.ea + ((wm * 16 + (lane & 15)) * 4 + (lane >> 4)) * C::SM;
      const uint8_t* peb = cu.eb + ((wn * 16 + (lane & 15)) * 4 + (lane >> 4)) * C::SN;
#pragma unroll
      for (int q = 0; q < (C::SM + 3) / 4; q++) ea_w[q] = reinterpret_cast<const uint32_t*>(pea)[q];
#pragma unroll
      for (int q = 0; q < (C::SN + 3) / 4; q++) eb_w[q] = reinterpret_cast<const uint32_t*>(peb)[q];
      v8i xf = frag(cu.a, wm * C::WTM, lane);
#pragma unroll
      for (int i = 0; i < C::SM; i++) {
        const v8i xn = i + 1 < C::SM ? frag(cu.a, wm * C::WTM + (i + 1) * 16, lane) : xf;
        const int sa_i = static_cast<int>(ea_w[i / 4] >> (8 * (i % 4)));
#pragma unroll
        for (int j = 0; j < C::SN; j++) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[j], xf, acc[i][j], 0, 0, 0, static_cast<int>(eb_w[j / 4] >> (8 * (j % 4))), 0, sa_i);
        }
        xf = xn;
      }
    } else {
      // Row i's MFMAs are interleaved with the fold of row i-1 (for i = 0, the previous
      // step's last row), so no fold waits on the MFMA just issued.
      static_assert(C::SM % 2 == 0, "row parity must repeat across steps");
      const float sbv = cu.sb[(wn * C::WTN) / 128];
      const float* psa = cu.sa + (wm * 16 + (lane & 15)) * C::SM;
      float srow[C::SM];
#pragma unroll
      for (int i = 0; i < C::SM; i++) srow[i] = psa[i];
      v8i xf = frag(cu.a, wm * C::WTM, lane);
#pragma unroll
      for (int i = 0; i < C::SM; i++) {
        const v8i xn = i + 1 < C::SM ? frag(cu.a, wm * C::WTM + (i + 1) * 16, lane) : xf;
        const int ip = i == 0 ? C::SM - 1 : i - 1;
        const float sp = i == 0 ? pend_s : srow[i - 1] * sbv;
#pragma unroll
        for (int j = 0; j < C::SN; j++) {
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          pr[i & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf, z, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; r++) acc[ip][j][r] = fmaf(pr[(i + 1) & 1][j][r], sp, acc[ip][j][r]);
          __builtin_amdgcn_sched_barrier(0);
        }
        xf = xn;
      }
      pend_s = srow[C::SM - 1] * sbv;
    }
    if (kb + 1 < nkb) commit(1 - Q, nx);  // waits for set 1-Q only, not the loads just issued
  }
};

// Computes one BM x BN output tile and stores it.
template <class C, bool MX, int SA_FMT, int SB_FMT>
__device__ void run_tile(const GemmParams& p, Stage<C>& s0, Stage<C>& s1, const Tile& t) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // bytes per unit of the scale strides (packed UE8M0 strides count 4-byte words)
  const int sa_w = MX ? 1 : (SA_FMT == FP8Q_SCALE_UE8M0 ? (p.sa_packed ? 4 : 1) : 4);
  const int sb_w = (MX || SB_FMT == FP8Q_SCALE_UE8M0) ? 1 : 4;
  TileRun<C, MX, SA_FMT, SB_FMT> r{p};
  r.A = p.a + t.e * p.a_se + t.row0 * p.lda;
  r.B = p.b + t.we * p.b_se;
  r.SA = static_cast<const uint8_t*>(p.sa) + (t.e * p.sa_se + t.row0 * p.sa_sm) * sa_w;
  r.SB = static_cast<const uint8_t*>(p.sb) + t.we * p.sb_se * sb_w;
  r.m0 = t.tm * C::BM;
  r.n0 = t.tn * C::BN;
  r.rmax = t.rows - 1;
  r.nmax = p.N - 1;
  r.nkb = static_cast<int>(p.K / BK);
  r.wave = wave;
  r.lane = lane;
  r.wm = wave % C::WAVES_M;
  r.wn = wave / C::WAVES_M;
#pragma unroll
  for (int i = 0; i < C::SM; i++)
#pragma unroll
    for (int j = 0; j < C::SN; j++) r.acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < C::SN; j++) r.pr[1][j] = v4f{0.f, 0.f, 0.f, 0.f};
  r.pend_s = 0.f;

  r.issue(0, 0);
  r.commit(0, s0);
  r.issue(1, min(1, r.nkb - 1));
  for (int kb = 0; kb < r.nkb; kb += 2) {
    r.template step<0>(s0, s1, kb);
    if (kb + 1 < r.nkb) r.template step<1>(s1, s0, kb + 1);
  }
  if constexpr (!MX) {  // the last row's fold is still pending
#pragma unroll
    for (int j = 0; j < C::SN; j++)
#pragma unroll
      for (int q = 0; q < 4; q++)
        r.acc[C::SM - 1][j][q] = fmaf(r.pr[(C::SM - 1) & 1][j][q], r.pend_s, r.acc[C::SM - 1][j][q]);
  }
  __syncthreads();  // the next tile's first loads overwrite stage 0
  const int64_t m0 = r.m0, n0 = r.n0;
  const int wm = r.wm, wn = r.wn;
  v4f (&acc)[C::SM][C::SN] = r.acc;

  // epilogue: lane holds Y[m][n..n+3], m = m0+wm*WTM+i*16+lane%16, n = n0+wn*WTN+j*16+4*(lane/16)
  uint16_t* Y = p.y + t.e * p.y_se + t.row0 * p.ldy;
#pragma unroll
  for (int i = 0; i < C::SM; i++) {
    const int64_t m = m0 + wm * C::WTM + i * 16 + (lane & 15);
    if (m >= t.rows || (p.m_indices && p.m_indices[m] != t.we)) continue;
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

// Tile list of a launch. Dense: ceil(M/BM) x ceil(N/BN) tiles in grouped order (GROUP_M
// m tiles share each sweep over n, so operand rows are reused from L2). Masked: the
// valid tiles of each expert, found through an exclusive prefix of tile counts over the
// experts that every workgroup builds in LDS (part: kThreads ints of scratch, pref: E + 1).
template <class C>
__device__ int64_t build_tile_list(const GemmParams& p, int32_t* part, int32_t* pref) {
  const int tid = threadIdx.x;
  const int64_t tiles_n = (p.N + C::BN - 1) / C::BN;
  if (!p.masked_m && !p.seg_indptr) return ((p.M + C::BM - 1) / C::BM) * tiles_n;
  const int E = static_cast<int>(p.E);
  const int per = (E + C::kThreads - 1) / C::kThreads;
  const int beg = min(tid * per, E), end = min(beg + per, E);
  int32_t local = 0;
  for (int i = beg; i < end; i++) {
    const int64_t r = group_rows(p, i);
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
    const int64_t r = group_rows(p, i);
    run += static_cast<int32_t>(((r + C::BM - 1) / C::BM) * tiles_n);
  }
  if (tid == C::kThreads - 1) pref[E] = part[C::kThreads - 1];
  __syncthreads();
  return pref[E];
}

template <class C>
__device__ Tile tile_at(const GemmParams& p, const int32_t* pref, int64_t t) {
  const int64_t tiles_n = (p.N + C::BN - 1) / C::BN;
  Tile tile;
  tile.row0 = 0;
  tile.skip = false;
  if (p.masked_m || p.seg_indptr) {
    int lo = 0, hi = static_cast<int>(p.E);  // pref[lo] <= t < pref[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pref[mid] <= t) lo = mid; else hi = mid;
    }
    const int64_t r = group_rows(p, lo);
    const int64_t tm_e = (r + C::BM - 1) / C::BM;
    const int64_t local = t - pref[lo];
    tile.tm = local % tm_e;  // m tiles of one (group, n tile) are adjacent
    tile.tn = local / tm_e;
    tile.rows = r;
    if (p.masked_m) {
      tile.e = lo;
      tile.we = lo;
    } else {
      tile.e = 0;
      tile.row0 = seg_begin(p, lo);
      tile.we = p.seg_weight ? p.seg_weight[lo] : lo;
      tile.skip = tile.we < 0 || tile.we >= p.W;
    }
  } else {
    const int64_t tiles_m = (p.M + C::BM - 1) / C::BM;
    const int64_t in_group = C::GROUP_M * tiles_n;
    const int64_t first_m = (t / in_group) * C::GROUP_M;
    const int64_t gm = min(tiles_m - first_m, static_cast<int64_t>(C::GROUP_M));
    tile.e = 0;
    tile.tm = first_m + (t % in_group) % gm;
    tile.tn = (t % in_group) / gm;
    tile.rows = p.M;
    tile.we = 0;
    if (p.m_indices) {  // the block's weight is its first row's (blocks of BM = 128 rows)
      tile.we = p.m_indices[tile.tm * C::BM];
      tile.skip = tile.we < 0 || tile.we >= p.W;
    }
  }
  // The tile is the same for every lane; say so to the compiler, which cannot tell for values
  // read from memory, so that the addresses built from it stay in scalar registers (every
  // field is below 2^31).
  auto u = [](int64_t v) { return static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(v))); };
  tile.e = u(tile.e);
  tile.tm = u(tile.tm);
  tile.tn = u(tile.tn);
  tile.rows = u(tile.rows);
  tile.row0 = u(tile.row0);
  tile.we = u(tile.we);
  tile.skip = u(tile.skip ? 1 : 0) != 0;
  return tile;
}

// The tiles of this workgroup: an XCD-contiguous split of the tile list (tile_order.h).
__device__ __forceinline__ TileSpan my_tiles(const GemmParams& p, int64_t tiles) {
  return tile_span(tiles, blockIdx.x, gridDim.x, p.xcds);
}

template <class C, bool MX, int SA_FMT, int SB_FMT>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_kernel(GemmParams p) {
  __shared__ Stage<C> stage0;
  __shared__ Stage<C> stage1;
  __shared__ int32_t part[C::kThreads];
  extern __shared__ int32_t pref[];  // masked only, E + 1 entries
  const TileSpan tr = my_tiles(p, build_tile_list<C>(p, part, pref));
  for (int64_t t = tr.beg; t < tr.end; t += tr.stride)
  {
    const Tile tile = tile_at<C>(p, pref, t);
    if (!tile.skip) run_tile<C, MX, SA_FMT, SB_FMT>(p, stage0, stage1, tile);  // (uniform per workgroup)
  }
}

// ------------------------------------------------------------------ direct-to-LDS pipeline
// The same 256x128 tiles and 8 wavefronts of 64x64, but operand tiles and scales travel
// global -> LDS with global_load_lds (no register staging), through three LDS stages:
// while step kb computes from stage kb%3, stage (kb+1)%3 holds step kb+1 and stage
// (kb+2)%3 is being filled. The one barrier of a step sits before its last subtile row:
// by then every wavefront has read what it needs of stage kb%3 and has seen its own loads
// of step kb+1 land, so after the barrier step kb+3 is loaded into stage kb%3 and the
// first operands of step kb+1 are read into registers while the last row's MFMAs run.
// A load therefore has two steps to land.
//
// 256x256 tiles need 64 KB per step, so only two stages fit: step kb+2 is loaded into
// stage kb%2 after the barrier of step kb and has one (twice as long) step to land.
// In both, a step's loads go out in two parts (activation blocks after the barrier,
// weight blocks and scales before the next step's first two rows), not as one burst.
//
// The loads are written as inline assembly so that the compiler, which cannot tell LDS
// stages apart, does not wait for them before unrelated LDS reads; the waits are explicit
// (s_waitcnt vmcnt) and the K loop contains no other vector-memory instruction, so the
// counts are exact. M0 holds the LDS destination of each load; nothing else in these
// kernels uses M0.
//
// Scales reach LDS the same way, which limits this path to scale layouts that can be
// moved in aligned 4-byte pieces: fp32 activation scales (any strides), UE8M0 activation
// scales stored column-major ([K/128][M], M a multiple of 4) or packed four K blocks per
// word (any word strides: each step loads a row's word and reads byte kb % 4), fp32
// weight-block scales, and MX32 E8M0 bytes stored [rows][K/32] with rows a multiple of 4
// bytes apart. Other layouts use the register-staged kernel above.
//
// Scales stored per row along K (fp32 [M][K/128], E8M0 [rows][K/32]) put each row's word
// of one step in a different cache line. When K is a multiple of 512 and rows are 16-byte
// aligned, the grouped modes load four steps of a row's scales with one 16-byte load,
// once every four steps, into a two-slot ring (slot g%2 holds steps 4g..4g+3): group g+1
// is loaded after the barrier of step 4g-1, when nobody reads group g-1 any more, and is
// first read four steps later. The scale load of the other steps (and of the wavefronts
// without a scale to move) rereads group 0 into a 1 KB area nobody reads, so every step
// still issues the same loads.
// kScE8E8: UE8M0 column-major activation scales and UE8M0 weight-block scales, both applied
// by the scaled MFMA, so BLOCK128 needs no fold (accumulation runs in the matrix core)
// kScPkE8: the same with the activation scales as packed UE8M0 words
enum ScaleMode {
  kScF32Row = 0, kScE8Col = 1, kScMx = 2, kScF32Grp = 3, kScMxGrp = 4, kScE8Pk = 5, kScE8E8 = 6, kScPkE8 = 7
};

// LDS layout of the direct-to-LDS kernel for tile shape C: kStages stages, each holding
// both operand tiles of one K step and (per-step scale modes) the step's scales, followed
// by a spare word per lane. 256x128 tiles use three stages; 256x256 tiles (two weight
// blocks per tile) fit two.
template <int SCM, class C>
struct DmaLayout {
  static constexpr bool kGrouped = SCM == kScF32Grp || SCM == kScMxGrp;
  static constexpr int kStages = C::BM * BK + C::BN * BK > 48 * 1024 ? 2 : 3;
  static constexpr int kScOff = C::BM * BK + C::BN * BK;  // per-step modes: scale area inside a stage
  static constexpr int kScArea = C::BN == 256 ? 2304 : 1792;
  static constexpr int kSpare = kScArea - 256;  // the spare word of each lane
  static constexpr int kStage = kScOff + (kGrouped ? 0 : kScArea);
  static constexpr int kRing = kStages * kStage;  // grouped modes: two slots, then the dummy area
  static constexpr int kSlot = 6144;
  static constexpr int kDummy = kRing + 2 * kSlot;
  static constexpr int kBytes = kGrouped ? kDummy + 1024 : kStages * kStage;
  static constexpr int kMaxPrefix = kGrouped ? 700 : 2048;  // masked launches: at most this many experts
  static_assert(SCM != kScMxGrp || C::BN == 128, "grouped MX32 scales use 256x128 tiles");
  static_assert(kBytes + 4 * (kMaxPrefix + 1) <= 160 * 1024, "LDS");
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)p));
}

// lane l: LDS [lds + 16 l, +16) <- global [base + voff, +16). sc1 (device scope): the
// data has no reuse inside one CU, and this measured a few percent faster than the
// default policy (nt was much slower).
__device__ __forceinline__ void dma16(uint32_t lds, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc1" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}
// lane l: LDS [lds + 4 l, +4) <- global [base + voff, +4)
__device__ __forceinline__ void dma4(uint32_t lds, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2 sc1" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Tile shapes of the direct-to-LDS kernel: 256x128 outputs per workgroup as 8 wave tiles
// of 64(m) x 64(n); 256x256 as 8 wave tiles of 128(m) x 64(n); 128x256 as 8 wave tiles of
// 64x64 (masked launches: less padding in experts with few rows). (One wavefront per SIMD
// with 128x64 wave tiles in a 256x128 tile reads 25% less from LDS but measured slower:
// no second wavefront covers a stall.)
using DmaCfg = TileCfg<256, 128, 4, 2, 4>;
using DmaCfgW = TileCfg<256, 256, 2, 4, 4>;
using DmaCfgT = TileCfg<128, 256, 2, 4, 4>;
using DmaCfgW4 = TileCfg<256, 256, 2, 2, 4>;  // four waves of 128 x 128

// Per-tile state of the direct-to-LDS loop.
template <class C, int SCM>
struct DmaRun {
  using L = DmaLayout<SCM, C>;
  static constexpr int kStages = L::kStages;
  static constexpr bool MX = SCM == kScMx || SCM == kScMxGrp;
  static constexpr bool F32 = SCM == kScF32Row || SCM == kScF32Grp;
  // UE8M0 activation scales are powers of two: the matrix core applies them (E8M0 operand
  // scale of the activation rows, weights at 2^0), and the fold multiplies by the
  // weight-block scale alone, the same for every lane. P * 2^e * sb rounds exactly like
  // P * (2^e * sb), so the result is the same as folding the product of both scales.
  static constexpr bool E8 = SCM == kScE8Col || SCM == kScE8Pk;
  // UE8M0 scales on both sides: the weight-block byte (one per wave and step) goes to the
  // matrix core with the activation bytes, and the products accumulate with no fold
  static constexpr bool E8W = SCM == kScE8E8 || SCM == kScPkE8;
  static constexpr bool NOFOLD = MX || E8W;
  static constexpr int SM = C::SM, SN = C::SN;
  static_assert((C::BM == 256 || C::BM == 128) && (SN == 4 || SN == 8) && C::WTN == 16 * SN, "wave tiles");
  static constexpr int kW = C::kWaves;
  static constexpr int kLA = (C::BM / 8) / kW, kLB = (C::BN / 8) / kW;  // 1 KB blocks per wave
  static constexpr int kSc = L::kGrouped ? 1 : 8 / kW;                // scale jobs per wave
  // loads per wave and step: tile blocks, then scale jobs
  static constexpr int kGroup = kLA + kLB + kSc;
  static constexpr int kPerStep = SN * SM;  // MFMAs per wave and step

  const GemmParams& p;
  uint8_t* smem;       // three stages
  uint32_t smem_lds;   // LDS address of smem
  int nkb, lane, wave, wm, wn;
  const uint8_t* a_base;  // A + m0*lda (step kb adds kb*128)
  const uint8_t* b_base;  // B + n0*ldb
  uint32_t a_off[kLA], b_off[kLB];
  // Scale jobs: 8 per step across the workgroup (see run_tile_dma); those without a scale
  // to move load 4 bytes of A into a spare area, so every wave issues kGroup loads.
  const uint8_t* s_base[kSc];
  uint32_t s_off[kSc];
  int64_t s_step[kSc];
  int s_shift[kSc];  // the job's source advances by s_step every 2^s_shift steps
  uint32_t s_lds[kSc];
  // grouped modes: this wave's 16-byte scale load (role: ea/sa rows, eb rows or sb, or
  // none), its source for group 0, the bytes per group, its ring offset; ngroups = nkb/4
  const uint8_t* g_base;
  uint32_t g_off, g_lds;
  int g_step, ngroups;
  bool g_role;
  // operands of the current step
  v8i wf[SN];
  v8i x0, x1;
  float sa[SM], sb;
  uint32_t ea[SM], eb[SN];
  v4f acc[SM][SN];
  // BLOCK128 fold pipeline: the product of MFMA t of a step from stage S sits in
  // pr[(kSlot0 * S + t) % kRingN] and is folded kLag MFMAs later; the last kLag of a step
  // are folded at the start of the next one with that step's last-row factor pend_s. The
  // slot numbering runs on across steps (a step holds a multiple of kRingN MFMAs).
  static constexpr int kLag = 3;  // MFMAs between a product and its fold
  static constexpr int kRingN = kLag + 1;
  static_assert(kLag == 2 || kPerStep % kRingN == 0, "ring numbering must run on across steps");
  static constexpr int kSlot0 = kStages == 3 ? kPerStep : 0;
  v4f pr[kRingN];
  float pend_s;

  // The loads of step kb + kStages go out in two parts: the activation blocks right after
  // the barrier of step kb (which frees the stage) and the weight blocks and the scale load
  // before rows 0 and 1 of step kb + 1, so the texture path sees no burst of every wave's
  // loads at once (3-8% faster than one burst after the barrier). The wait before each
  // barrier is unchanged: the loads issued after those of the step it needs are exactly
  // one step's worth (none with two stages). A grouped mode's four-step scale group still
  // goes out after the barrier of the same step as before (the ring slot it fills is free
  // from there) and has landed before the step that carries it, two steps before the
  // group's first read.
  static constexpr bool kSplit = true;
  static_assert(!kSplit || SM >= 3, "the weight loads go out before rows 0 and 1");
  __device__ __forceinline__ void issue_a(int st, int kb) {
    const uint32_t base = smem_lds + st * L::kStage;
    const uint8_t* ap = a_base + kb * BK;
#pragma unroll
    for (int q = 0; q < kLA; q++) dma16(base + (wave * kLA + q) * 1024, ap, a_off[q]);
  }
  template <int PART>
  __device__ __forceinline__ void issue_b(int st, int kb) {
    const uint32_t base = smem_lds + st * L::kStage;
    const uint8_t* bp = b_base + kb * BK;
    constexpr int h = kLB / 2;
#pragma unroll
    for (int q = PART * h; q < (PART + 1) * h; q++) dma16(base + C::BM * BK + (wave * kLB + q) * 1024, bp, b_off[q]);
    if constexpr (PART == 1) issue_scales(st, kb);
  }

  __device__ __forceinline__ void issue(int st, int kb) {
    const uint32_t base = smem_lds + st * L::kStage;
    const uint8_t* ap = a_base + kb * BK;
#pragma unroll
    for (int q = 0; q < kLA; q++) dma16(base + (wave * kLA + q) * 1024, ap, a_off[q]);
    const uint8_t* bp = b_base + kb * BK;
#pragma unroll
    for (int q = 0; q < kLB; q++) dma16(base + C::BM * BK + (wave * kLB + q) * 1024, bp, b_off[q]);
    issue_scales(st, kb);
  }
  // the scale load of step kb (grouped modes: a four-step group or the dummy)
  __device__ __forceinline__ void issue_scales(int st, int kb) {
    const uint32_t base = smem_lds + st * L::kStage;
    if constexpr (L::kGrouped) {
      // tiles of step kb carry scale group (kb+2)/4 when kb%4 == 2 (groups 0 and 1 with
      // the first two steps); the group index is clamped (a reload writes equal bytes)
      const bool real = g_role && (kb <= 1 || (kb & 3) == 2);
      const int g = kb <= 1 ? kb : min((kb + 2) >> 2, ngroups - 1);
      const uint32_t dst = real ? smem_lds + L::kRing + (g & 1) * L::kSlot + g_lds : smem_lds + L::kDummy;
      dma16(dst, g_base + (real ? g * g_step : 0), g_off);
    } else {
#pragma unroll
      for (int q = 0; q < kSc; q++)
        dma4(base + L::kScOff + s_lds[q], s_base[q] + (kb >> s_shift[q]) * s_step[q], s_off[q]);
    }
  }

  __device__ __forceinline__ const uint8_t* stage(int st) const { return smem + st * L::kStage; }

  // scales of step kb (held in stage st, or in the ring)
  __device__ __forceinline__ void load_scales(int st, int kb) {
    if constexpr (L::kGrouped) {
      const uint8_t* ring = smem + L::kRing + ((kb >> 2) & 1) * L::kSlot;
      const int q = kb & 3;
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < SM; i++) ea[i] = ring[16 * (wm * C::WTM + i * 16 + (lane & 15)) + 4 * q + (lane >> 4)];
#pragma unroll
        for (int j = 0; j < SN; j++) eb[j] = ring[4096 + 16 * (wn * C::WTN + j * 16 + (lane & 15)) + 4 * q + (lane >> 4)];
      } else {
#pragma unroll
        for (int i = 0; i < SM; i++) sa[i] = reinterpret_cast<const float*>(ring)[4 * (wm * C::WTM + i * 16 + (lane & 15)) + q];
        sb = reinterpret_cast<const float*>(ring + 4096 + ((wn * C::WTN) / 128) * 1024)[q];
      }
      return;
    }
    const uint8_t* sc = stage(st) + L::kScOff;
    if constexpr (E8W) {
#pragma unroll
      for (int i = 0; i < SM; i++) {
        const int row = wm * C::WTM + i * 16 + (lane & 15);
        ea[i] = SCM == kScPkE8 ? sc[4 * row + (kb & 3)] : sc[row];  // packed: the row's word of 4 K blocks
      }
      // the weight block's word of K blocks 4(kb/4) .. +3 (the same for every lane)
      const uint32_t w = sc[1024 + ((wn * C::WTN) / 128) * 256 + (kb & 3)];
#pragma unroll
      for (int j = 0; j < SN; j++) eb[j] = w;
    } else if constexpr (MX) {
      // one lane offset for all reads (kept opaque, so each read is that register plus an
      // immediate offset rather than a hoisted address per row: with four waves of 128x128
      // the hoisted addresses did not fit the registers)
      int lo = 4 * (lane & 15) + (lane >> 4);
      asm volatile("" : "+v"(lo));
      const uint8_t* sa_l = sc + 4 * wm * C::WTM + lo;
      const uint8_t* sb_l = sc + 1024 + 4 * wn * C::WTN + lo;
#pragma unroll
      for (int i = 0; i < SM; i++) ea[i] = sa_l[64 * i];
#pragma unroll
      for (int j = 0; j < SN; j++) eb[j] = sb_l[64 * j];
    } else {
#pragma unroll
      for (int i = 0; i < SM; i++) {
        const int row = wm * C::WTM + i * 16 + (lane & 15);
        if constexpr (F32)
          sa[i] = reinterpret_cast<const float*>(sc)[row];
        else if constexpr (SCM == kScE8Pk)
          ea[i] = sc[4 * row + (kb & 3)];  // the row's word of K blocks 4(kb/4) .. +3
        else if constexpr (E8)
          ea[i] = sc[row];
        else
          sa[i] = scale_value<FP8Q_SCALE_UE8M0>(sc[row]);
      }
      // the weight-block scale of this wave's 64 columns (one word per 128-column block;
      // every lane reads the same word)
      sb = reinterpret_cast<const float*>(sc + 1024 + ((wn * C::WTN) / 128) * 256)[0];
    }
  }

  // First operands of the step held in stage st.
  __device__ __forceinline__ void load_ops(int st) {
    const uint8_t* s = stage(st);
#pragma unroll
    for (int j = 0; j < SN; j++) wf[j] = frag(s + C::BM * BK, wn * C::WTN + j * 16, lane);
    x0 = frag(s, wm * C::WTM, lane);
    if constexpr (kAhead == 2) x1 = frag(s, wm * C::WTM + 16, lane);
    load_scales(st, 0);
  }

  // MFMA t = 4i + j of the step computed from stage S, then (BLOCK128) the fold of MFMA
  // t-2 (for t < 2: the previous step's last two) with factor f[] of its row. With
  // NXT >= 0, weight fragment j of the next step is read from stage NXT right after it.
  template <int S, int NXT, int T>
  __device__ __forceinline__ void mf(const v8i& xf, const float (&f)[SM], const uint32_t (&eas)[SM],
                                     const uint32_t (&ebs)[SN]) {
    constexpr int i = T / SN, j = T % SN;
    if constexpr (NOFOLD) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf, acc[i][j], 0, 0, 0,
                                                                   static_cast<int>(ebs[j]), 0,
                                                                   static_cast<int>(eas[i]));
    } else {
      constexpr int g = kSlot0 * S + T;
      constexpr int slot = g % kRingN, pslot = (g + 1) % kRingN;
      constexpr int ip = T >= kLag ? (T - kLag) / SN : SM - 1;
      constexpr int jp = T >= kLag ? (T - kLag) % SN : SN - kLag + T;
      const float sp = T >= kLag ? f[ip] : pend_s;
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      if constexpr (E8)
        pr[slot] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf, z, 0, 0, 0, 127, 0,
                                                                    static_cast<int>(eas[i]));
      else
        pr[slot] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf, z, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; r++) acc[ip][jp][r] = fmaf(pr[pslot][r], sp, acc[ip][jp][r]);
    }
    if constexpr (NXT >= 0) wf[j] = frag(stage(NXT) + C::BM * BK, wn * C::WTN + j * 16, lane);
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int S, int NXT, int I, int... J>
  __device__ __forceinline__ void row_j(const v8i& xf, const float (&f)[SM], const uint32_t (&eas)[SM],
                                       const uint32_t (&ebs)[SN], std::integer_sequence<int, J...>) {
    (mf<S, NXT, SN * I + J>(xf, f, eas, ebs), ...);
  }
  template <int S, int NXT, int I>
  __device__ __forceinline__ void row(const v8i& xf, const float (&f)[SM], const uint32_t (&eas)[SM],
                                     const uint32_t (&ebs)[SN]) {
    row_j<S, NXT, I>(xf, f, eas, ebs, std::make_integer_sequence<int, SN>{});
  }

  // Activation fragments are read kAhead = 2 rows before their MFMAs (the first two of a
  // step during the previous step's last row).
  static constexpr int kAhead = 2;

  // rows 0..SM-2 of a step; row I first reads the activation fragment of row I+kAhead
  template <int S, int... I>
  __device__ __forceinline__ void rows(v8i (&xs)[SM], const float (&f)[SM], int kb, std::integer_sequence<int, I...>) {
    ((pre<S, I>(xs), spread<S, I>(kb), row<S, -1, I>(xs[I], f, ea, eb)), ...);
  }
  template <int S, int I>
  __device__ __forceinline__ void spread(int kb) {
    if constexpr (kSplit && I < 2) issue_b<I>((S + kStages - 1) % kStages, min(kb + kStages - 1, nkb - 1));
  }
  template <int S, int I>
  __device__ __forceinline__ void pre(v8i (&xs)[SM]) {
    if constexpr (I + kAhead < SM) xs[I + kAhead] = frag(stage(S), wm * C::WTM + (I + kAhead) * 16, lane);
  }

  // the folds still pending after the last step (which used stage S)
  template <int S>
  __device__ __forceinline__ void drain() {
#pragma unroll
    for (int q = 0; q < kLag; q++) {
      const int slot = (kSlot0 * S + kPerStep - kLag + q) % kRingN;
#pragma unroll
      for (int r = 0; r < 4; r++)
        acc[SM - 1][SN - kLag + q][r] = fmaf(pr[slot][r], pend_s, acc[SM - 1][SN - kLag + q][r]);
    }
  }

  // K step kb computed from stage S: rows 0..SM-2, the barrier, the loads of step kb+3,
  // the next step's first operands, the last row.
  template <int S>
  __device__ __forceinline__ void step(int kb) {
    constexpr int NX = (S + 1) % kStages;
    float f[SM];
    if constexpr (!NOFOLD) {
      // two stages: the previous step's last two products move to the slots of MFMAs -2 and -1
      constexpr int s0 = (kPerStep - 2) % 3, s1 = (kPerStep - 1) % 3;
      if constexpr (kLag == 2 && kStages == 2 && (s0 != 1 || s1 != 2)) {
        const v4f p0 = pr[s0], p1 = pr[s1];
        pr[1] = p0;
        pr[2] = p1;
      }
      // (E8: one value for the wave, moved to a scalar register here rather than where it
      // is read, so the last row of the previous step does not wait for that read)
      const float sbs = E8 ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sb))) : sb;
#pragma unroll
      for (int i = 0; i < SM; i++) f[i] = E8 ? sbs : sa[i] * sbs;
    }
    v8i xs[SM];
    xs[0] = x0;
    if constexpr (kAhead == 2) xs[1] = x1;
    rows<S>(xs, f, kb, std::make_integer_sequence<int, SM - 1>{});
    // Every load of step kb+1 by this wave has landed (with three stages, only step
    // kb+2's group, issued later, may still be in flight), and its reads of stage S are done.
    wait_vmcnt<(kStages - 2) * kGroup>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Past the end the step index is clamped: the stage it fills is never read again,
    // and every step keeps the same load count and no branch.
    if constexpr (kSplit)
      issue_a(S, min(kb + kStages, nkb - 1));
    else
      issue(S, min(kb + kStages, nkb - 1));
    uint32_t ea_c[SM], eb_c[SN];
    if constexpr (MX || E8 || E8W) {
#pragma unroll
      for (int i = 0; i < SM; i++) ea_c[i] = ea[i];
    }
    if constexpr (NOFOLD) {
#pragma unroll
      for (int j = 0; j < SN; j++) eb_c[j] = eb[j];
    }
    // the next step's first activation fragments and scales, into registers freed by
    // rows 0 and 1, in flight during the whole last row
    x0 = frag(stage(NX), wm * C::WTM, lane);
    if constexpr (kAhead == 2) x1 = frag(stage(NX), wm * C::WTM + 16, lane);
    load_scales(NX, kb + 1);
    __builtin_amdgcn_sched_barrier(0);
    row<S, NX, SM - 1>(xs[SM - 1], f, ea_c, eb_c);
    if constexpr (!NOFOLD) pend_s = f[SM - 1];
  }
};

template <class C, int SCM>
__device__ void run_tile_dma(const GemmParams& p, uint8_t* smem, const Tile& t) {
  using R = DmaRun<C, SCM>;
  R r{p};
  r.smem = smem;
  r.smem_lds = lds_addr(smem);
  r.lane = threadIdx.x & 63;
  r.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  r.wm = r.wave % C::WAVES_M;
  r.wn = r.wave / C::WAVES_M;
  r.nkb = static_cast<int>(p.K / BK);
  const int lane = r.lane, wave = r.wave;
  const int64_t m0 = t.tm * C::BM, n0 = t.tn * C::BN;
  const int64_t rmax = t.rows - 1, nmax = p.N - 1;
  const uint8_t* A = p.a + t.e * p.a_se + t.row0 * p.lda;
  const uint8_t* B = p.b + t.we * p.b_se;
  r.a_base = A + m0 * p.lda;
  r.b_base = B + n0 * p.ldb;
  // lane l of a 1 KB block: tile row blk*8 + l/8, LDS chunk l%8 = logical chunk ^ swz(row)
#pragma unroll
  for (int q = 0; q < R::kLA; q++) {
    const int row = (wave * R::kLA + q) * 8 + (lane >> 3), c = (lane & 7) ^ swz(row);
    r.a_off[q] = static_cast<uint32_t>((min(m0 + row, rmax) - m0) * p.lda + c * 16);
  }
#pragma unroll
  for (int q = 0; q < R::kLB; q++) {
    const int row = (wave * R::kLB + q) * 8 + (lane >> 3), c = (lane & 7) ^ swz(row);
    r.b_off[q] = static_cast<uint32_t>((min(n0 + row, nmax) - n0) * p.ldb + c * 16);
  }

  // Scale job js = q * kW + wave (8 per step). Default: 4 bytes of A into the spare area.
  constexpr int kNb = C::BN / 128;  // weight blocks per tile
#pragma unroll
  for (int q = 0; q < R::kSc; q++) {
    const int js = q * R::kW + wave;
    r.s_base[q] = r.a_base;
    r.s_off[q] = 0;
    r.s_step[q] = 0;
    r.s_shift[q] = 0;
    r.s_lds[q] = R::L::kSpare;
    if constexpr (SCM == kScE8Pk || SCM == kScPkE8) {
      if (js < 4) {  // packed word (K blocks 4(kb/4)..+3) of tile row 64 js + lane
        const uint8_t* SA = static_cast<const uint8_t*>(p.sa) + (t.e * p.sa_se + t.row0 * p.sa_sm) * 4;
        const int row = js * 64 + lane;
        r.s_base[q] = SA + m0 * p.sa_sm * 4;
        r.s_off[q] = static_cast<uint32_t>((min(m0 + row, rmax) - m0) * p.sa_sm * 4);
        r.s_step[q] = p.sa_sk * 4;
        r.s_shift[q] = 2;
        r.s_lds[q] = js * 256;
      }
    } else if constexpr (SCM == kScF32Row) {
      if (js < 4) {  // fp32 scale of tile row 64 js + lane
        const uint8_t* SA = static_cast<const uint8_t*>(p.sa) + (t.e * p.sa_se + t.row0 * p.sa_sm) * 4;
        const int row = js * 64 + lane;
        r.s_base[q] = SA + m0 * p.sa_sm * 4;
        r.s_off[q] = static_cast<uint32_t>((min(m0 + row, rmax) - m0) * p.sa_sm * 4);
        r.s_step[q] = p.sa_sk * 4;
        r.s_lds[q] = js * 256;
      }
    } else if constexpr (SCM == kScE8Col || SCM == kScE8E8) {
      if (js == 0) {  // the 4 bytes of tile rows 4*lane .. 4*lane + 3 (clamped to the last full word)
        const uint8_t* SA = static_cast<const uint8_t*>(p.sa) + t.e * p.sa_se + t.row0;  // (row0 % 4 == 0)
        r.s_base[q] = SA + m0;
        r.s_off[q] = static_cast<uint32_t>(min(m0 + 4 * lane, p.M - 4) - m0);
        r.s_step[q] = p.sa_sk;
        r.s_lds[q] = 0;
      }
    } else if constexpr (SCM == kScMx || SCM == kScMxGrp) {
      // E8M0 word (K blocks 4kb..4kb+3) of a row: bytes 4kb.. of a row-major byte row, or
      // word (row, kb) of packed scales (strides in words; with column-major words the 64
      // lanes of a job read 256 contiguous bytes instead of 64 rows' worth of lines)
      const int64_t a_row = p.sa_packed ? p.sa_sm * 4 : p.sa_sm, a_step = p.sa_packed ? p.sa_sk * 4 : 4;
      const int64_t b_row = p.sb_packed ? p.sb_sn * 4 : p.sb_sn, b_step = p.sb_packed ? p.sb_sk * 4 : 4;
      if (js < 4) {  // A row 64 js + lane
        const uint8_t* SA = static_cast<const uint8_t*>(p.sa);
        const int row = js * 64 + lane;
        r.s_base[q] = SA + m0 * a_row;
        r.s_off[q] = static_cast<uint32_t>((min(m0 + row, rmax) - m0) * a_row);
        r.s_step[q] = a_step;
        r.s_lds[q] = js * 256;
      } else if (js < 4 + C::BN / 64) {  // B row 64 (js-4) + lane
        const uint8_t* SB = static_cast<const uint8_t*>(p.sb);
        const int row = (js - 4) * 64 + lane;
        r.s_base[q] = SB + n0 * b_row;
        r.s_off[q] = static_cast<uint32_t>((min(n0 + row, nmax) - n0) * b_row);
        r.s_step[q] = b_step;
        r.s_lds[q] = 1024 + (js - 4) * 256;
      }
    }
    if constexpr (SCM == kScE8E8 || SCM == kScPkE8) {
      // UE8M0 weight block nb of the tile: the word of its K blocks 4(kb/4) .. +3, moved
      // every fourth step (every lane loads it) to [1024 + 256 nb, +256)
      const int nb = js - (SCM == kScE8E8 ? 1 : 4);
      if (nb >= 0 && nb < kNb) {
        const uint8_t* SB = static_cast<const uint8_t*>(p.sb) + t.we * p.sb_se;
        r.s_base[q] = SB + min(n0 / 128 + nb, nmax / 128) * p.sb_sn;
        r.s_off[q] = 0;
        r.s_step[q] = 4;
        r.s_shift[q] = 2;
        r.s_lds[q] = 1024 + 256 * nb;
      }
    }
    if constexpr (SCM == kScF32Row || SCM == kScE8Col || SCM == kScE8Pk) {
      // the scale of weight block nb of the tile, one fp32 word per step (every lane loads
      // it; the word lands 64 times in [1024 + 256 nb, +256) of the scale area). A block
      // past the last column reloads the last block's word.
      const int nb = js - (SCM == kScE8Col ? 1 : 4);
      if (nb >= 0 && nb < kNb) {
        const uint8_t* SB = static_cast<const uint8_t*>(p.sb) + t.we * p.sb_se * 4;
        r.s_base[q] = SB + min(n0 / 128 + nb, nmax / 128) * p.sb_sn * 4;
        r.s_off[q] = 0;
        r.s_step[q] = p.sb_sk * 4;
        r.s_lds[q] = 1024 + 256 * nb;
      }
    }
  }
  // Grouped modes: wave w's 16-byte job moves four steps of scales of 64 rows (w < 4:
  // activation rows 64w + lane; MX32 w = 4, 5: weight rows 64(w-4) + lane; BLOCK128
  // w = 4 (and 5 in 256-column tiles): the scale of weight block w-4 of the tile, every
  // lane the same 16 bytes, at 4 KB + 1 KB (w-4)). Others only load the dummy. Ring slot
  // layout: [0, 4 KB) activation rows x 16 bytes, from 4 KB the rest.
  r.g_role = false;
  r.g_base = r.a_base;
  r.g_off = 0;
  r.g_step = 16;
  r.g_lds = 0;
  r.ngroups = r.nkb / 4;
  if constexpr (SCM == kScF32Grp) {
    if (wave < 4) {
      const uint8_t* SA = static_cast<const uint8_t*>(p.sa) + (t.e * p.sa_se + t.row0 * p.sa_sm) * 4;
      const int row = wave * 64 + lane;
      r.g_role = true;
      r.g_base = SA + m0 * p.sa_sm * 4;
      r.g_off = static_cast<uint32_t>((min(m0 + row, rmax) - m0) * p.sa_sm * 4);
      r.g_lds = wave * 1024;
    } else if (wave - 4 < kNb) {  // weight block wave-4 of the tile (clamped past the last column)
      const uint8_t* SB = static_cast<const uint8_t*>(p.sb) + t.we * p.sb_se * 4;
      r.g_role = true;
      r.g_base = SB + min(n0 / 128 + (wave - 4), nmax / 128) * p.sb_sn * 4;
      r.g_lds = 4096 + (wave - 4) * 1024;
    }
  } else if constexpr (SCM == kScMxGrp) {
    if (wave < 4) {
      const uint8_t* SA = static_cast<const uint8_t*>(p.sa);
      const int row = wave * 64 + lane;
      r.g_role = true;
      r.g_base = SA + m0 * p.sa_sm;
      r.g_off = static_cast<uint32_t>((min(m0 + row, rmax) - m0) * p.sa_sm);
      r.g_lds = wave * 1024;
    } else if (wave < 6) {
      const uint8_t* SB = static_cast<const uint8_t*>(p.sb);
      const int row = (wave - 4) * 64 + lane;
      r.g_role = true;
      r.g_base = SB + n0 * p.sb_sn;
      r.g_off = static_cast<uint32_t>((min(n0 + row, nmax) - n0) * p.sb_sn);
      r.g_lds = 4096 + (wave - 4) * 1024;
    }
  }
#pragma unroll
  for (int i = 0; i < C::SM; i++)
#pragma unroll
    for (int j = 0; j < C::SN; j++) r.acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // the folds at the start of the first step add 0 * 0 (MFMAs -kLag .. -1)
#pragma unroll
  for (int q = 0; q < R::kRingN; q++) r.pr[q] = v4f{0.f, 0.f, 0.f, 0.f};
  r.pend_s = 0.f;

  const int nkb = r.nkb;
  r.issue(0, 0);
  if constexpr (R::kSplit && R::kStages == 2)
    r.issue_a(1, min(1, nkb - 1));  // the rest of step 1 goes out during step 0's first rows
  else
    r.issue(1, min(1, nkb - 1));
  if constexpr (R::kStages == 3 && R::kSplit) {
    r.issue_a(2, min(2, nkb - 1));  // the rest of step 2 goes out during step 0's first rows
    wait_vmcnt<R::kGroup + R::kLA>();  // step 0 has landed
  } else if constexpr (R::kStages == 3) {
    r.issue(2, min(2, nkb - 1));
    wait_vmcnt<2 * R::kGroup>();  // step 0 has landed; steps 1 and 2 may be in flight
  } else if constexpr (R::kSplit) {
    wait_vmcnt<R::kLA>();  // step 0 has landed; step 1's activation blocks may be in flight
  } else {
    wait_vmcnt<R::kGroup>();  // step 0 has landed; step 1 may be in flight
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  r.load_ops(0);
  if constexpr (R::kStages == 3) {
    for (int kb = 0; kb < nkb; kb += 3) {
      r.template step<0>(kb);
      if (kb + 1 < nkb) r.template step<1>(kb + 1);
      if (kb + 2 < nkb) r.template step<2>(kb + 2);
    }
  } else {
    for (int kb = 0; kb < nkb; kb += 2) {
      r.template step<0>(kb);
      if (kb + 1 < nkb) r.template step<1>(kb + 1);
    }
  }
  if constexpr (!R::NOFOLD) {  // the last step's last folds are still pending
    const int s_last = (nkb - 1) % R::kStages;
    if (s_last == 0) r.template drain<0>();
    else if (s_last == 1) r.template drain<1>();
    else r.template drain<2 % R::kStages>();
  }
  // no load is in flight and nobody reads a stage any more before the next tile's loads
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // epilogue: lane holds Y[m][n..n+3], m = m0+wm*WTM+i*16+lane%16, n = n0+wn*WTN+j*16+4*(lane/16)
  uint16_t* Y = p.y + t.e * p.y_se + t.row0 * p.ldy;
  const int wm = r.wm, wn = r.wn;
#pragma unroll
  for (int i = 0; i < C::SM; i++) {
    const int64_t m = m0 + wm * C::WTM + i * 16 + (lane & 15);
    if (m >= t.rows || (p.m_indices && p.m_indices[m] != t.we)) continue;
    uint16_t* yrow = Y + m * p.ldy;
#pragma unroll
    for (int j = 0; j < C::SN; j++) {
      const int64_t n = n0 + wn * C::WTN + j * 16 + 4 * (lane >> 4);
      const uint32_t h0 = bf16_rne(r.acc[i][j][0]), h1 = bf16_rne(r.acc[i][j][1]);
      const uint32_t h2 = bf16_rne(r.acc[i][j][2]), h3 = bf16_rne(r.acc[i][j][3]);
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

template <int SCM, class C>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_dma_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DmaLayout<SCM, C>::kBytes];
  __shared__ int32_t pref[DmaLayout<SCM, C>::kMaxPrefix + 1];  // masked only, E + 1 entries
  int32_t* part = reinterpret_cast<int32_t*>(smem);  // scan scratch, used before any load
  const TileSpan tr = my_tiles(p, build_tile_list<C>(p, part, pref));
  for (int64_t t = tr.beg; t < tr.end; t += tr.stride)
  {
    const Tile tile = tile_at<C>(p, pref, t);
    if (!tile.skip) run_tile_dma<C, SCM>(p, smem, tile);  // (uniform per workgroup)
  }
}

// ------------------------------------------------------------------ skinny GEMM (small M)
// For M <= 128 the product is bound by streaming B (the weights) from HBM and A from L2,
// and 256x128 tiles would leave most CUs idle. Each workgroup owns 16 rows of B (one MFMA
// n slice) against all M rows of A; its four waves split the K blocks four ways (block kb
// goes to wave kb % 4) and the four partial sums are added through LDS at the end.
// BLOCK128 only. Two variants: the kernel below loads MFMA fragments straight from global
// memory into registers, U blocks ahead (any scale layout); the LDS-staged one after it
// moves whole cache lines and is about twice as fast (used whenever its tables fit LDS).
constexpr int kSkinnyThreads = 256;
constexpr int64_t kSkinnyMaxM = 128;  // at most 8 m subtiles

template <int SM>
struct SkinnyCfg {
  static constexpr int U = SM == 1 ? 8 : (SM == 2 ? 6 : (SM <= 4 ? 3 : 2));  // K blocks in flight per wave
};

__device__ __forceinline__ v8i frag_global(const uint8_t* row, int kb, int lane) {
  const uint8_t* p = row + kb * BK + (lane >> 4) * 16;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 64);
  v8i v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

template <int SM, int SA_FMT, int SB_FMT>
__global__ __launch_bounds__(kSkinnyThreads) void gemm_skinny_kernel(GemmParams p) {
  constexpr int U = SkinnyCfg<SM>::U;
  __shared__ v4f red[4][SM][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int nkb = static_cast<int>(p.K / BK);
  const uint8_t* wrow = p.b + min(n0 + (lane & 15), p.N - 1) * p.ldb;
  const uint8_t* xrow[SM];
  int64_t mrow[SM];
#pragma unroll
  for (int i = 0; i < SM; i++) {
    mrow[i] = min(static_cast<int64_t>(i * 16 + (lane & 15)), p.M - 1);
    xrow[i] = p.a + mrow[i] * p.lda;
  }
  const int64_t nb = n0 / 128;
  v4f acc[SM];
#pragma unroll
  for (int i = 0; i < SM; i++) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kb0 = wave; kb0 < nkb; kb0 += 4 * U) {
    v8i wf[U], xf[U][SM];
    uint32_t sa_raw[U][SM], sb_raw[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int kb = min(kb0 + 4 * u, nkb - 1);  // clamped: blocks past the end are loaded, not used
      wf[u] = frag_global(wrow, kb, lane);
#pragma unroll
      for (int i = 0; i < SM; i++) {
        xf[u][i] = frag_global(xrow[i], kb, lane);
        const int64_t si = sa_index(p, mrow[i], kb);
        sa_raw[u][i] = SA_FMT == FP8Q_SCALE_F32 ? static_cast<const uint32_t*>(p.sa)[si]
                                                : static_cast<const uint8_t*>(p.sa)[si];
      }
      const int64_t bi = nb * p.sb_sn + kb * p.sb_sk;
      sb_raw[u] = SB_FMT == FP8Q_SCALE_F32 ? static_cast<const uint32_t*>(p.sb)[bi]
                                           : static_cast<const uint8_t*>(p.sb)[bi];
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      if (kb0 + 4 * u < nkb) {
        const float sbv = scale_value<SB_FMT>(sb_raw[u]);
#pragma unroll
        for (int i = 0; i < SM; i++) {
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[u], xf[u][i], z, 0, 0, 0, 0, 0, 0);
          const float sv = scale_value<SA_FMT>(sa_raw[u][i]) * sbv;
#pragma unroll
          for (int r = 0; r < 4; r++) acc[i][r] = fmaf(pr[r], sv, acc[i][r]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < SM; i++) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < SM; i++) {
      v4f t = red[0][i][lane];
#pragma unroll
      for (int w = 1; w < 4; w++) {
        const v4f o = red[w][i][lane];
        t[0] += o[0]; t[1] += o[1]; t[2] += o[2]; t[3] += o[3];
      }
      const int64_t m = i * 16 + (lane & 15);
      if (m >= p.M) continue;
      uint16_t* yrow = p.y + m * p.ldy;
      const int64_t n = n0 + 4 * (lane >> 4);
      const uint32_t h0 = bf16_rne(t[0]), h1 = bf16_rne(t[1]), h2 = bf16_rne(t[2]), h3 = bf16_rne(t[3]);
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

// Small M through LDS: the same split (16 rows of B per workgroup, K blocks dealt to the
// four waves in turn, partial sums added through LDS), but each wave moves its K blocks
// (all M rows of A plus the 16 rows of B, 128 bytes each) into a private ring of LDS
// stages with global_load_lds, one full cache line per 8 lanes, kStages-1 blocks ahead.
// A wave only reads its own stages, so the K loop needs no barrier: the wave's own
// vmcnt wait makes a stage readable, and its own LDS reads complete before it refills
// the stage. The activation scales of the workgroup ([K/128][MR]) and the weight-block
// scales ([K/128], as fp32) are read into LDS tables before the loop, so the loop issues no other
// vector-memory instruction and the vmcnt counts are exact. Fragment reads use the same
// XOR swizzle as the large kernels. The result equals the register-loading kernel's bit
// for bit (same per-wave block order and reduction order).
template <int SM>
struct SkinnyDmaCfg {
  static constexpr int MR = 16 * SM;                      // activation rows per block
  static constexpr int kStage = (MR + 16) * BK;           // A rows, then B rows
  static constexpr int kStages = SM >= 8 ? 2 : (SM >= 4 ? 3 : 4);
  static constexpr int kLoads = MR / 8 + 2;               // 1 KB loads per block
  static constexpr int kRing = 4 * kStages * kStage;      // all four waves
};

size_t skinny_dma_lds(int sm, int sa_fmt, int64_t nkb) {
  auto ring = [](int s) -> size_t {
    switch (s) {
      case 1: return SkinnyDmaCfg<1>::kRing;
      case 2: return SkinnyDmaCfg<2>::kRing;
      case 4: return SkinnyDmaCfg<4>::kRing;
      default: return SkinnyDmaCfg<8>::kRing;
    }
  };
  const size_t tab = static_cast<size_t>(nkb) * (16 * sm) * (sa_fmt == FP8Q_SCALE_F32 ? 4 : 1);
  return ring(sm) + ((tab + 15) & ~size_t(15)) + static_cast<size_t>(nkb) * 4;
}

template <int SM, int SA_FMT>
__global__ __launch_bounds__(kSkinnyThreads, 1) void gemm_skinny_dma_kernel(GemmParams p) {
  using D = SkinnyDmaCfg<SM>;
  constexpr int MR = D::MR, KS = D::kStages, KG = D::kLoads;
  constexpr int sab = SA_FMT == FP8Q_SCALE_F32 ? 4 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int nkb = static_cast<int>(p.K / BK);
  uint8_t* sa_tab = smem + D::kRing;  // [nkb][MR] bytes or floats
  float* sb_tab = reinterpret_cast<float*>(sa_tab + ((static_cast<size_t>(nkb) * MR * sab + 15) & ~size_t(15)));

  // this wave's loads: lane l of a 1 KB block covers row blk*8 + l/8 at LDS chunk l%8,
  // which holds logical chunk (l%8) ^ swz(row)
  const uint32_t ring = lds_addr(smem) + wave * KS * D::kStage;
  uint32_t xo[MR / 8], wo[2];
#pragma unroll
  for (int q = 0; q < MR / 8; q++) {
    const int row = q * 8 + (lane >> 3), c = (lane & 7) ^ swz(row);
    xo[q] = static_cast<uint32_t>(min(static_cast<int64_t>(row), p.M - 1) * p.lda + c * 16);
  }
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int row = q * 8 + (lane >> 3), c = (lane & 7) ^ swz(row);
    wo[q] = static_cast<uint32_t>((min(n0 + row, p.N - 1) - n0) * p.ldb + c * 16);
  }
  const uint8_t* wbase = p.b + n0 * p.ldb;
  const int nblk = (nkb - wave + 3) / 4;  // blocks kb = wave + 4 i
  // block i of this wave into stage st (past the end: block 0, so every step issues the
  // same loads and stays inside A and B; such a stage is never read)
  auto issue = [&](int st, int i) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's reads of the stage are done
    const int kb = i < nblk ? wave + 4 * i : 0;
    const uint32_t dst = ring + st * D::kStage;
#pragma unroll
    for (int q = 0; q < MR / 8; q++) dma16(dst + q * 1024, p.a + kb * BK, xo[q]);
#pragma unroll
    for (int q = 0; q < 2; q++) dma16(dst + MR * BK + q * 1024, wbase + kb * BK, wo[q]);
  };

  v4f acc[SM];
#pragma unroll
  for (int i = 0; i < SM; i++) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS - 1; s++) issue(s, s);
  // Scale tables (rows past M repeat row M-1; their outputs are never stored). All of a
  // thread's table loads are issued before any of them is waited for, after the first
  // blocks' loads, so their latency overlaps; both are complete before the K loop.
  {
    constexpr int U = 32;
    const int total = nkb * MR;
    for (int base = tid; base < total; base += kSkinnyThreads * U) {
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int idx = base + u * kSkinnyThreads;
        v[u] = 0;
        if (idx < total) {
          const int kb = idx / MR;
          const int64_t m = min(static_cast<int64_t>(idx % MR), p.M - 1);
          const int64_t si = sa_index(p, m, kb);
          v[u] = SA_FMT == FP8Q_SCALE_F32 ? static_cast<const uint32_t*>(p.sa)[si] : static_cast<const uint8_t*>(p.sa)[si];
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int idx = base + u * kSkinnyThreads;
        if (idx < total) {
          if constexpr (SA_FMT == FP8Q_SCALE_F32)
            reinterpret_cast<uint32_t*>(sa_tab)[idx] = v[u];
          else
            sa_tab[idx] = static_cast<uint8_t>(v[u]);
        }
      }
    }
    const int64_t nb = n0 / 128;
    for (int kb = tid; kb < nkb; kb += kSkinnyThreads) {
      const int64_t bi = nb * p.sb_sn + kb * p.sb_sk;
      sb_tab[kb] = p.sb_fmt == FP8Q_SCALE_F32 ? static_cast<const float*>(p.sb)[bi]
                                              : scale_value<FP8Q_SCALE_UE8M0>(static_cast<const uint8_t*>(p.sb)[bi]);
    }
  }
  __syncthreads();
  const uint8_t* ring_p = smem + wave * KS * D::kStage;
  for (int i = 0; i < nblk; i++) {
    const int st = i % KS;
    issue((i + KS - 1) % KS, i + KS - 1);
    wait_vmcnt<(KS - 1) * KG>();  // block i has landed
    const uint8_t* s = ring_p + st * D::kStage;
    const v8i wf = frag(s + MR * BK, 0, lane);
    v8i xf[SM];
#pragma unroll
    for (int j = 0; j < SM; j++) xf[j] = frag(s, j * 16, lane);
    const int kb = wave + 4 * i;
    const float sbv = sb_tab[kb];
#pragma unroll
    for (int j = 0; j < SM; j++) {
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[j], z, 0, 0, 0, 0, 0, 0);
      const int r = kb * MR + j * 16 + (lane & 15);
      const float sav = SA_FMT == FP8Q_SCALE_F32 ? reinterpret_cast<const float*>(sa_tab)[r]
                                                 : scale_value<FP8Q_SCALE_UE8M0>(sa_tab[r]);
      const float sv = sav * sbv;
#pragma unroll
      for (int q = 0; q < 4; q++) acc[j][q] = fmaf(pr[q], sv, acc[j][q]);
    }
    // (the frags are in registers before the next iteration refills this stage: the
    // MFMAs above consumed them)
  }
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with its ring; reuse it for the reduction
  v4f* red = reinterpret_cast<v4f*>(smem);  // [4 waves][SM][64]
#pragma unroll
  for (int j = 0; j < SM; j++) red[(wave * SM + j) * 64 + lane] = acc[j];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < SM; j++) {
      v4f t = red[j * 64 + lane];
#pragma unroll
      for (int w = 1; w < 4; w++) {
        const v4f o = red[(w * SM + j) * 64 + lane];
        t[0] += o[0]; t[1] += o[1]; t[2] += o[2]; t[3] += o[3];
      }
      const int64_t m = j * 16 + (lane & 15);
      if (m >= p.M) continue;
      uint16_t* yrow = p.y + m * p.ldy;
      const int64_t n = n0 + 4 * (lane >> 4);
      const uint32_t h0 = bf16_rne(t[0]), h1 = bf16_rne(t[1]), h2 = bf16_rne(t[2]), h3 = bf16_rne(t[3]);
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

// Small M through registers: each workgroup owns 16 rows of B (one MFMA n slice) against all
// M rows of A, like the kernels above, but its waves take contiguous ranges of the K blocks
// and load their fragments of A and B (and the scales) straight from global memory into
// registers, a pass of P blocks at a time, the next pass issued before the current one is
// computed. With K = 7168 a wave's whole range is in flight from the start for M <= 16, so
// the launch pays about one memory latency instead of one per block. The operand fragments
// are buffer loads: a lane's row and chunk are a fixed 32-bit offset, the block a scalar
// offset, so a load costs no address arithmetic; rows past N or M read as zeros (the
// buffer's bounds) and are never stored. The partial sums of the waves are added through
// LDS in wave order (fixed, so results are reproducible), each wave finishing one 16-row
// slice of the output.
template <int SM>
struct SmallCfg {
  // Eight waves (two per SIMD, 256 VGPRs each). Blocks per pass: two passes of fragments
  // (B 8 VGPRs, A 8 per 16 rows, scales) fit the registers.
  static_assert(SM == 1, "M <= 16");
  static constexpr int kWaves = 8;
  static constexpr int P = 4;
};

constexpr int kBufWord3 = 0x00020000;  // raw buffer resource: 32-bit data format, no swizzle

__device__ __forceinline__ v8i frag_buffer(__amdgpu_buffer_rsrc_t r, uint32_t voff, int kb) {
  const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, kb * BK, 0));
  const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 64, kb * BK, 0));
  v8i v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

template <int SM, int SA_FMT, int SB_FMT>
__global__ __launch_bounds__(64 * SmallCfg<SM>::kWaves, 1) void gemm_small_m_kernel(GemmParams p) {
  constexpr int P = SmallCfg<SM>::P, kSmallWaves = SmallCfg<SM>::kWaves;
  constexpr int sab = SA_FMT == FP8Q_SCALE_F32 ? 4 : 1, sbb = SB_FMT == FP8Q_SCALE_F32 ? 4 : 1;
  __shared__ v4f red[kSmallWaves][SM][64];
  // Every parameter is read here, before any branch, so the kernel-argument loads go out as
  // one batch (read where they are used, they became several dependent round trips). The
  // launcher guarantees that every offset below fits in 31 bits.
  const uint8_t* const A = p.a;
  const uint8_t* const B = p.b;
  const uint8_t* const SA = static_cast<const uint8_t*>(p.sa);
  const uint8_t* const SB = static_cast<const uint8_t*>(p.sb);
  uint16_t* const Y = p.y;
  const int M = static_cast<int>(p.M), N = static_cast<int>(p.N), nkb = static_cast<int>(p.K / BK);
  const int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);
  const int sa_sm = static_cast<int>(p.sa_sm), sa_sk = static_cast<int>(p.sa_sk);
  const int sb_sn = static_cast<int>(p.sb_sn), sb_sk = static_cast<int>(p.sb_sk);
  const int64_t ldy = p.ldy;
  const bool packed = p.sa_packed != 0;
  // (an empty statement that uses every parameter: it keeps the compiler from sinking their
  // loads into later blocks)
  asm volatile("" ::"s"(A), "s"(B), "s"(SA), "s"(SB), "s"(Y), "s"(M), "s"(N), "s"(nkb), "s"(lda), "s"(ldb),
               "s"(ldy), "s"(sa_sm), "s"(sa_sk), "s"(sb_sn), "s"(sb_sk), "s"(p.sa_packed));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16;
  const int kb_beg = (nkb * wave) / kSmallWaves, kb_end = (nkb * (wave + 1)) / kSmallWaves;
  const int l16 = lane & 15, chunk = (lane >> 4) * 16;
  // B: this workgroup's rows (fewer than 16 in the last one); A: all M rows
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(B + static_cast<int64_t>(n0) * ldb), 0, min(16, N - n0) * ldb, kBufWord3);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A), 0, M * lda, kBufWord3);
  const uint32_t wo = static_cast<uint32_t>(l16 * ldb + chunk);
  uint32_t xo[SM], sa_row[SM];
#pragma unroll
  for (int i = 0; i < SM; i++) {
    xo[i] = static_cast<uint32_t>((i * 16 + l16) * lda + chunk);
    // activation scale (m, kb) at byte sa_row[i] + sa_col(kb): packed UE8M0 words hold K
    // blocks 4j..4j+3 of a row in bytes 0..3 (strides in words), other layouts one element
    // per (m, kb); rows past M read row M - 1
    const int m = min(i * 16 + l16, M - 1);
    sa_row[i] = static_cast<uint32_t>(packed ? 4 * m * sa_sm : m * sa_sm * sab);
  }
  auto sa_col = [&](int kb) -> uint32_t {
    return static_cast<uint32_t>(packed ? 4 * (kb >> 2) * sa_sk + (kb & 3) : kb * sa_sk * sab);
  };
  const uint8_t* const sb_row = SB + static_cast<int64_t>((n0 / 128) * sb_sn) * sbb;

  struct Pass {
    v8i w[P];
    v8i x[P][SM];
    uint32_t sa[P][SM];
    uint32_t sb[P];
  };
  // loads of blocks kb0 .. kb0+P-1; indices past the wave's range reload its last block
  // (a wave with an empty range, when K has fewer than one block per wave, reloads block 0),
  // whose products are then not added
  const int kb_last = max(kb_end - 1, 0);
  auto issue = [&](Pass& b, int kb0) {
#pragma unroll
    for (int u = 0; u < P; u++) {
      const int kb = min(kb0 + u, kb_last);
      b.w[u] = frag_buffer(rb, wo, kb);
      const uint32_t sc = sa_col(kb);
#pragma unroll
      for (int i = 0; i < SM; i++) {
        b.x[u][i] = frag_buffer(ra, xo[i], kb);
        const uint32_t so = sa_row[i] + sc;
        b.sa[u][i] = SA_FMT == FP8Q_SCALE_F32 ? *reinterpret_cast<const uint32_t*>(SA + so) : SA[so];
      }
      const uint32_t bo = static_cast<uint32_t>(kb * sb_sk * sbb);
      b.sb[u] = SB_FMT == FP8Q_SCALE_F32 ? *reinterpret_cast<const uint32_t*>(sb_row + bo) : sb_row[bo];
    }
  };
  v4f acc[SM];
#pragma unroll
  for (int i = 0; i < SM; i++) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  // products of blocks outside the range are computed and dropped (a select, no branch)
  auto compute = [&](const Pass& b, int kb0) {
#pragma unroll
    for (int u = 0; u < P; u++) {
      const bool valid = kb0 + u < kb_end;
      const float sbv = scale_value<SB_FMT>(b.sb[u]);
#pragma unroll
      for (int i = 0; i < SM; i++) {
        const v4f z = {0.f, 0.f, 0.f, 0.f};
        const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b.w[u], b.x[u][i], z, 0, 0, 0, 0, 0, 0);
        const float sv = scale_value<SA_FMT>(b.sa[u][i]) * sbv;
#pragma unroll
        for (int r = 0; r < 4; r++) acc[i][r] = valid ? fmaf(pr[r], sv, acc[i][r]) : acc[i][r];
      }
    }
  };
  Pass b0, b1;
  issue(b0, kb_beg);
  issue(b1, kb_beg + P);
  for (int kb0 = kb_beg;; kb0 += 2 * P) {
    compute(b0, kb0);
    if (kb0 + P >= kb_end) break;
    if (kb0 + 2 * P < kb_end) issue(b0, kb0 + 2 * P);
    compute(b1, kb0 + P);
    if (kb0 + 2 * P >= kb_end) break;
    if (kb0 + 3 * P < kb_end) issue(b1, kb0 + 3 * P);
  }
#pragma unroll
  for (int i = 0; i < SM; i++) red[wave][i][lane] = acc[i];
  __syncthreads();
  // wave w finishes 16-row slices w, w + kSmallWaves, ...: the partials added in wave order
  for (int i = wave; i < SM; i += kSmallWaves) {
    v4f t = red[0][i][lane];
#pragma unroll
    for (int w = 1; w < kSmallWaves; w++) {
      const v4f o = red[w][i][lane];
      t[0] += o[0]; t[1] += o[1]; t[2] += o[2]; t[3] += o[3];
    }
    const int m = i * 16 + l16;
    if (m >= M) continue;
    uint16_t* yrow = Y + m * ldy;
    const int n = n0 + 4 * (lane >> 4);
    const uint32_t h0 = bf16_rne(t[0]), h1 = bf16_rne(t[1]), h2 = bf16_rne(t[2]), h3 = bf16_rne(t[3]);
    if (n + 3 < N) {
      *reinterpret_cast<uint32_t*>(yrow + n) = h0 | (h1 << 16);
      *reinterpret_cast<uint32_t*>(yrow + n + 2) = h2 | (h3 << 16);
    } else {
      if (n < N) yrow[n] = static_cast<uint16_t>(h0);
      if (n + 1 < N) yrow[n + 1] = static_cast<uint16_t>(h1);
      if (n + 2 < N) yrow[n + 2] = static_cast<uint16_t>(h2);
    }
  }
}

// Whether every offset of the small-M kernel fits in 31 bits (else the large kernels run it).
bool small_m_fits(const GemmParams& p) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t sab = p.sa_fmt == FP8Q_SCALE_F32 ? 4 : 1, sbb = p.sb_fmt == FP8Q_SCALE_F32 ? 4 : 1;
  const int64_t nkb = p.K / BK;
  const int64_t sa_max = p.sa_packed ? 4 * ((p.M - 1) * p.sa_sm + ((nkb - 1) / 4) * p.sa_sk) + 3
                                     : ((p.M - 1) * p.sa_sm + (nkb - 1) * p.sa_sk) * sab + sab;
  const int64_t sb_max = (((p.N - 1) / 128) * p.sb_sn + (nkb - 1) * p.sb_sk) * sbb + sbb;
  return p.M * p.lda < lim && 16 * p.ldb < lim && p.N < (int64_t(1) << 30) && sa_max < lim && sb_max < lim &&
         p.lda < lim && p.ldb < lim && p.K < lim;
}

template <int SM, int SA_FMT, int SB_FMT>
void launch_small_m_sm(const GemmParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.N + 15) / 16)), block(64 * SmallCfg<SM>::kWaves);
  hipLaunchKernelGGL((gemm_small_m_kernel<SM, SA_FMT, SB_FMT>), grid, block, 0, s, p);
}

// M <= kSmallMaxM: the register kernel above; larger M (up to kSkinnyMaxM) takes the split-K
// kernel below when the caller gives a workspace, else the LDS-staged kernel, which moves
// whole cache lines (there every workgroup streams all of A). Graph-replayed at N = 4096,
// K = 7168: M = 32 in the register kernel (two 16-row slices) 16.7 us, split-K 13.7, the
// LDS-staged kernel 14.7; at M = 128 the register kernel measured 36.6 against 23.5 us.
constexpr int64_t kSmallMaxM = 16;

template <int SA_FMT, int SB_FMT>
void launch_small_m(const GemmParams& p, hipStream_t s) {
  launch_small_m_sm<1, SA_FMT, SB_FMT>(p, s);
}

template <int SM, int SA_FMT, int SB_FMT>
void launch_skinny(const GemmParams& p, hipStream_t s) {
  const int grid = static_cast<int>((p.N + 15) / 16);
  hipLaunchKernelGGL((gemm_skinny_kernel<SM, SA_FMT, SB_FMT>), dim3(grid), dim3(kSkinnyThreads), 0, s, p);
}

template <int SA_FMT, int SB_FMT>
void launch_skinny_m(const GemmParams& p, hipStream_t s) {
  if (p.M <= 16) launch_skinny<1, SA_FMT, SB_FMT>(p, s);
  else if (p.M <= 32) launch_skinny<2, SA_FMT, SB_FMT>(p, s);
  else if (p.M <= 64) launch_skinny<4, SA_FMT, SB_FMT>(p, s);
  else launch_skinny<8, SA_FMT, SB_FMT>(p, s);
}

template <int SM, int SA_FMT>
int launch_skinny_dma(const GemmParams& p, size_t lds, hipStream_t s) {
  auto kern = gemm_skinny_dma_kernel<SM, SA_FMT>;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return -1;
  hipLaunchKernelGGL(kern, dim3(static_cast<int>((p.N + 15) / 16)), dim3(kSkinnyThreads), lds, s, p);
  return 0;
}

// The LDS-staged small-M kernel when its scale tables and rings fit (any BLOCK128 scale
// layout; weight-block scales decoded to fp32 in its table); returns false to use the
// register-loading one.
bool try_skinny_dma(const GemmParams& p, hipStream_t s) {
  if (p.lda >= (int64_t(1) << 25) || p.ldb >= (int64_t(1) << 28)) return false;
  const int sm = p.M <= 16 ? 1 : (p.M <= 32 ? 2 : (p.M <= 64 ? 4 : 8));
  const size_t lds = skinny_dma_lds(sm, p.sa_fmt, p.K / BK);
  if (lds > 160 * 1024) return false;
  const bool f = p.sa_fmt == FP8Q_SCALE_F32;
  int rc;
  switch (sm) {
    case 1: rc = f ? launch_skinny_dma<1, FP8Q_SCALE_F32>(p, lds, s) : launch_skinny_dma<1, FP8Q_SCALE_UE8M0>(p, lds, s); break;
    case 2: rc = f ? launch_skinny_dma<2, FP8Q_SCALE_F32>(p, lds, s) : launch_skinny_dma<2, FP8Q_SCALE_UE8M0>(p, lds, s); break;
    case 4: rc = f ? launch_skinny_dma<4, FP8Q_SCALE_F32>(p, lds, s) : launch_skinny_dma<4, FP8Q_SCALE_UE8M0>(p, lds, s); break;
    default: rc = f ? launch_skinny_dma<8, FP8Q_SCALE_F32>(p, lds, s) : launch_skinny_dma<8, FP8Q_SCALE_UE8M0>(p, lds, s); break;
  }
  return rc == 0;
}

// ------------------------------------------------------------------ small M, split K
// For 16 < M <= 128 the kernels above give every workgroup 16 columns and all of K, so each
// streams all M x K of A through its CU (0.9 MB at M = 128, 256 times over). Here a workgroup
// owns C = 64 NF columns (four waves, NF 16-column MFMA slices each) and one of S contiguous
// ranges of the K blocks, so A is read once per C columns and per range while the grid
// (ceil(N / C) x S workgroups) still fills the chip.
//   * The A rows of the whole range go to LDS (straight from global memory, whole cache
//     lines) before anything else is issued, so the only loads still in flight afterwards
//     are the B fragments, and the waits the compiler places before each MFMA wait for
//     exactly the fragment it reads: the loop runs while B streams in.
//   * Each wave loads its B fragments of the whole range into registers (buffer loads of
//     each row's contiguous K range, issued back to back, so the rows stream from HBM
//     together).
//   * The steps are software-pipelined: step i reads the A fragments of block i + 1 from
//     LDS, runs the MFMAs of block i (each into its own registers) and scales and adds the
//     products of block i - 1, so LDS, the matrix core and the vector ALU work at once.
// With S > 1 the partial sums go to an fp32 workspace [S][M][N] and a second kernel adds
// them in range order (fixed, so results are reproducible) and rounds to bf16; with S == 1
// the bf16 output is stored directly.
template <int SM>
struct SplitCfg {
  static constexpr int MR = 16 * SM;              // A rows held per block
  static constexpr int NF = SM == 8 ? 2 : 1;      // 16-column slices per wave
  static constexpr int C = 64 * NF;               // columns per workgroup
  static constexpr int kMaxBlocks = SM == 8 ? 7 : 14;  // K blocks of a range (registers)
  static constexpr int kLoads = MR / 32;          // 1 KB A pieces per wave and block
  static constexpr int kA = kMaxBlocks * MR * BK; // 112 KB
  static constexpr int kLds = kA + kMaxBlocks * (MR + 1) * 4;
  static_assert(kLds <= 160 * 1024, "A range and scale tables fit in LDS");
  static_assert(C % 128 == 0 || 128 % C == 0, "a column tile lies in one weight scale block");
};

template <int SM, int SA_FMT, int SB_FMT>
__global__ __launch_bounds__(256, 1) void gemm_splitk_kernel(GemmParams p, int S) {
  using D = SplitCfg<SM>;
  constexpr int MR = D::MR, NF = D::NF, KL = D::kLoads, NB = D::kMaxBlocks;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint8_t* const A = p.a;
  const uint8_t* const B = p.b;
  const int M = static_cast<int>(p.M), N = static_cast<int>(p.N), nkb = static_cast<int>(p.K / BK);
  const int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = blockIdx.x % S, nt = blockIdx.x / S;
  const int n0 = nt * D::C;
  const int kb0 = (nkb * ks) / S, nblk = (nkb * (ks + 1)) / S - kb0;  // 1 <= nblk <= NB (host)
  float* const sa_tab = reinterpret_cast<float*>(smem + D::kA);     // [nblk][MR]
  float* const sb_tab = sa_tab + NB * MR;                           // [nblk]

  // 1. scale tables of the range: rows past M repeat row M - 1 (their outputs are not stored)
  constexpr int U = (NB * MR + 255) / 256;  // entries per thread
  const int total = nblk * MR;
  uint32_t tv[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const int idx = tid + u * 256;
    tv[u] = 0;
    if (idx < total) {
      const int64_t si = sa_index(p, min(idx % MR, M - 1), kb0 + idx / MR);
      tv[u] = SA_FMT == FP8Q_SCALE_F32 ? static_cast<const uint32_t*>(p.sa)[si] : static_cast<const uint8_t*>(p.sa)[si];
    }
  }
  uint32_t tw = 0;
  if (tid < nblk) {
    const int64_t bi = (n0 / 128) * p.sb_sn + static_cast<int64_t>(kb0 + tid) * p.sb_sk;
    tw = SB_FMT == FP8Q_SCALE_F32 ? static_cast<const uint32_t*>(p.sb)[bi] : static_cast<const uint8_t*>(p.sb)[bi];
  }

  // 2. A blocks kb0 .. kb0 + nblk - 1, rows 0 .. MR - 1 (rows past M read row M - 1). Block i
  // is at LDS i * MR * BK; the wave's 1 KB pieces q = wave * KL + j hold rows 8q .. 8q + 7
  // (lane l: row 8q + l/8, LDS chunk l%8 = logical chunk (l%8) ^ swz(row)).
  {
    uint32_t voff[KL];
#pragma unroll
    for (int j = 0; j < KL; j++) {
      const int row = (wave * KL + j) * 8 + (lane >> 3), c = (lane & 7) ^ swz(row);
      voff[j] = static_cast<uint32_t>(min(row, M - 1) * lda + c * 16);
    }
    const uint32_t base = lds_addr(smem);
    for (int i = 0; i < nblk; i++) {
#pragma unroll
      for (int j = 0; j < KL; j++) dma16(base + i * MR * BK + (wave * KL + j) * 1024, A + (kb0 + i) * BK, voff[j]);
    }
  }
  asm volatile("" ::: "memory");

  // 3. B: rows n0 + 16 (NF wave + f) + lane%16 of the range, fragments straight to registers
  // (rows past N read as zeros: the buffer ends at row N - 1). The first kLead blocks now
  // (blocks past the range repeat the last one, so every wave issues 2 NF kLead loads), each
  // later one kLead steps ahead of its use: the requests of all CUs then reach memory
  // roughly in block order, so early blocks return early and the steps overlap the stream.
  // With 64 rows (a quarter of the MFMAs per step) everything at once measured faster.
  constexpr int kLead = SM == 8 ? 4 : NB;
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(B + static_cast<int64_t>(n0) * ldb), 0, min(D::C, N - n0) * ldb, kBufWord3);
  uint32_t wo[NF];
#pragma unroll
  for (int f = 0; f < NF; f++) wo[f] = static_cast<uint32_t>(((wave * NF + f) * 16 + l16) * ldb + (lane >> 4) * 16);
  v8i wf[NF][NB];
#pragma unroll
  for (int u = 0; u < kLead; u++) {
#pragma unroll
    for (int f = 0; f < NF; f++) wf[f][u] = frag_buffer(rb, wo[f], kb0 + min(u, nblk - 1));
  }
  asm volatile("" ::: "memory");

  // 4. the tables and this wave's A pieces have landed once at most the B loads are in flight
  wait_vmcnt<2 * NF * kLead>();
#pragma unroll
  for (int u = 0; u < U; u++) {
    const int idx = tid + u * 256;
    if (idx < total) sa_tab[idx] = scale_value<SA_FMT>(tv[u]);
  }
  if (tid < nblk) sb_tab[tid] = scale_value<SB_FMT>(tw);
  // every wave's A pieces and table entries are in LDS (a bare barrier: __syncthreads would
  // also wait for the B loads)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  v4f acc[NF][SM];
#pragma unroll
  for (int f = 0; f < NF; f++)
#pragma unroll
    for (int j = 0; j < SM; j++) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v8i xf[2][SM];   // A fragments of blocks i (xf[i & 1]) and i + 1
  v4f pr[2][NF][SM];  // products of blocks i (pr[i & 1]) and i - 1
  float sv[SM];    // scales of the block being added
  // products of block b (held in pr[h]) scaled by their row and block scales into acc
  auto add_block = [&](int h, int b) {
#pragma unroll
    for (int j = 0; j < SM; j++)
#pragma unroll
      for (int f = 0; f < NF; f++)
#pragma unroll
        for (int r = 0; r < 4; r++) acc[f][j][r] = fmaf(pr[h][f][j][r], sv[j], acc[f][j][r]);
    (void)b;
  };
  auto load_scales = [&](int b) {
    const float sbv = sb_tab[b];
#pragma unroll
    for (int j = 0; j < SM; j++) sv[j] = sa_tab[b * MR + j * 16 + l16] * sbv;
  };
#pragma unroll
  for (int j = 0; j < SM; j++) xf[0][j] = frag(smem, j * 16, lane);
#pragma unroll
  for (int i = 0; i < NB; i++) {
    if (i < nblk) {
      const int h = i & 1;
      if (i > 0) load_scales(i - 1);  // before the prefetch: LDS reads complete in order
      if (i + 1 < nblk) {
        const uint8_t* st = smem + (i + 1) * MR * BK;
#pragma unroll
        for (int j = 0; j < SM; j++) xf[h ^ 1][j] = frag(st, j * 16, lane);
      }
      if (i + kLead < NB && i + kLead < nblk) {
#pragma unroll
        for (int f = 0; f < NF; f++) wf[f][i + kLead] = frag_buffer(rb, wo[f], kb0 + i + kLead);
      }
      const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < NF; f++)
#pragma unroll
        for (int j = 0; j < SM; j++)
          pr[h][f][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[f][i], xf[h][j], z, 0, 0, 0, 0, 0, 0);
      if (i > 0) add_block(h ^ 1, i - 1);
    }
  }
  load_scales(nblk - 1);
  if ((nblk - 1) & 1)
    add_block(1, nblk - 1);
  else
    add_block(0, nblk - 1);

  // lane holds rows m = 16 j + lane%16, columns n .. n+3, n = n0 + 16 (NF wave + f) + 4 (lane/16)
#pragma unroll
  for (int f = 0; f < NF; f++) {
    const int n = n0 + (wave * NF + f) * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < SM; j++) {
      const int m = j * 16 + l16;
      if (m >= M) continue;
      if (S > 1) {
        float* prow = p.ws + (static_cast<int64_t>(ks) * M + m) * N;
        if (n + 3 < N && (N & 3) == 0) {
          *reinterpret_cast<v4f*>(prow + n) = acc[f][j];
        } else {
#pragma unroll
          for (int r = 0; r < 4; r++)
            if (n + r < N) prow[n + r] = acc[f][j][r];
        }
      } else {
        uint16_t* yrow = p.y + m * p.ldy;
        const uint32_t h0 = bf16_rne(acc[f][j][0]), h1 = bf16_rne(acc[f][j][1]);
        const uint32_t h2 = bf16_rne(acc[f][j][2]), h3 = bf16_rne(acc[f][j][3]);
        if (n + 3 < N) {
          *reinterpret_cast<uint32_t*>(yrow + n) = h0 | (h1 << 16);
          *reinterpret_cast<uint32_t*>(yrow + n + 2) = h2 | (h3 << 16);
        } else {
          if (n < N) yrow[n] = static_cast<uint16_t>(h0);
          if (n + 1 < N) yrow[n + 1] = static_cast<uint16_t>(h1);
          if (n + 2 < N) yrow[n + 2] = static_cast<uint16_t>(h2);
        }
      }
    }
  }
}

constexpr int kMaxSplit = 16;
constexpr int kMinRangeBlocks = 4;

// Y[m][n] = bf16( sum over the S ranges, in range order, of part[s][m][n] ); each thread four
// consecutive columns of one row, all S loads issued before the first add.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S, int M, int N,
                                                            uint16_t* __restrict__ y, int64_t ldy) {
  const int nq = (N + 3) / 4;
  const int64_t total = static_cast<int64_t>(M) * nq;
  const int64_t plane = static_cast<int64_t>(M) * N;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; t < total;
       t += static_cast<int64_t>(gridDim.x) * 256) {
    const int m = static_cast<int>(t / nq), n = static_cast<int>(t % nq) * 4;
    const float* src = part + static_cast<int64_t>(m) * N + n;
    uint16_t* yrow = y + m * ldy;
    if (n + 3 < N && (N & 3) == 0) {
      v4f v[kMaxSplit];
#pragma unroll
      for (int s = 0; s < kMaxSplit; s++)
        if (s < S) v[s] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + s * plane));
      v4f a = v[0];
#pragma unroll
      for (int s = 1; s < kMaxSplit; s++)
        if (s < S) { a[0] += v[s][0]; a[1] += v[s][1]; a[2] += v[s][2]; a[3] += v[s][3]; }
      *reinterpret_cast<uint32_t*>(yrow + n) = bf16_rne(a[0]) | (bf16_rne(a[1]) << 16);
      *reinterpret_cast<uint32_t*>(yrow + n + 2) = bf16_rne(a[2]) | (bf16_rne(a[3]) << 16);
    } else {
      for (int r = 0; r < 4 && n + r < N; r++) {
        float a = src[r];
        for (int s = 1; s < S; s++) a += src[r + s * plane];
        yrow[n + r] = static_cast<uint16_t>(bf16_rne(a));
      }
    }
  }
}

// The split for a problem on `cus` CUs: sm 16-row slices of A (M <= 64: 4, else 8), the
// fewest ranges that keep every range within the blocks a workgroup holds, raised (up to
// kMaxSplit) until the grid fills the chip, but not below kMinRangeBlocks blocks per range
// unless the register limit needs shorter ones: for a small problem a second launch (the
// reduction) costs more than the parallelism buys (M=64, N=256, K=512: 7.8 us with 4 ranges,
// 5.7 us with one). Ranges differ by at most one block.
struct SplitPlan {
  int sm;      // 4 or 8
  int S;       // K ranges
  int64_t ws;  // workspace bytes (0 when S == 1)
  bool ok;
};

SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int cus) {
  SplitPlan pl{M <= 64 ? 4 : 8, 1, 0, false};
  if (M <= kSmallMaxM || M > kSkinnyMaxM || K % BK != 0 || N < 1) return pl;
  const int64_t nkb = K / BK;
  const int64_t C = pl.sm == 8 ? SplitCfg<8>::C : SplitCfg<4>::C;
  const int64_t nbmax = pl.sm == 8 ? SplitCfg<8>::kMaxBlocks : SplitCfg<4>::kMaxBlocks;
  const int64_t tiles = (N + C - 1) / C;
  const int64_t s_min = (nkb + nbmax - 1) / nbmax;  // ranges short enough for the registers
  const int64_t s_fill = std::max<int64_t>(1, std::min<int64_t>(cus / tiles, kMaxSplit));
  const int64_t s_len = std::max<int64_t>(1, nkb / kMinRangeBlocks);  // ranges of >= kMinRangeBlocks blocks
  const int64_t S = std::max(s_min, std::min<int64_t>(std::min(s_fill, s_len), nkb));
  if (S > kMaxSplit || (nkb + S - 1) / S > nbmax) return pl;
  pl.S = static_cast<int>(S);
  pl.ws = S > 1 ? S * M * N * 4 : 0;
  pl.ok = true;
  return pl;
}

template <int SM, int SA_FMT, int SB_FMT>
int launch_splitk_sm(const GemmParams& p, int S, hipStream_t s) {
  using D = SplitCfg<SM>;
  auto kern = gemm_splitk_kernel<SM, SA_FMT, SB_FMT>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, D::kLds) !=
      hipSuccess)
    return -1;
  const int grid = static_cast<int>((p.N + D::C - 1) / D::C) * S;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), D::kLds, s, p, S);
  if (S > 1) {
    const int64_t work = p.M * ((p.N + 3) / 4);
    const int rgrid = static_cast<int>(std::min<int64_t>((work + 255) / 256, 4096));
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(rgrid), dim3(256), 0, s, static_cast<const float*>(p.ws), S,
                       static_cast<int>(p.M), static_cast<int>(p.N), p.y, p.ldy);
  }
  return 0;
}

// The split-K path when the problem fits it and the workspace is large enough; false to use
// another kernel.
bool try_splitk(const GemmParams& p, const DeviceShape& ds, hipStream_t s) {
  const SplitPlan pl = split_plan(p.M, p.N, p.K, ds.cus);
  if (!pl.ok || (pl.S > 1 && (p.ws == nullptr || p.ws_bytes < pl.ws))) return false;
  if ((reinterpret_cast<uintptr_t>(p.ws) & 15) != 0) return false;
  // every offset of the kernel in 31 bits
  const int64_t lim = int64_t(1) << 31;
  if (p.M * p.lda >= lim || 128 * p.ldb >= lim || p.N >= (int64_t(1) << 30) || p.K >= lim || p.M * p.ldy >= lim)
    return false;
  const bool f = p.sa_fmt == FP8Q_SCALE_F32, g = p.sb_fmt == FP8Q_SCALE_F32;
  int rc;
  if (pl.sm == 4) {
    rc = f ? (g ? launch_splitk_sm<4, FP8Q_SCALE_F32, FP8Q_SCALE_F32>(p, pl.S, s)
                : launch_splitk_sm<4, FP8Q_SCALE_F32, FP8Q_SCALE_UE8M0>(p, pl.S, s))
           : (g ? launch_splitk_sm<4, FP8Q_SCALE_UE8M0, FP8Q_SCALE_F32>(p, pl.S, s)
                : launch_splitk_sm<4, FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, pl.S, s));
  } else {
    rc = f ? (g ? launch_splitk_sm<8, FP8Q_SCALE_F32, FP8Q_SCALE_F32>(p, pl.S, s)
                : launch_splitk_sm<8, FP8Q_SCALE_F32, FP8Q_SCALE_UE8M0>(p, pl.S, s))
           : (g ? launch_splitk_sm<8, FP8Q_SCALE_UE8M0, FP8Q_SCALE_F32>(p, pl.S, s)
                : launch_splitk_sm<8, FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, pl.S, s));
  }
  return rc == 0;
}

template <class C, bool MX, int SA_FMT, int SB_FMT>
void launch(const GemmParams& p, int grid, hipStream_t s) {
  const size_t lds = (p.masked_m || p.seg_indptr) ? static_cast<size_t>(p.E + 1) * sizeof(int32_t) : 0;
  hipLaunchKernelGGL((gemm_kernel<C, MX, SA_FMT, SB_FMT>), dim3(grid), dim3(C::kThreads), lds, s, p);
}

// Persistent grid: one resident workgroup per CU (at most as many as tiles), a multiple of
// the XCD count so that every XCD runs the same number of workgroups.
int grid_for(int64_t tiles, const DeviceShape& ds) {
  int64_t g = std::min<int64_t>(tiles, ds.cus);
  g = ((g + ds.xcds - 1) / ds.xcds) * ds.xcds;
  return static_cast<int>(std::max<int64_t>(g, ds.xcds));
}

int finish(const char* what) {
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(FP8Q_ELAUNCH, std::string(what) + ": " + hipGetErrorString(err));
  return FP8Q_OK;
}

// Whether the direct-to-LDS kernel can move this problem's scales (see its description),
// and with which scale mode; -1 selects the register-staged kernel.
bool u32_ok(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

int dma_mode(const GemmParams& p, bool mx) {
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (p.lda >= (int64_t(1) << 24) || p.ldb >= (int64_t(1) << 24)) return -1;
  const bool k512 = p.K % 512 == 0;
  if (mx) {
    // per operand: a row-major byte layout (4-byte words per step) or packed words with
    // any word strides; the 32-bit lane offsets of a 256-row tile must fit
    auto operand_ok = [&](bool packed, int64_t sm, int64_t sk, const void* s) {
      if (packed) return sm < (int64_t(1) << 22);
      return sk == 1 && sm < (int64_t(1) << 24) && sm % 4 == 0 && u32_ok(s);
    };
    if (!operand_ok(p.sa_packed, p.sa_sm, p.sa_sk, p.sa) || !operand_ok(p.sb_packed, p.sb_sn, p.sb_sk, p.sb)) return -1;
    if (!p.sa_packed && !p.sb_packed && k512 && p.sa_sm % 16 == 0 && p.sb_sn % 16 == 0 && a16(p.sa) && a16(p.sb))
      return kScMxGrp;
    return kScMx;
  }
  const int64_t E = (p.masked_m || p.seg_indptr) ? p.E : 1;  // groups in the device tile list
  if (p.sb_fmt != FP8Q_SCALE_F32) {
    // UE8M0 weight-block bytes, row-major [N/128][K/128] in whole 4-byte words (per weight),
    // with UE8M0 column-major activation scales: both go to the matrix core
    const bool w8 = p.sb_fmt == FP8Q_SCALE_UE8M0 && !p.sa_packed && p.sa_fmt == FP8Q_SCALE_UE8M0 && p.sb_sk == 1 &&
                    p.sb_sn % 4 == 0 && p.sb_sn < (int64_t(1) << 30) && (p.K / BK) % 4 == 0 && u32_ok(p.sb) &&
                    ((E == 1 && p.W <= 1) || p.sb_se % 4 == 0);
    if (p.sa_packed) {
      const bool w8p = p.sb_fmt == FP8Q_SCALE_UE8M0 && p.sb_sk == 1 && p.sb_sn % 4 == 0 &&
                       p.sb_sn < (int64_t(1) << 30) && (p.K / BK) % 4 == 0 && u32_ok(p.sb) &&
                       ((E == 1 && p.W <= 1) || p.sb_se % 4 == 0);
      return w8p && p.sa_sm < (int64_t(1) << 22) && E <= DmaLayout<kScPkE8, DmaCfg>::kMaxPrefix ? kScPkE8 : -1;
    }
    const bool col = p.sa_sm == 1 && p.sa_sk % 4 == 0 && p.M % 4 == 0 && u32_ok(p.sa) && !p.seg_indptr &&
                     (p.masked_m == nullptr || p.sa_se % 4 == 0) && E <= DmaLayout<kScE8E8, DmaCfg>::kMaxPrefix;
    return w8 && col ? kScE8E8 : -1;
  }
  if (p.sa_packed)
    return p.sa_sm < (int64_t(1) << 22) && E <= DmaLayout<kScE8Pk, DmaCfg>::kMaxPrefix ? kScE8Pk : -1;
  if (p.sa_fmt == FP8Q_SCALE_F32) {
    if (p.sa_sm >= (int64_t(1) << 22)) return -1;
    const bool grp = k512 && p.sa_sk == 1 && p.sa_sm % 4 == 0 && a16(p.sa) && p.sb_sk == 1 && p.sb_sn % 4 == 0 &&
                     a16(p.sb) && (E == 1 || (p.sa_se % 4 == 0 && p.sb_se % 4 == 0)) &&
                     E <= DmaLayout<kScF32Grp, DmaCfg>::kMaxPrefix;
    if (grp) return kScF32Grp;
    return E <= DmaLayout<kScF32Row, DmaCfg>::kMaxPrefix ? kScF32Row : -1;
  }
  // (segments start at any row, so their byte columns are not 4-byte aligned)
  const bool col = p.sa_sm == 1 && p.sa_sk % 4 == 0 && p.M % 4 == 0 && u32_ok(p.sa) && !p.seg_indptr &&
                   (p.masked_m == nullptr || p.sa_se % 4 == 0) && E <= DmaLayout<kScE8Col, DmaCfg>::kMaxPrefix;
  return col ? kScE8Col : -1;
}

template <int SCM, class C = DmaCfg>
void launch_dma(const GemmParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_dma_kernel<SCM, C>), dim3(grid), dim3(C::kThreads), 0, s, p);
}

}  // namespace

// Flat problems with at least one full round of 256x256 tiles: the columns [0, n1) that
// should run as 256x256 tiles when the rest runs as 128x256 tiles in a second launch, or 0
// for one launch. Cost in rounds of 256x256 tiles; a 128x256 tile takes about 0.8 of one
// (half the MFMA work at a lower MFMA utilisation; measured on 8192x7168x2048, where the
// split takes 143 instead of 150 us). A split must save at least 3%.
int64_t wide_split_columns(const GemmParams& p, int64_t cus) {
  const int64_t mt = (p.M + 255) / 256, nt = (p.N + 255) / 256, mh = (p.M + 127) / 128;
  auto rounds = [cus](int64_t tiles) { return static_cast<double>((tiles + cus - 1) / cus); };
  const double whole = rounds(mt * nt);
  double best = whole;
  int64_t best_n1 = 0;
  for (int64_t nt1 = nt - 1; nt1 >= 1; nt1--) {  // on equal cost, the most columns in 256x256 tiles
    const double c = rounds(mt * nt1) + 0.8 * rounds(mh * (nt - nt1));
    if (c < best) {
      best = c;
      best_n1 = nt1 * 256;
    }
  }
  return best < 0.97 * whole ? best_n1 : 0;
}

// UE8M0 activation scales stored row-major ([rows][K/128] bytes, K % 512 == 0) whose rows
// and expert blocks start on 4-byte boundaries are packed words under another name: byte kb
// of row m is byte kb % 4 of word m * (sa_sm / 4) + kb / 4. They are read as such, which
// gives them the direct-to-LDS kernel's per-row word loads.
GemmParams rows_as_words(const GemmParams& p) {
  GemmParams q = p;
  if (!p.sa_packed && p.sa_fmt == FP8Q_SCALE_UE8M0 && p.sa_sk == 1 && p.sa_sm % 4 == 0 && p.sa_se % 4 == 0 &&
      p.K % 512 == 0 && (reinterpret_cast<uintptr_t>(p.sa) & 3) == 0) {
    q.sa_packed = 1;
    q.sa_sm = p.sa_sm / 4;
    q.sa_se = p.sa_se / 4;
  }
  return q;
}

int launch_gemm_block128(const GemmParams& p_in, int64_t expected_m, hipStream_t stream) {
  using C = Large;
  const DeviceShape ds = current_device_shape();
  GemmParams p = rows_as_words(p_in);
  p.xcds = ds.xcds;
  // launch sizing only (the device tile list decides the work): masked and segment launches
  // use the row hint; a segment adds at most one partial tile
  auto tiles_for = [&](int64_t bm, int64_t bn) -> int64_t {
    const int64_t tn = (p.N + bn - 1) / bn;
    const int64_t rows = expected_m > 0 ? std::min<int64_t>(expected_m, p.M) : p.M;
    if (p.masked_m) return p.E * ((rows + bm - 1) / bm) * tn;
    if (p.seg_indptr) return ((rows + bm - 1) / bm + p.E) * tn;
    return ((p.M + bm - 1) / bm) * tn;
  };
  const int grid = grid_for(tiles_for(C::BM, C::BN), ds);
  const bool a8 = p.sa_fmt == FP8Q_SCALE_UE8M0, b8 = p.sb_fmt == FP8Q_SCALE_UE8M0;
  const bool grouped = p.masked_m || p.seg_indptr || p.m_indices;
  if (!grouped && p.M <= kSmallMaxM && small_m_fits(p)) {
    if (a8 && b8) launch_small_m<FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, stream);
    else if (a8) launch_small_m<FP8Q_SCALE_UE8M0, FP8Q_SCALE_F32>(p, stream);
    else if (b8) launch_small_m<FP8Q_SCALE_F32, FP8Q_SCALE_UE8M0>(p, stream);
    else launch_small_m<FP8Q_SCALE_F32, FP8Q_SCALE_F32>(p, stream);
    return finish("block-scaled GEMM launch");
  }
  if (!grouped && p.M <= kSkinnyMaxM) {
    if (try_splitk(p, ds, stream)) return finish("block-scaled GEMM launch");
    if (try_skinny_dma(p, stream)) return finish("block-scaled GEMM launch");
    if (a8 && b8) launch_skinny_m<FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, stream);
    else if (a8) launch_skinny_m<FP8Q_SCALE_UE8M0, FP8Q_SCALE_F32>(p, stream);
    else if (b8) launch_skinny_m<FP8Q_SCALE_F32, FP8Q_SCALE_UE8M0>(p, stream);
    else launch_skinny_m<FP8Q_SCALE_F32, FP8Q_SCALE_F32>(p, stream);
    return finish("block-scaled GEMM launch");
  }
  const int dm = dma_mode(p, false);
  if (p.m_indices && dm < 0)
    return fail(FP8Q_EUNSUPPORTED, "block-scaled contiguous grouped GEMM: activation scales must be fp32, UE8M0 "
                                   "column-major (rows a multiple of 4) or packed UE8M0 words (or row-major UE8M0 "
                                   "rows of whole words) with fp32 weight "
                                   "scales, or UE8M0 column-major or packed with UE8M0 weight scales in whole "
                                   "4-byte words");
  if ((p.masked_m && (dm == kScE8Col || dm == kScF32Row || dm == kScE8Pk || dm == kScE8E8 || dm == kScPkE8)) ||
      (p.seg_indptr && dm >= 0) || p.m_indices) {
    // grouped: 128-row tiles pad a group's rows to a multiple of 128 instead of 256 (and
    // are the aligned blocks of the contiguous layout)
    using T = DmaCfgT;
    const int g = grid_for(tiles_for(T::BM, T::BN), ds);
    if (dm == kScE8Col) launch_dma<kScE8Col, T>(p, g, stream);
    else if (dm == kScE8E8) launch_dma<kScE8E8, T>(p, g, stream);
    else if (dm == kScPkE8) launch_dma<kScPkE8, T>(p, g, stream);
    else if (dm == kScE8Pk) launch_dma<kScE8Pk, T>(p, g, stream);
    else if (dm == kScF32Grp) launch_dma<kScF32Grp, T>(p, g, stream);
    else launch_dma<kScF32Row, T>(p, g, stream);
    return finish("block-scaled grouped GEMM launch");
  }
  if (!grouped &&
      (dm == kScE8Col || dm == kScF32Row || dm == kScF32Grp || dm == kScE8Pk || dm == kScE8E8 || dm == kScPkE8)) {
    // 256x256 tiles halve the operand bytes each tile loads per output; used when they
    // still give every CU a tile
    using W = DmaCfgW;
    const int64_t wt = ((p.M + W::BM - 1) / W::BM) * ((p.N + W::BN - 1) / W::BN);
    if (wt >= ds.cus) {
      auto wide = [&](const GemmParams& q, int64_t tiles) {
        if (dm == kScE8Col) launch_dma<kScE8Col, W>(q, grid_for(tiles, ds), stream);
        else if (dm == kScE8E8) launch_dma<kScE8E8, W>(q, grid_for(tiles, ds), stream);
        else if (dm == kScPkE8) launch_dma<kScPkE8, W>(q, grid_for(tiles, ds), stream);
        else if (dm == kScE8Pk) launch_dma<kScE8Pk, W>(q, grid_for(tiles, ds), stream);
        else if (dm == kScF32Grp) launch_dma<kScF32Grp, W>(q, grid_for(tiles, ds), stream);
        else launch_dma<kScF32Row, W>(q, grid_for(tiles, ds), stream);
      };
      const int64_t n1 = wide_split_columns(p, ds.cus);
      if (n1 == 0) {
        wide(p, wt);
        return finish("block-scaled GEMM launch");
      }
      // columns [0, n1) in whole rounds of 256x256 tiles, the rest in 128x256 tiles that
      // fill the last round (a second launch on the same stream)
      GemmParams p1 = p, p2 = p;
      p1.N = n1;
      p2.N = p.N - n1;
      p2.b = p.b + n1 * p.ldb;
      p2.sb = static_cast<const uint8_t*>(p.sb) + (n1 / 128) * p.sb_sn * (p.sb_fmt == FP8Q_SCALE_F32 ? 4 : 1);
      p2.y = p.y + n1;
      wide(p1, ((p.M + W::BM - 1) / W::BM) * (n1 / W::BN));
      using T = DmaCfgT;
      const int g = grid_for(((p.M + T::BM - 1) / T::BM) * ((p2.N + T::BN - 1) / T::BN), ds);
      if (dm == kScE8Col) launch_dma<kScE8Col, T>(p2, g, stream);
      else if (dm == kScE8E8) launch_dma<kScE8E8, T>(p2, g, stream);
      else if (dm == kScPkE8) launch_dma<kScPkE8, T>(p2, g, stream);
      else if (dm == kScE8Pk) launch_dma<kScE8Pk, T>(p2, g, stream);
      else if (dm == kScF32Grp) launch_dma<kScF32Grp, T>(p2, g, stream);
      else launch_dma<kScF32Row, T>(p2, g, stream);
      return finish("block-scaled GEMM launch");
    }
  }
  if (dm == kScF32Row) launch_dma<kScF32Row>(p, grid, stream);
  else if (dm == kScF32Grp) launch_dma<kScF32Grp>(p, grid, stream);
  else if (dm == kScE8Col) launch_dma<kScE8Col>(p, grid, stream);
  else if (dm == kScE8E8) launch_dma<kScE8E8>(p, grid, stream);
  else if (dm == kScPkE8) launch_dma<kScPkE8>(p, grid, stream);
  else if (dm == kScE8Pk) launch_dma<kScE8Pk>(p, grid, stream);
  else if (a8 && b8) launch<C, false, FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, grid, stream);
  else if (a8) launch<C, false, FP8Q_SCALE_UE8M0, FP8Q_SCALE_F32>(p, grid, stream);
  else if (b8) launch<C, false, FP8Q_SCALE_F32, FP8Q_SCALE_UE8M0>(p, grid, stream);
  else launch<C, false, FP8Q_SCALE_F32, FP8Q_SCALE_F32>(p, grid, stream);
  return finish("block-scaled GEMM launch");
}

int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const SplitPlan pl = split_plan(M, N, K, current_device_shape().cus);
  return pl.ok ? pl.ws : 0;
}

int launch_gemm_mx32(const GemmParams& p_in, hipStream_t stream) {
  using C = Large;
  const DeviceShape ds = current_device_shape();
  GemmParams p = p_in;
  p.xcds = ds.xcds;
  const int64_t tiles = ((p.M + C::BM - 1) / C::BM) * ((p.N + C::BN - 1) / C::BN);
  const int dm = dma_mode(p, true);
  using W = DmaCfgW;
  const int64_t wt = ((p.M + W::BM - 1) / W::BM) * ((p.N + W::BN - 1) / W::BN);
  if (dm >= 0 && wt >= ds.cus) {
    // 256x256 tiles with per-step scale loads (8 jobs: 256 activation and 256 weight rows),
    // as four waves of 128x128 (one per SIMD): with no fold the 256 accumulators of a lane
    // fit, and each wave reads a quarter less from LDS per MFMA than a 128x64 wave. 8192^3,
    // same box, three interleaved rounds: 482-488 us against 509-515 for eight 128x64 waves.
    launch_dma<kScMx, DmaCfgW4>(p, grid_for(wt, ds), stream);
    return finish("MXFP8 GEMM launch");
  }
  if (dm == kScMxGrp) launch_dma<kScMxGrp>(p, grid_for(tiles, ds), stream);
  else if (dm == kScMx) launch_dma<kScMx>(p, grid_for(tiles, ds), stream);
  else launch<C, true, FP8Q_SCALE_UE8M0, FP8Q_SCALE_UE8M0>(p, grid_for(tiles, ds), stream);
  return finish("MXFP8 GEMM launch");
}

}  // namespace fp8q

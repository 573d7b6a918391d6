// api_gemm.hip — C ABI of the block-scaled GEMM calls: argument validation (host only,
// before any device call), the device check, then the launch. Semantics: include/fp8q.h.
#include "fp8q_internal.h"

#include <mutex>

// Device scratch of fp8q_gemm_blockscaled_noalloc (the split-K partial sums): every device
// the library's code is loaded on holds its own copy until the process ends. Host code uses
// the per-device address from hipGetSymbolAddress, never this name.
static __device__ __align__(256) uint8_t scratch[FP8Q_NOALLOC_SCRATCH_BYTES];

namespace fp8q {
namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];  // device address of `scratch`, per device

// This device's scratch address, looked up on the first call with the device current.
int scratch_address(const std::string& pre, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(FP8Q_EDEVICE, pre + "no current HIP device");
  if (dev >= kScratchDevices) return fail(FP8Q_EUNSUPPORTED, pre + "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(FP8Q_EDEVICE, pre + "hipGetSymbolAddress(scratch) failed: " + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FP8Q_OK;
}

constexpr int64_t kMaxExperts = 4096;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_fmt(int f) { return f == FP8Q_SCALE_F32 || f == FP8Q_SCALE_UE8M0; }

// Checks shared by the dense and the grouped call. rows = rows of A and Y per expert.
int check_operands(const std::string& pre, const uint8_t* a, int64_t lda, const void* sa, int sa_fmt,
                   int64_t sa_sm, int64_t sa_sk, const uint8_t* b, int64_t ldb, const void* sb,
                   int sb_fmt, int64_t sb_sn, int64_t sb_sk, const uint16_t* y, int64_t ldy,
                   int64_t rows, int64_t N, int64_t K, int mode) {
  if (mode != FP8Q_GEMM_BLOCK128 && mode != FP8Q_GEMM_MX32)
    return fail(FP8Q_EUNSUPPORTED, pre + "mode must be BLOCK128 or MX32");
  const bool packed = sa_fmt == FP8Q_SCALE_UE8M0_PACKED;
  const bool b_packed = sb_fmt == FP8Q_SCALE_UE8M0_PACKED;
  if (mode == FP8Q_GEMM_MX32) {
    const bool e8 = (sa_fmt == FP8Q_SCALE_UE8M0 || packed) && (sb_fmt == FP8Q_SCALE_UE8M0 || b_packed);
    if (!e8) return fail(FP8Q_EUNSUPPORTED, pre + "MX32 scales must be E8M0 bytes (UE8M0 or UE8M0_PACKED)");
  } else if (!(valid_fmt(sa_fmt) || packed) || !valid_fmt(sb_fmt)) {
    return fail(FP8Q_EUNSUPPORTED, pre + "scale formats must be F32 or UE8M0 (activation scales also "
                                         "UE8M0_PACKED)");
  }
  if (rows < 0 || N < 0 || K < 0) return fail(FP8Q_EINVAL, pre + "negative size");
  if (K % 128 != 0) return fail(FP8Q_EINVAL, pre + "K must be a multiple of 128");
  if (packed && mode == FP8Q_GEMM_BLOCK128 && K % 512 != 0)
    return fail(FP8Q_EINVAL, pre + "packed UE8M0 activation scales need K a multiple of 512");
  if (lda < 0 || ldb < 0 || ldy < 0 || sa_sm < 0 || sa_sk < 0 || sb_sn < 0 || sb_sk < 0)
    return fail(FP8Q_EINVAL, pre + "negative stride");
  if (rows == 0 || N == 0 || K == 0) return FP8Q_OK;
  if (!a || !b || !y || !sa || !sb) return fail(FP8Q_EINVAL, pre + "null tensor pointer");
  if ((rows > 1 && lda < K) || (N > 1 && ldb < K)) return fail(FP8Q_EINVAL, pre + "lda and ldb must be >= K");
  if (rows > 1 && ldy < N) return fail(FP8Q_EINVAL, pre + "ldy must be >= N (rows of y overlap)");
  if (!aligned(a, 16) || !aligned(b, 16) || lda % 16 != 0 || ldb % 16 != 0)
    return fail(FP8Q_EALIGN, pre + "a, b and their row strides must be 16-byte aligned");
  if (!aligned(y, 4) || ldy % 2 != 0) return fail(FP8Q_EALIGN, pre + "y must be 4-byte aligned with an even ldy");
  if ((sa_fmt != FP8Q_SCALE_UE8M0 && !aligned(sa, 4)) || (sb_fmt != FP8Q_SCALE_UE8M0 && !aligned(sb, 4)))
    return fail(FP8Q_EALIGN, pre + "fp32 scales and packed UE8M0 words must be 4-byte aligned");
  return FP8Q_OK;
}

// shared tail of the two packed-row grouped calls: checks, then the launch
int grouped_rows_entry(const std::string& pre, const uint8_t* a, int64_t lda, const void* sa, int sa_fmt,
                       int64_t sa_sm, int64_t sa_sk, const uint8_t* b, int64_t b_se, int64_t ldb, const void* sb,
                       int sb_fmt, int64_t sb_se, int64_t sb_sn, int64_t sb_sk, uint16_t* y, int64_t ldy,
                       const int32_t* seg_indptr, const int32_t* seg_weight, const int32_t* m_indices, int64_t S,
                       int64_t T, int64_t W, int64_t N, int64_t K, int64_t expected_rows, void* stream) {
  set_error("");
  if (S < 0 || T < 0 || W < 0 || b_se < 0 || sb_se < 0 || expected_rows < 0)
    return fail(FP8Q_EINVAL, pre + "negative size, stride or expected_rows");
  if (T >= (int64_t(1) << 31)) return fail(FP8Q_EUNSUPPORTED, pre + "at most 2^31 - 1 rows");
  if (seg_indptr && S > 2048) return fail(FP8Q_EUNSUPPORTED, pre + "at most 2048 segments");
  // the device builds a 32-bit prefix of the segments' tile counts (segments may overlap,
  // so each can reach every row): bound its total
  if (seg_indptr && S * ((T + 127) / 128) * ((N + 127) / 128) >= (int64_t(1) << 31))
    return fail(FP8Q_EUNSUPPORTED, pre + "too many output tiles over the segments");
  int rc = check_operands(pre, a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, y, ldy, T, N,
                          K, FP8Q_GEMM_BLOCK128);
  if (rc != FP8Q_OK) return rc;
  if (T == 0 || N == 0 || K == 0 || W == 0 || (seg_indptr && S == 0)) return FP8Q_OK;
  if ((seg_indptr == nullptr) == (m_indices == nullptr)) return fail(FP8Q_EINVAL, pre + "row mapping is required");
  if (b_se % 16 != 0) return fail(FP8Q_EALIGN, pre + "weight stride of b must be a multiple of 16 bytes");
  if (W > 1 && b_se < (N - 1) * ldb + K) return fail(FP8Q_EINVAL, pre + "weights of b overlap");
  rc = check_current_device();
  if (rc != FP8Q_OK) return rc;
  GemmParams p{};
  p.a = a;
  p.sa = sa;
  p.b = b;
  p.sb = sb;
  p.y = y;
  p.masked_m = nullptr;
  p.seg_indptr = seg_indptr;
  p.seg_weight = seg_indptr ? seg_weight : nullptr;
  p.m_indices = m_indices;
  p.M = T;
  p.N = N;
  p.K = K;
  p.E = seg_indptr ? S : 1;
  p.W = W;
  p.lda = lda;
  p.ldb = ldb;
  p.ldy = ldy;
  p.b_se = b_se;
  p.sa_sm = sa_sm;
  p.sa_sk = sa_sk;
  p.sb_sn = sb_sn;
  p.sb_sk = sb_sk;
  p.sb_se = sb_se;
  p.sa_packed = sa_fmt == FP8Q_SCALE_UE8M0_PACKED ? 1 : 0;
  p.sa_fmt = p.sa_packed ? FP8Q_SCALE_UE8M0 : sa_fmt;
  p.sb_fmt = sb_fmt;
  return launch_gemm_block128(p, expected_rows, static_cast<hipStream_t>(stream));
}

// the dense call, with an optional fp32 workspace (nullptr: the paths that need none)
int dense_entry(const std::string& pre, const uint8_t* a, int64_t lda, const void* sa, int sa_fmt, int64_t sa_sm,
                int64_t sa_sk, const uint8_t* b, int64_t ldb, const void* sb, int sb_fmt, int64_t sb_sn,
                int64_t sb_sk, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, int mode, float* ws,
                int64_t ws_bytes, void* stream) {
  set_error("");
  int rc = check_operands(pre, a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, y, ldy, M,
                          N, K, mode);
  if (rc != FP8Q_OK || M == 0 || N == 0 || K == 0) return rc;
  rc = check_current_device();
  if (rc != FP8Q_OK) return rc;
  GemmParams p{};
  p.a = a;
  p.sa = sa;
  p.b = b;
  p.sb = sb;
  p.y = y;
  p.masked_m = nullptr;
  p.M = M;
  p.N = N;
  p.K = K;
  p.E = 1;
  p.lda = lda;
  p.ldb = ldb;
  p.ldy = ldy;
  p.sa_sm = sa_sm;
  p.sa_sk = sa_sk;
  p.sb_sn = sb_sn;
  p.sb_sk = sb_sk;
  p.sa_packed = sa_fmt == FP8Q_SCALE_UE8M0_PACKED ? 1 : 0;
  p.sa_fmt = p.sa_packed ? FP8Q_SCALE_UE8M0 : sa_fmt;
  p.sb_packed = sb_fmt == FP8Q_SCALE_UE8M0_PACKED ? 1 : 0;
  p.sb_fmt = p.sb_packed ? FP8Q_SCALE_UE8M0 : sb_fmt;
  p.ws = ws;
  p.ws_bytes = ws_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return mode == FP8Q_GEMM_MX32 ? launch_gemm_mx32(p, s) : launch_gemm_block128(p, 0, s);
}

}  // namespace
}  // namespace fp8q

extern "C" {

int fp8q_gemm_blockscaled(const uint8_t* a, int64_t lda, const void* sa, int sa_fmt, int64_t sa_sm,
                          int64_t sa_sk, const uint8_t* b, int64_t ldb, const void* sb, int sb_fmt,
                          int64_t sb_sn, int64_t sb_sk, uint16_t* y, int64_t ldy, int64_t M, int64_t N,
                          int64_t K, int mode, void* stream) {
  return fp8q::dense_entry("fp8q_gemm_blockscaled: ", a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn,
                           sb_sk, y, ldy, M, N, K, mode, nullptr, 0, stream);
}

int fp8q_gemm_blockscaled_ws(const uint8_t* a, int64_t lda, const void* sa, int sa_fmt, int64_t sa_sm,
                             int64_t sa_sk, const uint8_t* b, int64_t ldb, const void* sb, int sb_fmt,
                             int64_t sb_sn, int64_t sb_sk, uint16_t* y, int64_t ldy, int64_t M, int64_t N,
                             int64_t K, int mode, void* workspace, int64_t workspace_bytes, void* stream) {
  using namespace fp8q;
  const std::string pre = "fp8q_gemm_blockscaled_ws: ";
  if (workspace_bytes < 0) {
    set_error("");
    return fail(FP8Q_EINVAL, pre + "negative workspace size");
  }
  if (workspace && !aligned(workspace, 16)) {
    set_error("");
    return fail(FP8Q_EALIGN, pre + "workspace must be 16-byte aligned");
  }
  return dense_entry(pre, a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, y, ldy, M, N, K, mode,
                     static_cast<float*>(workspace), workspace ? workspace_bytes : 0, stream);
}

int fp8q_gemm_blockscaled_noalloc(const uint8_t* a, int64_t lda, const void* sa, int sa_fmt, int64_t sa_sm,
                                  int64_t sa_sk, const uint8_t* b, int64_t ldb, const void* sb, int sb_fmt,
                                  int64_t sb_sn, int64_t sb_sk, uint16_t* y, int64_t ldy, int64_t M, int64_t N,
                                  int64_t K, int mode, void* stream) {
  using namespace fp8q;
  const std::string pre = "fp8q_gemm_blockscaled_noalloc: ";
  set_error("");
  int rc = check_operands(pre, a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, y, ldy, M,
                          N, K, mode);
  if (rc != FP8Q_OK || M == 0 || N == 0 || K == 0) return rc;
  rc = check_current_device();
  if (rc != FP8Q_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(pre, &ws);
  if (rc != FP8Q_OK) return rc;
  const int64_t need = mode == FP8Q_GEMM_BLOCK128 ? gemm_workspace_bytes(M, N, K) : 0;
  if (need > FP8Q_NOALLOC_SCRATCH_BYTES)
    return fail(FP8Q_EUNSUPPORTED, pre + "this shape needs " + std::to_string(need) +
                                       " bytes of scratch, more than the library's " +
                                       std::to_string(FP8Q_NOALLOC_SCRATCH_BYTES));
  return dense_entry(pre, a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, y, ldy, M, N, K, mode,
                     static_cast<float*>(ws), FP8Q_NOALLOC_SCRATCH_BYTES, stream);
}

int64_t fp8q_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int mode) {
  using namespace fp8q;
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || mode != FP8Q_GEMM_BLOCK128) return 0;
  if (M == 0 || N == 0 || K == 0 || check_current_device() != FP8Q_OK) return 0;
  return gemm_workspace_bytes(M, N, K);
}

int fp8q_grouped_gemm_masked(const uint8_t* a, int64_t a_se, int64_t lda, const void* sa, int sa_fmt,
                             int64_t sa_se, int64_t sa_sm, int64_t sa_sk, const uint8_t* b, int64_t b_se,
                             int64_t ldb, const void* sb, int sb_fmt, int64_t sb_se, int64_t sb_sn,
                             int64_t sb_sk, uint16_t* y, int64_t y_se, int64_t ldy,
                             const int32_t* masked_m, int64_t expected_m, int64_t E, int64_t cap,
                             int64_t N, int64_t K, void* stream) {
  using namespace fp8q;
  set_error("");
  const std::string pre = "fp8q_grouped_gemm_masked: ";
  if (E < 0 || cap < 0) return fail(FP8Q_EINVAL, pre + "negative size");
  if (E > kMaxExperts) return fail(FP8Q_EUNSUPPORTED, pre + "at most 4096 experts");
  if (a_se < 0 || b_se < 0 || y_se < 0 || sa_se < 0 || sb_se < 0 || expected_m < 0)
    return fail(FP8Q_EINVAL, pre + "negative stride or expected_m");
  int rc = check_operands(pre, a, lda, sa, sa_fmt, sa_sm, sa_sk, b, ldb, sb, sb_fmt, sb_sn, sb_sk, y, ldy,
                          cap, N, K, FP8Q_GEMM_BLOCK128);
  if (rc != FP8Q_OK) return rc;
  if (E == 0 || cap == 0 || N == 0 || K == 0) return FP8Q_OK;
  if (!masked_m) return fail(FP8Q_EINVAL, pre + "masked_m is required");
  if (E > 1 && y_se < (cap - 1) * ldy + N) return fail(FP8Q_EINVAL, pre + "y experts overlap");
  if (!aligned(a, 16) || a_se % 16 != 0 || b_se % 16 != 0)
    return fail(FP8Q_EALIGN, pre + "expert strides of a and b must be multiples of 16 bytes");
  if (y_se % 2 != 0) return fail(FP8Q_EALIGN, pre + "expert stride of y must be even");
  const int64_t tiles = E * ((cap + 127) / 128) * ((N + 127) / 128);
  if (tiles >= (int64_t(1) << 31)) return fail(FP8Q_EUNSUPPORTED, pre + "too many output tiles");
  rc = check_current_device();
  if (rc != FP8Q_OK) return rc;
  GemmParams p{};
  p.a = a;
  p.sa = sa;
  p.b = b;
  p.sb = sb;
  p.y = y;
  p.masked_m = masked_m;
  p.M = cap;
  p.N = N;
  p.K = K;
  p.E = E;
  p.W = E;
  p.lda = lda;
  p.ldb = ldb;
  p.ldy = ldy;
  p.a_se = a_se;
  p.b_se = b_se;
  p.y_se = y_se;
  p.sa_sm = sa_sm;
  p.sa_sk = sa_sk;
  p.sa_se = sa_se;
  p.sb_sn = sb_sn;
  p.sb_sk = sb_sk;
  p.sb_se = sb_se;
  p.sa_packed = sa_fmt == FP8Q_SCALE_UE8M0_PACKED ? 1 : 0;
  p.sa_fmt = p.sa_packed ? FP8Q_SCALE_UE8M0 : sa_fmt;
  p.sb_fmt = sb_fmt;
  return launch_gemm_block128(p, expected_m, static_cast<hipStream_t>(stream));
}

int fp8q_grouped_gemm_segments(const uint8_t* a, int64_t lda, const void* sa, int sa_fmt, int64_t sa_sm,
                               int64_t sa_sk, const uint8_t* b, int64_t b_se, int64_t ldb, const void* sb,
                               int sb_fmt, int64_t sb_se, int64_t sb_sn, int64_t sb_sk, uint16_t* y, int64_t ldy,
                               const int32_t* seg_indptr, const int32_t* seg_weight, int64_t S, int64_t T,
                               int64_t W, int64_t N, int64_t K, int64_t expected_rows, void* stream) {
  if (seg_indptr == nullptr && S > 0 && T > 0 && N > 0 && K > 0 && W > 0) {
    fp8q::set_error("");
    return fp8q::fail(FP8Q_EINVAL, "fp8q_grouped_gemm_segments: seg_indptr is required");
  }
  return fp8q::grouped_rows_entry("fp8q_grouped_gemm_segments: ", a, lda, sa, sa_fmt, sa_sm, sa_sk, b, b_se, ldb, sb,
                            sb_fmt, sb_se, sb_sn, sb_sk, y, ldy, seg_indptr, seg_weight, nullptr, S, T, W, N, K,
                            expected_rows, stream);
}

int fp8q_grouped_gemm_contiguous(const uint8_t* a, int64_t lda, const void* sa, int sa_fmt, int64_t sa_sm,
                                 int64_t sa_sk, const uint8_t* b, int64_t b_se, int64_t ldb, const void* sb,
                                 int sb_fmt, int64_t sb_se, int64_t sb_sn, int64_t sb_sk, uint16_t* y, int64_t ldy,
                                 const int32_t* m_indices, int64_t T, int64_t W, int64_t N, int64_t K,
                                 void* stream) {
  if (m_indices == nullptr && T > 0 && N > 0 && K > 0 && W > 0) {
    fp8q::set_error("");
    return fp8q::fail(FP8Q_EINVAL, "fp8q_grouped_gemm_contiguous: m_indices is required");
  }
  return fp8q::grouped_rows_entry("fp8q_grouped_gemm_contiguous: ", a, lda, sa, sa_fmt, sa_sm, sa_sk, b, b_se, ldb, sb,
                            sb_fmt, sb_se, sb_sn, sb_sk, y, ldy, nullptr, nullptr, m_indices, 0, T, W, N, K, 0,
                            stream);
}

}  // extern "C"

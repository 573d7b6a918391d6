// fp8q_internal.h — internal declarations shared by the HIP translation units of libfp8q.
// Not part of the public ABI (that is include/fp8q.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "fp8q.h"
#include "tile_order.h"

namespace fp8q {

// ------------------------------------------------------------------ host-side status
void set_error(const std::string& msg);  // thread-local detail for fp8q_last_error()
int fail(int status, const std::string& msg);

// Validates the current device once per device (gfx950 only).
int check_current_device();

// Compute units and XCDs of the current device, as queried by check_current_device (which
// must have returned FP8Q_OK on this device first).
struct DeviceShape {
  int cus;
  int xcds;
};
DeviceShape current_device_shape();

// ------------------------------------------------------------------ quant launcher
struct QuantParams {
  const void* x;
  uint8_t* q;
  void* s;
  const int32_t* masked_m;  // device, or nullptr (flat)
  int64_t E, M, K;          // K = quantized width
  int64_t x_se, x_sm;       // input strides (elements)
  int64_t q_se, q_sm;       // output strides (bytes)
  int64_t s_se, s_sm, s_sg; // scale strides (scale elements; packed UE8M0: 32-bit words of 4 groups)
  int32_t packed;           // UE8M0 exponents packed 4 per word (group g in byte g % 4 of word g / 4)
  int64_t nseg;             // segments per row
  int32_t chunks_per_seg;   // 1024-element chunks per segment
  int32_t chunks_per_row;   // ceil(K / 1024)
};

// group_size 32, 64 or 128, or K (per-token: one group per row); i8 = int8 output
int launch_group_quant(int in_dtype, int scale_fmt, int group_size, bool silu, bool i8,
                       QuantParams p, int64_t expected_m, hipStream_t stream);

// ------------------------------------------------------------------ GEMM launchers
struct GemmParams {
  const uint8_t* a;
  const void* sa;
  const uint8_t* b;
  const void* sb;
  uint16_t* y;
  const int32_t* masked_m;  // grouped masked only
  const int32_t* seg_indptr;  // segments only: device int32[E + 1] row ranges of the packed rows
  const int32_t* seg_weight;  // segments only: device int32[E] weight of each segment (or nullptr)
  const int32_t* m_indices;   // grouped contiguous only: device int32[M] weight of each row, -1 = none
  int64_t M, N, K;          // M = capacity per expert (masked) or packed rows (segments, contiguous)
  int64_t E;                // experts (masked), segments, or 1
  int64_t W;                // weights that B and sb hold (weight indices outside [0, W) are skipped)
  int64_t lda, ldb, ldy;
  int64_t a_se, b_se, y_se;
  int64_t sa_sm, sa_sk, sa_se;
  int64_t sb_sn, sb_sk, sb_se;
  int sa_fmt, sb_fmt;
  int sa_packed;  // UE8M0 activation scales packed 4 K blocks per 32-bit word (sa strides in words)
  int sb_packed;  // MX32 only: E8M0 weight scales packed likewise (sb strides in words)
  int xcds;       // XCDs of the device (workgroup b runs on XCD b % xcds)
  float* ws;          // dense BLOCK128 only: fp32 workspace of the split-K small-M path, or nullptr
  int64_t ws_bytes;   // its size
};

int launch_gemm_block128(const GemmParams& p, int64_t expected_m, hipStream_t stream);
// Bytes of workspace with which a dense BLOCK128 GEMM of this shape takes the split-K path on
// the current device (0: it needs none).
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int launch_gemm_mx32(const GemmParams& p, hipStream_t stream);

}  // namespace fp8q

// bench_kernels.hip — reference data-movement kernels for the benchmark's ceilings
// (libfp8q_bench.so, loaded only by bench.py; not part of the fp8q boundary).
//
// They move the same bytes as the kernels they are compared with and do no arithmetic:
//   fp8q_bench_copy    n bf16 values in, n bytes out (the high byte of each): the traffic of
//                      group quantization without its scales; each lane moves two 16-byte
//                      loads and one 16-byte store per item, as the quant kernel does.
//   fp8q_bench_stream  reads `bytes` once (one contiguous slice per workgroup, every load of
//                      a batch issued before any is used) and writes one word per workgroup:
//                      the weight traffic of the small-M GEMM, which is bound by reading B.
//   fp8q_bench_mfma    the large GEMM's per-step instruction mix with its operands already in
//                      registers: per step each wave runs the 8 x 4 scaled 16x16x128 FP8 MFMAs
//                      of a 128x64 wave tile on real e4m3 codes, and (fold = 1) folds each
//                      product into fp32 accumulators with one fma per value, as the BLOCK128
//                      kernels do, or (fold = 0) accumulates in the matrix core, as MXFP8
//                      does. Eight waves per workgroup (two per SIMD), like the GEMM.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_hi_bytes(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                                                     int64_t items) {
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; t < items;
       t += static_cast<int64_t>(gridDim.x) * 256) {
    const u32x4 a = reinterpret_cast<const u32x4*>(x)[2 * t];
    const u32x4 b = reinterpret_cast<const u32x4*>(x)[2 * t + 1];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t lo = j < 2 ? a[2 * j] : b[2 * (j - 2)];
      const uint32_t hi = j < 2 ? a[2 * j + 1] : b[2 * (j - 2) + 1];
      o[j] = ((lo >> 8) & 0xFFu) | ((lo >> 24) << 8) | (((hi >> 8) & 0xFFu) << 16) | ((hi >> 24) << 24);
    }
    reinterpret_cast<u32x4*>(q)[t] = o;
  }
}

constexpr int kBatch = 32;  // 16-byte loads per lane in flight (128 KB per workgroup)

__global__ __launch_bounds__(256) void stream_read(const uint8_t* __restrict__ w, int64_t bytes, int64_t slice,
                                                   uint32_t* __restrict__ out) {
  const int64_t beg = static_cast<int64_t>(blockIdx.x) * slice;
  const int64_t end = beg + slice < bytes ? beg + slice : bytes;
  uint32_t acc = 0;
  for (int64_t base = beg; base < end; base += 256 * 16 * kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; i++) {
      const int64_t off = base + (static_cast<int64_t>(i) * 256 + threadIdx.x) * 16;
      v[i] = off < end ? *reinterpret_cast<const u32x4*>(w + off) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kBatch; i++) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  }
  // one word per lane, so the loads cannot be dropped
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

template <bool FOLD>
__global__ __launch_bounds__(512, 1) void mfma_mix(const v8i_t* __restrict__ codes, int iters,
                                                   float* __restrict__ out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 512 + threadIdx.x;
  v8i_t a[2], b[4];  // operand fragments of this lane (6 x 32 bytes of codes)
#pragma unroll
  for (int i = 0; i < 2; i++) a[i] = codes[t * 6 + i];
#pragma unroll
  for (int j = 0; j < 4; j++) b[j] = codes[t * 6 + 2 + j];
  const float s = 1.0f + static_cast<float>(threadIdx.x & 7) * 0x1p-10f;  // a fold factor per lane
  v4f_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v4f_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; it++) {
    // the operands are opaque to the compiler from step to step, so no product is hoisted
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
#pragma unroll
    for (int i = 0; i < 8; i++) {
      // (opaque per row too: rows sharing a fragment must not share their products)
      asm volatile("" : "+v"(a[i & 1]));
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if constexpr (FOLD) {
          const v4f_t z = {0.f, 0.f, 0.f, 0.f};
          const v4f_t pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i & 1], z, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int r = 0; r < 4; r++) acc[i][j][r] = fmaf(pr[r], s, acc[i][j][r]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i & 1], acc[i][j], 0, 0, 0, 127, 0, 127);
        }
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) sum += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  out[t] = sum;  // one word per lane, so no MFMA can be dropped
}

}  // namespace

extern "C" {

// n % 16 == 0, x and q 16-byte aligned. Returns 0 or a HIP error code.
int fp8q_bench_copy(const void* x, void* q, int64_t n, int grid, void* stream) {
  if (n % 16 != 0 || grid < 1) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(copy_hi_bytes, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), n / 16);
  return static_cast<int>(hipGetLastError());
}

// bytes % 16 == 0, w 16-byte aligned, out holds grid * 256 words. Each workgroup reads a
// slice of ceil(bytes / grid) bytes rounded up to 16.
int fp8q_bench_stream(const void* w, int64_t bytes, void* out, int grid, void* stream) {
  if (bytes % 16 != 0 || grid < 1) return static_cast<int>(hipErrorInvalidValue);
  const int64_t slice = ((bytes + grid - 1) / grid + 15) / 16 * 16;
  hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(w), bytes, slice, static_cast<uint32_t*>(out));
  return static_cast<int>(hipGetLastError());
}

// codes holds grid * 512 * 192 bytes of e4m3 codes (16-byte aligned), out grid * 512 floats.
// Each lane runs iters steps of 32 MFMAs (2 * 16 * 16 * 128 flops each). Returns 0 or a HIP
// error code.
int fp8q_bench_mfma(const void* codes, int iters, int fold, void* out, int grid, void* stream) {
  if (iters < 1 || grid < 1) return static_cast<int>(hipErrorInvalidValue);
  if (fold)
    hipLaunchKernelGGL(mfma_mix<true>, dim3(grid), dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v8i_t*>(codes), iters, static_cast<float*>(out));
  else
    hipLaunchKernelGGL(mfma_mix<false>, dim3(grid), dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v8i_t*>(codes), iters, static_cast<float*>(out));
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"

/*
 * fp8q.h — C ABI of libfp8q.so: per-token-group FP8 quantization of activations
 * and the block-scaled FP8 GEMMs that consume it, for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute is defined by these sources:
 *   [PR30924]  prhub report of sglang PR #30924, "[JIT] Trait-driven
 *              per_token_group_quant: unify the quant kernel family (flat + masked)":
 *              section "实现拆解" items 1-2 (the trait axes: input/output dtype, group
 *              size, fp32 or UE8M0 scale, row- or column-major scale layout, fused
 *              silu_and_mul, flat or masked dispatch with masked_m / expected_m) and
 *              section "关键源码片段" (the _jit_module trait list and the UE8M0 test
 *              reference ref_fp8_ue8m0).
 *   [TF]       TeleFuser page "tf-kernel 安装与使用": the per-token FP8 example, where
 *              the caller pre-allocates the e4m3 output and the fp32 scale tensor; and
 *              the silu_and_mul example, where the last dimension splits into two halves.
 *   [FI]       "FlashInfer GEMM 学习笔记": section 6 (block-scaled FP8 / MXFP8 with
 *              block size 32, 2D non-swizzled scales) and section 7 (DeepGEMM's grouped
 *              masked FP8 "NT" groupwise GEMM driven by expected_m + masked_m).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or synchronises; it only validates arguments and enqueues kernels.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call is
 *     asynchronous on that stream.
 *   - Sizes and strides are signed 64-bit and counted in ELEMENTS of the tensor they
 *     describe (bytes for e4m3/UE8M0 tensors). The innermost (K) dimension of x, q, a
 *     and b is always contiguous.
 *   - e4m3 tensors are passed as uint8_t bytes in the OCP E4M3FN encoding (bias 7,
 *     no infinities, 0x7F/0xFF are NaN, largest finite 448 = 0x7E).
 *   - UE8M0 scale bytes encode 2^(byte-127); 0xFF is never produced.
 *   - Return value: FP8Q_OK (0) or one of the positive status codes below. On error
 *     nothing is enqueued and no output byte is written. fp8q_last_error() returns a
 *     thread-local description of the last failure on the calling thread.
 *   - A call with a zero-sized problem (E, M, N or K equal to 0) returns FP8Q_OK and
 *     enqueues nothing.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified (but in-bounds) output.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FP8Q_OK 0
#define FP8Q_EINVAL 1       /* null pointer with non-zero size, bad shape, stride or layout */
#define FP8Q_EUNSUPPORTED 2 /* dtype, group size, scale format or mode outside the supported set */
#define FP8Q_EALIGN 3       /* pointer or row stride not aligned as required */
#define FP8Q_EDEVICE 4      /* current device is not gfx950, or no device */
#define FP8Q_ELAUNCH 5      /* the HIP runtime reported an error at launch */

/* activation dtypes (input of the quant calls) */
#define FP8Q_DTYPE_BF16 0
#define FP8Q_DTYPE_F16 1
#define FP8Q_DTYPE_F32 2

/* scale formats */
#define FP8Q_SCALE_F32 0   /* one IEEE float per group: s = amax / 448 */
#define FP8Q_SCALE_UE8M0 1 /* one byte per group: s = 2^(byte-127), the smallest power of two >= amax/448 */
#define FP8Q_SCALE_UE8M0_PACKED 2 /* the same bytes, 4 groups per 32-bit word: group g is byte g % 4 (least
                                     significant first) of word g / 4; strides count words [PR30924 item 1,
                                     the `aligned` trait: number of groups a multiple of 4, UE8M0 only] */

/* GEMM scaling modes */
#define FP8Q_GEMM_BLOCK128 0 /* a: 1x128 scales per (row, K block); b: 128x128 scales per (N block, K block) */
#define FP8Q_GEMM_MX32 1     /* a and b: one E8M0 byte per (row, 32-wide K block), applied by scaled MFMA */

/*
 * fp8q_group_quant — per-token-group FP8 (e4m3fn) quantization  [PR30924 items 1-2, ref_fp8_ue8m0]
 *
 * x is viewed as [E][M][K] (flat calls use E = 1): element (e, m, k) is at
 * x + e*x_se + m*x_sm + k, with dtype `in_dtype`. Each row is cut into K/G groups of
 * G = group_size consecutive elements. For every group of every processed row:
 *   amax = max(max |x_i|, 1e-10f)                                  (fp32)
 *   FP8Q_SCALE_F32:   s = amax / 448 (IEEE fp32 division), stored as float;
 *                     multiplier inv = 1 / s (IEEE fp32 division)
 *   FP8Q_SCALE_UE8M0: r = amax / 448 (fp32); byte = biased_exponent(r) + (mantissa(r) != 0),
 *                     stored as uint8; multiplier inv = 2^(127 - (byte - 127)), exact
 *   q_i = e4m3_round_nearest_even( clamp(x_i * inv, -448, 448) )
 * q (uint8 e4m3 bytes) element (e, m, k) is at q + e*q_se + m*q_sm + k.
 * The scale of group g of row (e, m) is at s + e*s_se + m*s_sm + g*s_sg, counted in
 * scale elements (4-byte floats or single bytes). The layout is read from the strides:
 * s_sg == 1 means row-major [M][K/G], s_sm == 1 means column-major [K/G][M]; any other
 * combination is FP8Q_EINVAL.
 * FP8Q_SCALE_UE8M0_PACKED stores the same UE8M0 bytes 4 groups to a 32-bit word: byte
 * g % 4 of word (e, m, g / 4), which is at s + 4 * (e*s_se + m*s_sm + (g/4)*s_sg) bytes
 * (strides in words; row-major [M][K/G/4] or column-major [K/G/4][M] words as above).
 *
 * Dispatch:
 *   masked_m == NULL: flat — every row m < M of every e < E is processed.
 *   masked_m != NULL: masked (the EP-MoE layout) — masked_m is a DEVICE int32[E];
 *     expert e processes rows m < clamp(masked_m[e], 0, M) only. Rows at or beyond
 *     that bound are never read or written (q and s keep their previous contents).
 *     expected_m >= 0 is a host-side hint of the typical rows per expert used to size
 *     the launch; it never changes the result (0 = no hint).
 *
 * Per-token quantization [TF per-token FP8 example: scale [M, 1]]: group_size == K
 * makes the whole row one group (one scale per row, at s + e*s_se + m*s_sm; s_sg is
 * not used). It requires K % 16 == 0 and K <= 2^30.
 *
 * Requirements (else the status in brackets):
 *   in_dtype in {BF16, F16, F32}; group_size in {32, 64, 128} or == K   [EUNSUPPORTED]
 *   K % group_size == 0, E, M, K >= 0, strides non-negative             [EINVAL]
 *   x and q 16-byte aligned; x_sm, x_se (in bytes) and q_sm, q_se
 *   multiples of 16 bytes; F32 scales and packed words 4-byte aligned   [EALIGN]
 *   UE8M0_PACKED: (K / group_size) % 4 == 0                              [EINVAL]
 *   E <= 4096 when masked                                                [EUNSUPPORTED]
 */
int fp8q_group_quant(const void* x, int in_dtype, int64_t E, int64_t M, int64_t K,
                     int64_t x_se, int64_t x_sm,
                     uint8_t* q, int64_t q_se, int64_t q_sm,
                     void* s, int scale_fmt, int64_t s_se, int64_t s_sm, int64_t s_sg,
                     int group_size, const int32_t* masked_m, int64_t expected_m,
                     void* stream);

/*
 * fp8q_silu_mul_group_quant — fused silu_and_mul followed by group quantization
 * [PR30924 item 1 (fuse_silu_and_mul trait), item 4 (silu_and_mul_masked_post_quant_fwd);
 *  TF silu_and_mul example (last dimension split in two halves)]
 *
 * Same arguments and outputs as fp8q_group_quant, except that x is [E][M][2K]: the
 * gate is columns [0, K) and the up projection is columns [K, 2K) of each row, and
 * the value that is quantized is, in fp32,
 *   y_j = ( g_j / (1 + exp(-g_j)) ) * u_j
 * where exp is the fixed fp32 sequence below (so that every conforming implementation
 * produces the same bits), not a vendor math library:
 *   t = clamp(-g, -87, 88); n = rint(t * log2(e)); r = fma(-n, ln2_hi, t); r = fma(-n, ln2_lo, r);
 *   p = Horner of sum_{k=0..7} r^k / k! with fma; exp = p * 2^n (2^n built from its bits).
 * All constants are the fp32 values nearest to log2(e), ln 2 (hi part) and its remainder,
 * and 1/k!. y is not rounded to a narrower type before quantization.
 */
int fp8q_silu_mul_group_quant(const void* x, int in_dtype, int64_t E, int64_t M, int64_t K,
                              int64_t x_se, int64_t x_sm,
                              uint8_t* q, int64_t q_se, int64_t q_sm,
                              void* s, int scale_fmt, int64_t s_se, int64_t s_sm, int64_t s_sg,
                              int group_size, const int32_t* masked_m, int64_t expected_m,
                              void* stream);

/*
 * fp8q_group_quant_int8 — per-token-group quantization to int8
 * [PR30924 关键文件 (the ref_int8 reference; out_dtype int8 among the trait axes),
 *  风险与影响 (int8 codes move by one under approximate division, so the division here is
 *  IEEE)]
 *
 * Same arguments, layouts, dispatch and requirements as fp8q_group_quant (group_size
 * 32, 64, 128 or K), with int8 codes in q and fp32 scales only. For every group:
 *   amax = max(max |x_i|, 1e-10f)                                  (fp32)
 *   s = amax / 127 (IEEE fp32 division), stored as float; inv = 1 / s (IEEE fp32 division)
 *   q_i = round_to_nearest_even( clamp(x_i * inv, -127, 127) ), a two's-complement byte
 * scale_fmt other than FP8Q_SCALE_F32 is FP8Q_EUNSUPPORTED. No fused silu variant.
 */
int fp8q_group_quant_int8(const void* x, int in_dtype, int64_t E, int64_t M, int64_t K,
                          int64_t x_se, int64_t x_sm,
                          int8_t* q, int64_t q_se, int64_t q_sm,
                          float* s, int scale_fmt, int64_t s_se, int64_t s_sm, int64_t s_sg,
                          int group_size, const int32_t* masked_m, int64_t expected_m,
                          void* stream);

/*
 * fp8q_gemm_blockscaled — Y = dequant(A) * dequant(B)^T, bf16 output  [FI sections 6-7]
 *
 * A is [M][K] e4m3 (row m at a + m*lda), B is [N][K] e4m3 (row n at b + n*ldb): both
 * operands are K-major ("NT"). Y is [M][N] bf16 (element (m, n) at y + m*ldy + n, passed
 * as uint16_t bits).
 *   mode FP8Q_GEMM_BLOCK128:
 *     sa: one scale per (m, kb), kb = k/128, at sa + m*sa_sm + kb*sa_sk; sa_fmt F32 or UE8M0;
 *         or UE8M0_PACKED: byte kb % 4 of the 32-bit word at sa + 4*(m*sa_sm + (kb/4)*sa_sk)
 *         bytes (strides in words; K % 512 == 0 [EINVAL]; sa 4-byte aligned [EALIGN]).
 *     sb: one scale per (nb, kb), nb = n/128, at sb + nb*sb_sn + kb*sb_sk; sb_fmt F32 or UE8M0.
 *     Y[m][n] = bf16_rne( sum_kb sa(m,kb) * sb(n/128,kb) * sum_{k in kb} dec(A[m][k]) * dec(B[n][k]) )
 *   mode FP8Q_GEMM_MX32:
 *     sa: one E8M0 byte per (m, k/32) at sa + m*sa_sm + (k/32)*sa_sk; sb likewise per (n, k/32)
 *     (sa_fmt, sb_fmt = FP8Q_SCALE_UE8M0: the 2D non-swizzled layout of [FI] section 6).
 *     Either operand may instead use FP8Q_SCALE_UE8M0_PACKED: the four bytes of K blocks
 *     4j..4j+3 (one 128-wide K step) of a row in one 32-bit word, byte k/32 % 4 of the word
 *     at s + 4*(row*s_sm + (k/128)*s_sk) bytes (strides in words, s 4-byte aligned [EALIGN]).
 *     Column-major words (s_sm == 1, s_sk >= rows) are the layout this library reads
 *     fastest: one K step's scales of consecutive rows are contiguous. The activation
 *     layout is what fp8q_group_quant writes for group_size 32 with UE8M0_PACKED scales
 *     in column-major words.
 *     Y[m][n] = bf16_rne( sum_k 2^(sa-127) dec(A[m][k]) * 2^(sb-127) dec(B[n][k]) )
 * Accumulation is fp32; the result is rounded to bf16 once, at the end.
 *
 * Requirements: M, N, K >= 0, K % 128 == 0 [EINVAL]; a, b 16-byte aligned with lda, ldb
 * multiples of 16; y 4-byte aligned with ldy even [EALIGN]; lda, ldb >= K, ldy >= N [EINVAL].
 */
int fp8q_gemm_blockscaled(const uint8_t* a, int64_t lda,
                          const void* sa, int sa_fmt, int64_t sa_sm, int64_t sa_sk,
                          const uint8_t* b, int64_t ldb,
                          const void* sb, int sb_fmt, int64_t sb_sn, int64_t sb_sk,
                          uint16_t* y, int64_t ldy,
                          int64_t M, int64_t N, int64_t K, int mode, void* stream);

/*
 * fp8q_gemm_workspace_size / fp8q_gemm_blockscaled_ws — the dense call with a workspace
 * [FI sections 6-7, as fp8q_gemm_blockscaled]
 *
 * Same operation, arguments and requirements as fp8q_gemm_blockscaled, plus a caller-owned
 * device workspace. fp8q_gemm_workspace_size returns the bytes of workspace with which a
 * BLOCK128 problem of this shape takes the split-K path on the current device (today:
 * 16 < M <= 128, when the K blocks split into several ranges; their fp32 partial sums are
 * added in a fixed order by a second kernel), or 0 when the call needs none; it returns 0 for
 * MX32 and for arguments the GEMM would reject. With workspace_bytes at least that size the
 * call takes the split-K path; with a smaller or NULL workspace it runs exactly as
 * fp8q_gemm_blockscaled. Results of the two paths may differ in the last bits (summation
 * order) and both meet the accuracy of fp8q_gemm_blockscaled; each path is deterministic.
 * The workspace must be 16-byte aligned [EALIGN]; workspace_bytes < 0 is EINVAL. The
 * library writes only the first fp8q_gemm_workspace_size bytes; concurrent calls must not
 * share a workspace.
 */
int64_t fp8q_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int mode);

int fp8q_gemm_blockscaled_ws(const uint8_t* a, int64_t lda,
                             const void* sa, int sa_fmt, int64_t sa_sm, int64_t sa_sk,
                             const uint8_t* b, int64_t ldb,
                             const void* sb, int sb_fmt, int64_t sb_sn, int64_t sb_sk,
                             uint16_t* y, int64_t ldy,
                             int64_t M, int64_t N, int64_t K, int mode,
                             void* workspace, int64_t workspace_bytes, void* stream);

/*
 * fp8q_gemm_blockscaled_noalloc — for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc)
 *
 * Same arguments, requirements and results as fp8q_gemm_blockscaled_ws given a workspace of
 * fp8q_gemm_workspace_size bytes, but the workspace is a device array of the library,
 * FP8Q_NOALLOC_SCRATCH_BYTES (32 MiB) per device, instead of the caller's. The call allocates
 * nothing and calls no allocating routine: each device holds its own array from when the
 * library's code is loaded on it until the process ends, and the array's device address is
 * looked up on the first call on each device (a failed lookup is FP8Q_EDEVICE). A shape whose
 * workspace size exceeds FP8Q_NOALLOC_SCRATCH_BYTES is FP8Q_EUNSUPPORTED, before anything is
 * launched or written. All calls on one device share the array, which keeps the last call's
 * contents (nothing in it has to start at zero): calls that overlap in time on one device
 * (several streams or host threads) race on it, so the caller must order them.
 */
#define FP8Q_NOALLOC_SCRATCH_BYTES (32 << 20)

int fp8q_gemm_blockscaled_noalloc(const uint8_t* a, int64_t lda,
                                  const void* sa, int sa_fmt, int64_t sa_sm, int64_t sa_sk,
                                  const uint8_t* b, int64_t ldb,
                                  const void* sb, int sb_fmt, int64_t sb_sn, int64_t sb_sk,
                                  uint16_t* y, int64_t ldy,
                                  int64_t M, int64_t N, int64_t K, int mode, void* stream);

/*
 * fp8q_grouped_gemm_masked — per-expert BLOCK128 GEMM over the masked EP-MoE layout
 * [FI section 7: DeepGEMM grouped masked, expected_m + masked_m; PR30924 item 2]
 *
 * For every expert e < E: A_e = a + e*a_se ([cap][K], row stride lda),
 * sa_e = sa + e*sa_se (indexed like fp8q_gemm_blockscaled's sa), B_e = b + e*b_se
 * ([N][K], row stride ldb), sb_e = sb + e*sb_se, Y_e = y + e*y_se ([cap][N], row
 * stride ldy). Rows m < clamp(masked_m[e], 0, cap) of Y_e receive the BLOCK128 product
 * of A_e and B_e; rows at or beyond that bound are never written. masked_m is a
 * DEVICE int32[E]; expected_m is a host-side launch hint only (result-invariant).
 * Requirements as for fp8q_gemm_blockscaled, plus E <= 4096 [EUNSUPPORTED].
 */
int fp8q_grouped_gemm_masked(const uint8_t* a, int64_t a_se, int64_t lda,
                             const void* sa, int sa_fmt, int64_t sa_se, int64_t sa_sm, int64_t sa_sk,
                             const uint8_t* b, int64_t b_se, int64_t ldb,
                             const void* sb, int sb_fmt, int64_t sb_se, int64_t sb_sn, int64_t sb_sk,
                             uint16_t* y, int64_t y_se, int64_t ldy,
                             const int32_t* masked_m, int64_t expected_m,
                             int64_t E, int64_t cap, int64_t N, int64_t K, void* stream);

/*
 * fp8q_grouped_gemm_segments — BLOCK128 GEMM over ragged segments of packed rows
 * [FI section 7: SegmentGEMM, x[sum(seg_lens), d_in] with weights[num_weights, d_out, d_in]
 *  mapped through seg_indptr; Group GEMM for MoE experts with different token counts]
 *
 * a is [T][K] e4m3 packed rows (row t at a + t*lda) with activation scales sa indexed as
 * in fp8q_gemm_blockscaled over the T rows; b holds W weights of [N][K] e4m3 (weight w at
 * b + w*b_se, row stride ldb) with 128x128 scales sb + w*sb_se (indexed as in
 * fp8q_gemm_blockscaled); y is [T][N] bf16 (row t at y + t*ldy).
 * seg_indptr is a DEVICE int32[S + 1]: segment s is rows [seg_indptr[s], seg_indptr[s+1])
 * (both ends clamped to [0, T], an end below its start meaning an empty segment).
 * seg_weight is a DEVICE int32[S] or NULL: segment s uses weight seg_weight[s] (NULL: weight
 * s); a segment whose weight index is outside [0, W) is skipped. Each row of a segment gets
 * Y[t] = BLOCK128 product of row t of A and its segment's weight; rows of y in no computed
 * segment are never written (rows in two segments get either). expected_rows is a host hint of
 * the rows in all segments, for the launch size only (0: T).
 * Requirements as for fp8q_gemm_blockscaled, plus S <= 2048, T < 2^31 [EUNSUPPORTED];
 * b_se a multiple of 16 [EALIGN], weights not overlapping [EINVAL].
 */
int fp8q_grouped_gemm_segments(const uint8_t* a, int64_t lda,
                               const void* sa, int sa_fmt, int64_t sa_sm, int64_t sa_sk,
                               const uint8_t* b, int64_t b_se, int64_t ldb,
                               const void* sb, int sb_fmt, int64_t sb_se, int64_t sb_sn, int64_t sb_sk,
                               uint16_t* y, int64_t ldy,
                               const int32_t* seg_indptr, const int32_t* seg_weight,
                               int64_t S, int64_t T, int64_t W, int64_t N, int64_t K,
                               int64_t expected_rows, void* stream);

/*
 * fp8q_grouped_gemm_contiguous — grouped GEMM over packed rows tagged with their expert
 * [FI section 7: DeepGEMM GroupedContiguous, packed tokens + m_indices]
 *
 * Operands as in fp8q_grouped_gemm_segments. m_indices is a DEVICE int32[T]: the weight of
 * each row, or -1 for a padding row. Rows are taken in aligned blocks of 128: a block whose
 * first row holds a weight index e in [0, W) computes, for each of its rows t with
 * m_indices[t] == e, Y[t] = BLOCK128 product of row t of A and weight e; every other row
 * (padding, or a row whose index differs from its block's first row) is never written.
 * (The layout this serves puts each expert's rows at a 128-aligned offset and pads them
 * with -1 to a multiple of 128.)
 * Activation scales: fp32 (any strides), UE8M0 column-major with T % 4 == 0, or
 * UE8M0_PACKED, with fp32 weight scales; or UE8M0 column-major (T % 4 == 0) or UE8M0_PACKED
 * activation scales with UE8M0 weight scales in row-major [N/128][K/128] rows of whole
 * 4-byte words (K % 512 == 0, sb_sn % 4 == 0, sb_se % 4 == 0, sb 4-byte aligned). UE8M0
 * activation scales stored row-major (sa_sk == 1) in rows of whole 4-byte words
 * (K % 512 == 0, sa_sm % 4 == 0, sa 4-byte aligned) count as UE8M0_PACKED words.
 * [EUNSUPPORTED otherwise]. Other requirements as above.
 */
int fp8q_grouped_gemm_contiguous(const uint8_t* a, int64_t lda,
                                 const void* sa, int sa_fmt, int64_t sa_sm, int64_t sa_sk,
                                 const uint8_t* b, int64_t b_se, int64_t ldb,
                                 const void* sb, int sb_fmt, int64_t sb_se, int64_t sb_sn, int64_t sb_sk,
                                 uint16_t* y, int64_t ldy, const int32_t* m_indices,
                                 int64_t T, int64_t W, int64_t N, int64_t K, void* stream);

/* Human-readable name of a status code. Never returns NULL. */
const char* fp8q_status_string(int status);

/* Description of the last failure on this thread ("" if none). Never returns NULL. */
const char* fp8q_last_error(void);

/*
 * fp8q_device_check — FP8Q_OK if HIP device `device` exists and is a gfx950 (CDNA4)
 * part, else FP8Q_EDEVICE. The compute calls perform the same check on the current
 * device the first time they see it.
 */
int fp8q_device_check(int device);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */

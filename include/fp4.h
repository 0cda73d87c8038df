/*
 * fp4.h -- block-scaled 4-bit floating point (NVFP4 / MXFP4) on AMD MI355X.
 *
 * C ABI of libfp4.so.  Every entry point enqueues its work on `stream` (a
 * hipStream_t passed as void*; NULL is the default stream) and returns
 * without synchronizing.  All tensor pointers are DEVICE memory owned by the
 * caller; the library allocates nothing and keeps no state between calls, so
 * the calls are reentrant and may be issued from several host threads.
 *
 * Error behaviour: every argument is validated on the host before any HIP
 * call; on a validation error nothing is enqueued and no output is touched.
 * A failed launch returns FP4_EHIP (the HIP error is read and cleared).
 * Faults inside a kernel surface at the caller's next synchronization, as for
 * any kernel.  Nothing falls back to another algorithm: a combination the
 * library does not implement returns FP4_EUNSUPPORTED.
 *
 * Formats (aisyndicate.ch "FP4 auf Blackwell: Was NVFP4 fuer lokale KI
 * wirklich aendert", section "Was NVFP4 von frueheren 4-Bit-Formaten
 * unterscheidet"; pimento.cloud "FP8, NVFP4 czy AWQ?", section "Czym roznia
 * sie FP8, NVFP4, MXFP4 i AWQ?"):
 *   element  E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit;
 *            magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *   NVFP4    blocks of 16 elements, one E4M3 scale byte per block (bias 7,
 *            max 448) and one FP32 scale per tensor.
 *   MXFP4    blocks of 32 elements, one E8M0 scale byte per block (2^(c-127)).
 *
 * Layouts (canonical at this boundary):
 *   values   row-major [rows, k], contiguous; blocks run along k, so k must be
 *            a multiple of the block size (16 or 32).
 *   codes    uint8 [rows, k/2]: byte j of a row holds element 2j in its low
 *            nibble and element 2j+1 in its high nibble.
 *   scales   uint8 [rows, k/block], row-major, one byte per block.  The
 *            quantizers write NVFP4 bytes 0x00..0x7E and MXFP4 bytes
 *            0x00..0xFE; every call that reads scales accepts any byte:
 *            E4M3 with its sign bit (0x7F and 0xFF are NaN), E8M0 with
 *            0xFF NaN.  A NaN scale makes its block's values NaN (and the
 *            GEMM outputs they reach); FP8 output of a NaN is unspecified.
 *   tensor scale (NVFP4 only): one float in device memory.
 *
 * Rounding (the pages state none; these are the library's definitions):
 *   NVFP4 tensor scale s_t = fp32(max|x| / 2688) (2688 = 6 * 448), or 1 when
 *   that is 0.  Block scale = E4M3 nearest-even of fp32(a_b / fp32(6 s_t)),
 *   saturating at 448.  S_b = fp32(E4M3(sb) * s_t); elements are scaled by one
 *   multiply with r_b = fp32(1 / S_b) (a block with S_b == 0 or an infinite
 *   r_b keeps only sign bits) and rounded to E2M1 nearest-even with ties to
 *   the even code, saturating at 6; the sign of zero is kept.
 *   MXFP4 block scale = smallest 2^k with a_b <= 6 * 2^k ("rounded to the
 *   next power of two"), clamped to [2^-127, 2^127]; an all-zero block gets
 *   code 0.  Elements are x * 2^-k (exact) rounded as above.
 * Non-finite inputs are outside the contract (no fault, unspecified codes).
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4_NVFP4 = 0, /* 16-element blocks, E4M3 block scale + FP32 tensor scale */
  FP4_MXFP4 = 1  /* 32-element blocks, E8M0 block scale */
} fp4_format;

typedef enum {
  FP4_F32 = 0,  /* IEEE binary32 */
  FP4_BF16 = 1, /* bfloat16 */
  FP4_F16 = 2,  /* IEEE binary16 */
  FP4_E4M3 = 3  /* FP8 E4M3 (bias 7, max 448, no infinity) */
} fp4_dtype;

typedef enum {
  FP4_OK = 0,
  FP4_EINVAL = 1,       /* bad argument: null/misaligned pointer, bad size or enum */
  FP4_EUNSUPPORTED = 2, /* valid but not implemented combination */
  FP4_EHIP = 3          /* a HIP launch failed */
} fp4_status;

typedef enum {
  FP4_TSCALE_COMPUTE = 0, /* NVFP4: compute s_t from the data, write it to *tensor_scale */
  FP4_TSCALE_GIVEN = 1    /* NVFP4: read s_t from *tensor_scale (positive, finite) */
} fp4_tscale_mode;

/* Human-readable name of a status code (static string, never NULL). */
const char* fp4_status_string(fp4_status s);

/* Bytes of device workspace fp4_quantize / fp4_hadamard_quantize /
 * fp4_quantize_mse need for these arguments: nonzero only for NVFP4 in
 * FP4_TSCALE_COMPUTE mode (the per-workgroup partial maxima of the tensor
 * amax pass, read back by the quantizing pass). */
size_t fp4_quantize_workspace_size(fp4_format fmt, fp4_tscale_mode mode,
                                   int64_t rows, int64_t k);

/*
 * fp4_quantize -- block-scaled FP4 quantization of x [rows, k].
 * Defines: the NVFP4 / MXFP4 formats of the two pages cited above; the
 * "dynamic scaling" of the FP32 tensor scale (aisyndicate.ch, same section)
 * is FP4_TSCALE_COMPUTE.
 *   fmt           FP4_NVFP4 or FP4_MXFP4.
 *   x, x_dtype    input values, FP4_F32 / FP4_BF16 / FP4_F16; 16-byte aligned.
 *   rows, k       rows >= 0 (0 enqueues nothing), k > 0, k % block == 0,
 *                 rows * k < 2^40.
 *   codes         out, uint8 [rows, k/2]; 16-byte aligned.
 *   scales        out, uint8 [rows, k/block]; 4-byte aligned.
 *   tensor_scale  NVFP4: one device float, written (COMPUTE) or read (GIVEN);
 *                 MXFP4: must be NULL.
 *   mode          FP4_TSCALE_COMPUTE or FP4_TSCALE_GIVEN (ignored for MXFP4).
 *   workspace     device scratch of at least fp4_quantize_workspace_size()
 *                 bytes (may be NULL when that size is 0); 16-byte aligned.
 *                 Its contents on entry do not matter; calls that overlap
 *                 in time (other streams) must not share a workspace.
 * Returns FP4_OK, FP4_EINVAL or FP4_EHIP.
 */
fp4_status fp4_quantize(fp4_format fmt, const void* x, fp4_dtype x_dtype,
                        int64_t rows, int64_t k, uint8_t* codes,
                        uint8_t* scales, float* tensor_scale,
                        fp4_tscale_mode mode, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * fp4_quantize_noalloc -- fp4_quantize without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  It allocates
 * nothing (no hipMalloc / hipFree, no allocating library routine): the
 * partial maxima of FP4_TSCALE_COMPUTE mode go to a 4 KiB scratch array the
 * library holds in device memory, one copy per GPU, kept until the process
 * ends.  The max pass never needs more than that, whatever rows * k, so no
 * size is refused for lack of scratch (sizes are limited as in fp4_quantize);
 * nothing in the scratch has to start at zero.
 *   Arguments, results, alignment and errors as fp4_quantize (without
 *   workspace / workspace_bytes); FP4_EHIP also when the scratch cannot be
 *   located on the current device.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (several streams, several host threads) race and must
 *   be serialized by the caller.
 */
fp4_status fp4_quantize_noalloc(fp4_format fmt, const void* x, fp4_dtype x_dtype,
                                int64_t rows, int64_t k, uint8_t* codes,
                                uint8_t* scales, float* tensor_scale,
                                fp4_tscale_mode mode, void* stream);

/*
 * fp4_hadamard_quantize -- rotate each block of x by H_b / sqrt(b), then
 * quantize exactly as fp4_quantize does (the tensor amax of COMPUTE mode is
 * taken over the rotated values).
 * Defines: the blockwise Hadamard transform of MR-GPTQ, applied online to
 * activations and offline to weights (hyper.ai, paper 2509.23202, Abstract).
 *   b = block size (16 for NVFP4, 32 for MXFP4); H_b is the Sylvester
 *   Hadamard matrix, computed in fp32 as the butterfly stages h = 1, 2, ...,
 *   b/2, each pair (j, j+h) -> (y_j + y_{j+h}, y_j - y_{j+h}), then one
 *   multiply by fp32(1/sqrt(b)).  Because H_b H_b^T = b I, a rotated X times a
 *   rotated W^T equals X W^T.
 *   Arguments, alignment and errors as fp4_quantize.
 */
fp4_status fp4_hadamard_quantize(fp4_format fmt, const void* x,
                                 fp4_dtype x_dtype, int64_t rows, int64_t k,
                                 uint8_t* codes, uint8_t* scales,
                                 float* tensor_scale, fp4_tscale_mode mode,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * fp4_quantize_mse -- NVFP4 quantization whose block scale minimizes the
 * block's squared error.
 * Defines: the NVFP4 scaling of aisyndicate.ch "FP4 auf Blackwell", section
 * "Was NVFP4 von frueheren 4-Bit-Formaten unterscheidet" (the E4M3 block
 * scale is the factor with the least mean squared error over the block's 16
 * values, instead of a rounded power of two).
 *   Every positive finite E4M3 byte (1 .. 126) is tried as the block scale
 *   under the tensor scale s_t; each quantizes the block as fp4_quantize does
 *   for that byte (S_b = fp32(E4M3(sb) * s_t), q = x * fp32(1/S_b), E2M1
 *   round to nearest even); its error sum_i (x_i - v_i S_b)^2 is summed in
 *   fp64 in element order; the least error wins, ties going to the smaller
 *   byte.  A block of zeros keeps byte 0.  The output is ordinary NVFP4
 *   (fp4_dequantize and fp4_gemm take it as is).  About 10^4 fp64 operations
 *   per block: meant for weights quantized once.
 *   Arguments, alignment, workspace (fp4_quantize_workspace_size with
 *   FP4_NVFP4) and errors as fp4_quantize with fmt = FP4_NVFP4.
 */
fp4_status fp4_quantize_mse(const void* x, fp4_dtype x_dtype, int64_t rows,
                            int64_t k, uint8_t* codes, uint8_t* scales,
                            float* tensor_scale, fp4_tscale_mode mode,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * fp4_dequantize -- codes + scales -> values.
 * Defines: the inverse of the formats above; FP4_E4M3 output is the FP8 form
 * an NVFP4 KV cache is dequantized to before attention (hyper.ai story on the
 * NVFP4 KV cache).
 *   NVFP4: y = fp32(fp32(v * E4M3(sb)) * s_t) -- the exact product rounded
 *   once; MXFP4: y = v * 2^(c-127) (exact).  Then converted to out_dtype:
 *   FP4_F32 as is; FP4_BF16 / FP4_F16 round to nearest even; FP4_E4M3 round
 *   to nearest even, saturating to +-448 (never NaN).
 *   codes, scales   inputs, layouts above; 16- and 4-byte aligned.
 *   tensor_scale    NVFP4: one device float; MXFP4: must be NULL.
 *   rows, k         as fp4_quantize.
 *   out             [rows, k] of out_dtype; 16-byte aligned.
 * Returns FP4_OK, FP4_EINVAL or FP4_EHIP.
 */
fp4_status fp4_dequantize(fp4_format fmt, const uint8_t* codes,
                          const uint8_t* scales, const float* tensor_scale,
                          int64_t rows, int64_t k, void* out,
                          fp4_dtype out_dtype, void* stream);

/* Bytes of device workspace fp4_gemm needs for these sizes: nonzero only
 * where k is split over several workgroups per output tile (the slices'
 * fp32 partial sums, added in a fixed order by a second pass): large m with
 * few output tiles, which would leave most of the GPU idle, and a k of
 * more than one chunk with few activation rows (NVFP4, up to 64 rows: k a
 * multiple of 128 past 4096 values, or past 2048 where k is not a multiple
 * of 4096; MXFP4, up to 32 rows: k > 4096 a multiple of 2048).  Rows past
 * 16 go in groups of 16 that reuse one group's workspace. */
size_t fp4_gemm_workspace_size(fp4_format fmt, int64_t m, int64_t n, int64_t k);

/*
 * fp4_gemm -- W4A4 matrix multiply C = A B^T on quantized operands.
 * Defines: W4A4, both weights and activations 4-bit so the products run on
 * low-precision matrix units (pimento.cloud, section "Dlaczego W8A8 i W4A16
 * to nie to samo?").
 *   A = activations [m, k] (codes [m, k/2], scales [m, k/block], a_tscale);
 *   B = weights     [n, k] (codes [n, k/2], scales [n, k/block], b_tscale);
 *   both in the same format, blocks along k.  C[i, j] = sum over k of
 *   deq(A)[i, kk] * deq(B)[j, kk], accumulated in fp32: MXFP4 on the gfx950
 *   block-scaled MFMA (E8M0 scale per 32 values); NVFP4 by exact in-register
 *   products v * E4M3(sb) in fp16 on fp16 MFMA, times a_tscale * b_tscale at
 *   the end.
 *   c, c_dtype      out, row-major [m, n], FP4_F32 or FP4_BF16 (nearest even).
 *   a_tscale, b_tscale  NVFP4: device floats; MXFP4: must be NULL.
 *   workspace       at least fp4_gemm_workspace_size() bytes, 16-byte
 *                   aligned (may be NULL when that size is 0); its contents
 *                   on entry do not matter; calls that overlap must not
 *                   share one.
 *   m, n >= 0 (0 enqueues nothing), k > 0 with k % 32 == 0 (NVFP4 too).
 * Pointer alignment: codes 16 bytes, scales 4 bytes, c 16 bytes.
 * Returns FP4_OK, FP4_EINVAL, FP4_EUNSUPPORTED or FP4_EHIP.
 */
fp4_status fp4_gemm(fp4_format fmt, int64_t m, int64_t n, int64_t k,
                    const uint8_t* a_codes, const uint8_t* a_scales,
                    const float* a_tscale, const uint8_t* b_codes,
                    const uint8_t* b_scales, const float* b_tscale, void* c,
                    fp4_dtype c_dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * fp4_gemm_w4a16 -- C = X B^T with 16-bit activations and 4-bit weights.
 * Defines: W4A16, where only the weights are 4-bit and the products stay
 * 16-bit -- the form that speeds up token-by-token generation, whose
 * bottleneck is reading the weights (pimento.cloud "FP8, NVFP4 czy AWQ?",
 * section "Dlaczego W8A8 i W4A16 to nie to samo?").
 *   fmt           FP4_NVFP4 or FP4_MXFP4 (the weights' format).
 *   x, x_dtype    activations [m, k], FP4_BF16 / FP4_F16 / FP4_F32,
 *                 row-major, aligned to their element size.
 *   b_*           weights [n, k] as fp4_gemm's B; b_tscale NVFP4 only.
 *   c, c_dtype    out [m, n], FP4_F32 or FP4_BF16 (FP4_F16 / FP4_E4M3:
 *                 FP4_EUNSUPPORTED).
 *   workspace     at least fp4_gemm_w4a16_workspace_size() bytes, 16-byte
 *                 aligned (may be NULL when that size is 0); contents on
 *                 entry do not matter; calls that overlap must not share one.
 *   Numerics: the weights are widened exactly (v * E4M3 scale in fp16 or
 *   fp32, v * 2^e).  NVFP4 with bf16 or fp16 X, k a multiple of 128 from
 *   2048 on (at most 64 chunks of 2048 or 4096 values) and 16-byte aligned
 *   x / codes / scales takes the
 *   streaming path: each row of X is cut into pieces of 128 or 256 values,
 *   each piece scaled by the power of two that brings its max |x| into
 *   [1, 2) and rounded to fp16 (exact for every value above 2^-15 of that
 *   max), the products accumulate in fp32 on the matrix cores and each
 *   piece's partial sums are scaled back before they are added (for
 *   more than one chunk the sums of each chunk of 2048 or 4096 values go
 *   through the workspace).  MXFP4 with bf16 X and k a multiple of 2048
 *   takes the same path with the weights
 *   widened exactly to bf16 on the bf16 matrix cores.  Other shapes sum fp32
 *   products.  Tolerance against the float64 reference: relative Frobenius
 *   error <= 1e-3.
 *   m = 0 or n = 0 enqueues nothing.  Returns FP4_OK, FP4_EINVAL,
 *   FP4_EUNSUPPORTED or FP4_EHIP.
 */
fp4_status fp4_gemm_w4a16(fp4_format fmt, const void* x, fp4_dtype x_dtype,
                          int64_t m, int64_t n, int64_t k,
                          const uint8_t* b_codes, const uint8_t* b_scales,
                          const float* b_tscale, void* c, fp4_dtype c_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace fp4_gemm_w4a16 needs for these sizes: nonzero
 * only for a k of more than one chunk (NVFP4: a multiple of 128 past 4096
 * values, or past 2048 where k is not a multiple of 4096; MXFP4: k > 4096 a
 * multiple of 2048): the fp32 sums of each chunk of k for up to 16 rows of
 * X at a time. */
size_t fp4_gemm_w4a16_workspace_size(fp4_format fmt, int64_t m, int64_t n, int64_t k);

/* Bytes of device workspace fp4_quantize_gemm needs for these sizes. */
size_t fp4_quantize_gemm_workspace_size(fp4_format fmt, int64_t m, int64_t n,
                                        int64_t k);

/*
 * fp4_quantize_gemm -- quantize the activations and multiply: the result is
 * that of fp4_quantize(fmt, x, x_dtype, m, k, a_codes, a_scales, a_tscale,
 * FP4_TSCALE_COMPUTE, ...) followed by fp4_gemm(fmt, m, n, k, a_codes,
 * a_scales, a_tscale, b_codes, b_scales, b_tscale, c, c_dtype, ...), codes,
 * scales, tensor scale and C alike.
 * Defines: the decode step of a W4A4 layer -- activations quantized online
 * per call, the weights streamed once (cloudmagazin.com "FP8, FP4 und vLLM",
 * section "Rechnung": token-by-token decoding is bound by reading the
 * weights; hyper.ai, paper 2509.23202, Abstract: activations quantized
 * online).  With bf16 x and 1 <= m <= 16 the activation quantization
 * happens inside the GEMM's launch: NVFP4 for k = 2048 or 4096 and
 * n <= 16384 (every workgroup reducing max |x| over the whole tensor
 * itself), MXFP4 for k a multiple of 128 from 2048 on and any n (no
 * tensor-wide maximum; a k of more than one chunk -- past 4096 values, or
 * past 2048 where k is not a multiple of 4096 -- adds the reduction pass of
 * the split k).  Otherwise it runs as
 * the two calls.
 *   x            in, [m, k] of x_dtype, 16-byte aligned.
 *   a_codes, a_scales, a_tscale   out, as fp4_quantize (COMPUTE mode).
 *   b_*, c, c_dtype               as fp4_gemm.
 *   workspace    at least fp4_quantize_gemm_workspace_size() bytes, 16-byte
 *                aligned (may be NULL when that size is 0).
 * Every check of both calls runs before anything is enqueued.
 * Returns FP4_OK, FP4_EINVAL, FP4_EUNSUPPORTED or FP4_EHIP.
 */
fp4_status fp4_quantize_gemm(fp4_format fmt, const void* x, fp4_dtype x_dtype,
                             int64_t m, int64_t n, int64_t k, uint8_t* a_codes,
                             uint8_t* a_scales, float* a_tscale,
                             const uint8_t* b_codes, const uint8_t* b_scales,
                             const float* b_tscale, void* c, fp4_dtype c_dtype,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * fp4_kv_append -- write new K (or V) vectors into a 4-bit KV cache.
 * Defines: the write side of the hyper.ai story on the NVFP4 KV cache (new
 * K/V vectors go into the cache in NVFP4 form).
 *   x, x_dtype    new rows [batch, heads, t_new, k], FP4_F32 / FP4_BF16 /
 *                 FP4_F16, row-major, 16-byte aligned.
 *   positions     device int32 [batch]: row (b, h, i) is written at cache
 *                 position positions[b] + i; a position outside [0, t_max)
 *                 writes nothing (checked on the device, no error).
 *   codes         cache [batch, heads, t_max, k/2], 16-byte aligned.
 *   scales        cache [batch, heads, t_max, k/block], 4-byte aligned.
 *   tensor_scale  NVFP4: one device float, used as given (a cache keeps one
 *                 tensor scale for the tokens it already holds); MXFP4: NULL.
 *   Each row is quantized exactly as fp4_quantize quantizes it (GIVEN mode
 *   for NVFP4); rows of the cache that are not written are not touched.
 *   k % block == 0; batch, heads or t_new of 0 enqueue nothing; one call
 *   appends fewer than 2^34 values (else FP4_EUNSUPPORTED).
 *   Returns FP4_OK, FP4_EINVAL, FP4_EUNSUPPORTED or FP4_EHIP.
 */
fp4_status fp4_kv_append(fp4_format fmt, const void* x, fp4_dtype x_dtype, int64_t batch,
                         int64_t heads, int64_t t_new, int64_t k, const int32_t* positions,
                         uint8_t* codes, uint8_t* scales, const float* tensor_scale,
                         int64_t t_max, void* stream);

/* Bytes of device workspace fp4_attention_decode needs for these sizes. */
size_t fp4_attention_workspace_size(int64_t batch, int64_t q_heads, int64_t kv_heads,
                                    int64_t head_dim, int64_t t_max);

/*
 * fp4_attention_decode -- one query token per sequence attending over a
 * 4-bit KV cache dequantized to FP8.
 * Defines: the read side of the hyper.ai story on the NVFP4 KV cache (the
 * cached K and V are dequantized to FP8 before attention).  Each cached
 * element enters as exactly the E4M3 byte fp4_dequantize(..., FP4_E4M3)
 * gives it; then
 *   out[b, j, :] = sum_{t < seq_lens[b]} softmax_t(softmax_scale *
 *                  K[b, j/G, t, :] . q[b, j, :]) V[b, j/G, t, :]
 * with G = q_heads / kv_heads (grouped query heads); a sequence of length 0
 * gives zeros.
 *   fmt           FP4_NVFP4 or FP4_MXFP4 (both caches).
 *   q, q_dtype    [batch, q_heads, head_dim], FP4_BF16 or FP4_F16 (FP4_F32:
 *                 FP4_EUNSUPPORTED), 16-byte aligned.
 *   k_codes, k_scales, k_tscale, v_codes, v_scales, v_tscale
 *                 caches [batch, kv_heads, t_max, head_dim/2] (16-byte
 *                 aligned) and [.., head_dim/block] (4-byte aligned), as
 *                 fp4_kv_append writes them; tensor scales are device floats
 *                 (NVFP4) or NULL (MXFP4).
 *   seq_lens      device int32 [batch]; values are clamped to [0, t_max].
 *   out, out_dtype  [batch, q_heads, head_dim], FP4_F32 or FP4_BF16
 *                 (nearest even), 16-byte aligned.
 *   workspace     at least fp4_attention_workspace_size() bytes, 16-byte
 *                 aligned (split-token partial results).
 *   head_dim must be 128, q_heads / kv_heads at most 16 and t_max at most
 *   2^26 (else FP4_EUNSUPPORTED); q_heads must be a multiple of kv_heads.
 *   Numerics: K . q on the matrix cores with FP8 K widened exactly to the
 *   16-bit type of q, fp32 sums; fp32 softmax; the weights rounded to fp16
 *   (nearest even) for the weighted sum of V, fp32 sums.
 *   Returns FP4_OK, FP4_EINVAL, FP4_EUNSUPPORTED or FP4_EHIP.
 */
fp4_status fp4_attention_decode(fp4_format fmt, const void* q, fp4_dtype q_dtype,
                                int64_t batch, int64_t q_heads, int64_t kv_heads,
                                int64_t head_dim, const uint8_t* k_codes,
                                const uint8_t* k_scales, const float* k_tscale,
                                const uint8_t* v_codes, const uint8_t* v_scales,
                                const float* v_tscale, int64_t t_max, const int32_t* seq_lens,
                                float softmax_scale, void* out, fp4_dtype out_dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace fp4_gptq_quantize needs (0: sizes not accepted). */
size_t fp4_gptq_workspace_size(int64_t n, int64_t k, int64_t n_calib);

/*
 * fp4_gptq_quantize -- MR-GPTQ: quantize a weight matrix to FP4 with GPTQ's
 * error correction on blockwise-Hadamard-rotated weights.
 * Defines: hyper.ai, paper 2509.23202 (MR-GPTQ), Abstract (GPTQ adapted to
 * FP4 with blockwise Hadamard transforms, the rotation fused into the
 * weights); pimento.cloud "FP8, NVFP4 czy AWQ?", section "Czym roznia sie
 * FP8, NVFP4, MXFP4 i AWQ?" (GPTQ: layer-wise quantization with error
 * correction).
 *   w, w_dtype    weights [n, k] (F32 / BF16 / F16), 16-byte aligned.
 *   x, x_dtype    calibration activations [n_calib, k], 16-byte aligned.
 *   damp          H_jj += damp * mean(diag H) (GPTQ's damping; 0.01 typical).
 *   rotate        nonzero: W and X rotated by the format's blockwise
 *                 Hadamard (16 NVFP4, 32 MXFP4) first; the result is then
 *                 the operand for activations quantized with
 *                 fp4_hadamard_quantize.  0: no rotation (plain GPTQ).
 *   codes, scales, tensor_scale  out: as fp4_quantize writes them for the
 *                 (rotated) weights; NVFP4's tensor scale max |W| / 2688
 *                 (device float), MXFP4: must be NULL.
 *   Computes H = 2/N X^T X (fp64), zeroes the weights of features with
 *   H_jj = 0, damps, takes U = the upper Cholesky factor of H^-1 and walks
 *   the columns: each quantization block's scale from its current weights
 *   (the quantizer's rule), each column quantized as the quantizer does it
 *   (fp32), err = (w - q) / U_jj corrected into the later columns.  Linear
 *   algebra in fp64.  k % 128 == 0, k <= 16384 (else FP4_EUNSUPPORTED).
 *   workspace     at least fp4_gptq_workspace_size() bytes, 16-byte aligned
 *                 (fp64 copies of W and X, two k x k matrices).
 *   Returns FP4_OK, FP4_EINVAL, FP4_EUNSUPPORTED or FP4_EHIP.  A Hessian
 *   that is not positive definite after damping gives NaN weights.
 */
fp4_status fp4_gptq_quantize(fp4_format fmt, const void* w, fp4_dtype w_dtype, int64_t n,
                             int64_t k, const void* x, fp4_dtype x_dtype, int64_t n_calib,
                             double damp, int rotate, uint8_t* codes, uint8_t* scales,
                             float* tensor_scale, void* workspace, size_t workspace_bytes,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */

// Internal host-side launchers (not part of the C ABI).  Each validates
// nothing: fp4_api.cpp checks every argument before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Same values as fp4_format / fp4_dtype in include/fp4.h.
constexpr int kFmtNV = 0;
constexpr int kFmtMX = 1;
constexpr int kInF32 = 0;
constexpr int kInBF16 = 1;
constexpr int kInF16 = 2;
constexpr int kOutE4M3 = 3;

size_t quantize_workspace_bytes(int fmt, bool compute);

// The library's own scratch for launch_quantize's workspace on the current
// device (its address and size); looked up once per device.
hipError_t quantize_static_scratch(void** ptr, size_t* bytes);

// n = rows * k elements (a multiple of 16 for NVFP4, 32 for MXFP4).
hipError_t launch_quantize(int fmt, bool hadamard, const void* x, int dtype,
                           int64_t n, uint8_t* codes, uint8_t* scales,
                           float* tscale, bool compute, void* workspace,
                           hipStream_t stream);

// NVFP4 with the least-squared-error block scale; n = rows * k, a multiple
// of 16.  Same workspace as launch_quantize in compute mode.
hipError_t launch_quantize_mse(const void* x, int dtype, int64_t n, uint8_t* codes,
                               uint8_t* scales, float* tscale, bool compute, void* workspace,
                               hipStream_t stream);

hipError_t launch_dequantize(int fmt, const uint8_t* codes,
                             const uint8_t* scales, const float* tscale,
                             int64_t n, void* out, int out_dtype,
                             hipStream_t stream);

size_t gemm_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k);
// Split-k GEMMs: elements between two slices of fp32 partial sums (m n
// rounded up to a multiple of 4), and the pass that adds the nsplit slices
// in order, applies at * bt (NVFP4; at == nullptr: 1) and stores C.
int64_t gemm_split_stride(int64_t m, int64_t n);
// chunks of k for the decode stream kernels (0: a k they do not take)
int64_t gemm_stream_chunks(int64_t k);
hipError_t launch_split_reduce(const float* part, int nsplit, int64_t m, int64_t n, const float* at,
                               const float* bt, void* c, int c_dtype, hipStream_t stream);

hipError_t launch_gemm(int fmt, int64_t m, int64_t n, int64_t k,
                       const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_tscale, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_tscale, void* c,
                       int c_dtype, void* workspace, hipStream_t stream);

// MXFP4 decode GEMM on the block-scaled FP4 matrix instruction (m <= 16, k a
// multiple of 2048, any n, codes 16-byte and scales 8-byte aligned), with
// (quantize_gemm: bf16 X) or without the activation quantize in the launch;
// false (nothing launched) for any other shape.  k > 4096 splits over
// workgroups: gemm_mx_stream_workspace_bytes of workspace.
size_t gemm_mx_stream_workspace_bytes(int64_t m, int64_t n, int64_t k);
bool launch_gemm_mx_decode(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes,
                           const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                           void* c, int c_dtype, void* workspace, hipStream_t stream, hipError_t* err);
bool launch_quantize_gemm_mx_decode(int64_t m, int64_t n, int64_t k, const void* x, uint8_t* a_codes,
                                    uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                                    void* c, int c_dtype, void* workspace, hipStream_t stream, hipError_t* err);
// W4A16 with MXFP4 weights and bf16 X on the same kernel (any m, 16 rows per
// launch; k a multiple of 2048, any n); false (nothing launched) otherwise.
bool launch_gemm_w4a16_mx(int64_t m, int64_t n, int64_t k, const void* x, const uint8_t* b_codes,
                          const uint8_t* b_scales, void* c, int c_dtype, void* workspace, hipStream_t stream,
                          hipError_t* err);
// One-launch NVFP4 activation quantize (tensor scale from the data) + GEMM
// for the decode shapes; false (nothing launched) for any other shape.
bool launch_quantize_gemm_decode(int64_t m, int64_t n, int64_t k, const void* x,
                                 uint8_t* a_codes, uint8_t* a_scales, float* a_tscale,
                                 const uint8_t* b_codes, const uint8_t* b_scales,
                                 const float* b_tscale, void* c, int c_dtype, hipStream_t stream,
                                 hipError_t* err);

// W4A16: C [m, n] = X [m, k] (16-bit or fp32 activations, as they are) times
// the dequantized 4-bit weights B [n, k].
size_t gemm_w4a16_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_w4a16(int fmt, int64_t m, int64_t n, int64_t k, const void* x, int x_dtype,
                             const uint8_t* b_codes, const uint8_t* b_scales,
                             const float* b_tscale, void* c, int c_dtype, void* workspace,
                             hipStream_t stream);

// KV cache append: rows of x [batch, heads, t_new, k] quantized (NVFP4 with
// the given tensor scale) into a [batch, heads, t_max, ...] cache at
// positions[b] + i; rows outside [0, t_max) are not stored.  At most 2^31 - 1
// chunks of 8 values per call.
hipError_t launch_kv_append(int fmt, const void* x, int dtype, int64_t batch, int64_t heads,
                            int64_t t_new, int64_t k, const int32_t* positions, int64_t t_max,
                            uint8_t* codes, uint8_t* scales, const float* tscale,
                            hipStream_t stream);

// Decode attention over an FP4 KV cache (head_dim 128, q_heads a multiple
// of kv_heads by at most 16), K and V dequantized to FP8 E4M3 on the fly.
size_t attention_workspace_bytes(int64_t batch, int64_t q_heads, int64_t kv_heads, int64_t t_max);
hipError_t launch_attention_decode(int fmt, const void* q, int q_dtype, int64_t batch,
                                   int64_t q_heads, int64_t kv_heads, const uint8_t* k_codes,
                                   const uint8_t* k_scales, const float* k_tscale,
                                   const uint8_t* v_codes, const uint8_t* v_scales,
                                   const float* v_tscale, int64_t t_max, const int32_t* seq_lens,
                                   float softmax_scale, void* out, int out_dtype, void* workspace,
                                   hipStream_t stream);

// Blockwise Hadamard (hadamard = 16 or 32; 0 copies) of n values, fp32
// arithmetic, widened to fp64.
hipError_t launch_rotate_f64(const void* x, int dtype, int64_t n, int hadamard, double* out,
                             hipStream_t stream);

// MR-GPTQ of W [n, k] with calibration X [n_calib, k] (k % 128 == 0).
size_t gptq_workspace_bytes(int64_t n, int64_t k, int64_t n_calib);
hipError_t launch_gptq(int fmt, const void* w, int w_dtype, int64_t n, int64_t k, const void* x,
                       int x_dtype, int64_t n_calib, double damp, bool rotate, uint8_t* codes,
                       uint8_t* scales, float* tscale, void* workspace, hipStream_t stream);

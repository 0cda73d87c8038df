// C ABI of libfp4.so (declared in include/fp4.h): host-side argument checks
// and dispatch to the HIP launchers.  Every check runs before any HIP call,
// so a rejected call enqueues nothing and touches no output.
#include "fp4.h"

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace {

constexpr int64_t kMaxElements = int64_t(1) << 40;

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

int block_of(fp4_format f) { return f == FP4_NVFP4 ? 16 : 32; }

bool valid_format(fp4_format f) { return f == FP4_NVFP4 || f == FP4_MXFP4; }

fp4_status from_hip(hipError_t e) {
  if (e == hipSuccess) return FP4_OK;
  (void)hipGetLastError();   // clear the sticky launch error
  return FP4_EHIP;
}

// Shared checks of fp4_quantize / fp4_hadamard_quantize.
// check_workspace = false: the caller brings no workspace (the library's
// own scratch is used).
fp4_status check_quantize(fp4_format fmt, const void* x, fp4_dtype x_dtype,
                          int64_t rows, int64_t k, const uint8_t* codes,
                          const uint8_t* scales, const float* tensor_scale,
                          fp4_tscale_mode mode, const void* workspace,
                          size_t workspace_bytes, bool check_workspace = true) {
  if (!valid_format(fmt)) return FP4_EINVAL;
  if (x_dtype != FP4_F32 && x_dtype != FP4_BF16 && x_dtype != FP4_F16) return FP4_EINVAL;
  if (fmt == FP4_NVFP4 && mode != FP4_TSCALE_COMPUTE && mode != FP4_TSCALE_GIVEN) return FP4_EINVAL;
  if (rows < 0 || k <= 0 || k % block_of(fmt) != 0) return FP4_EINVAL;
  if (rows > 0 && k > kMaxElements / rows) return FP4_EINVAL;
  if (rows == 0) return FP4_OK;
  if (!x || !codes || !scales) return FP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return FP4_EINVAL;
  if (fmt == FP4_NVFP4) {
    if (!tensor_scale || !aligned(tensor_scale, 4)) return FP4_EINVAL;
    const size_t need = fp4_quantize_workspace_size(fmt, mode, rows, k);
    if (check_workspace && need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
      return FP4_EINVAL;
  } else if (tensor_scale) {
    return FP4_EINVAL;
  }
  return FP4_OK;
}

fp4_status quantize_common(bool hadamard, fp4_format fmt, const void* x,
                           fp4_dtype x_dtype, int64_t rows, int64_t k,
                           uint8_t* codes, uint8_t* scales, float* tensor_scale,
                           fp4_tscale_mode mode, void* workspace,
                           size_t workspace_bytes, void* stream) {
  fp4_status s = check_quantize(fmt, x, x_dtype, rows, k, codes, scales,
                                tensor_scale, mode, workspace, workspace_bytes);
  if (s != FP4_OK || rows == 0) return s;
  const bool compute = fmt == FP4_NVFP4 && mode == FP4_TSCALE_COMPUTE;
  return from_hip(launch_quantize((int)fmt, hadamard, x, (int)x_dtype, rows * k,
                                  codes, scales, tensor_scale, compute,
                                  workspace, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* fp4_status_string(fp4_status s) {
  switch (s) {
    case FP4_OK: return "FP4_OK";
    case FP4_EINVAL: return "FP4_EINVAL: invalid argument";
    case FP4_EUNSUPPORTED: return "FP4_EUNSUPPORTED: combination not implemented";
    case FP4_EHIP: return "FP4_EHIP: HIP launch failed";
  }
  return "unknown fp4_status";
}

size_t fp4_quantize_workspace_size(fp4_format fmt, fp4_tscale_mode mode,
                                   int64_t rows, int64_t k) {
  (void)rows;
  (void)k;
  if (!valid_format(fmt)) return 0;
  return quantize_workspace_bytes((int)fmt, fmt == FP4_NVFP4 && mode == FP4_TSCALE_COMPUTE);
}

fp4_status fp4_quantize(fp4_format fmt, const void* x, fp4_dtype x_dtype,
                        int64_t rows, int64_t k, uint8_t* codes,
                        uint8_t* scales, float* tensor_scale,
                        fp4_tscale_mode mode, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return quantize_common(false, fmt, x, x_dtype, rows, k, codes, scales,
                         tensor_scale, mode, workspace, workspace_bytes, stream);
}

fp4_status fp4_hadamard_quantize(fp4_format fmt, const void* x,
                                 fp4_dtype x_dtype, int64_t rows, int64_t k,
                                 uint8_t* codes, uint8_t* scales,
                                 float* tensor_scale, fp4_tscale_mode mode,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return quantize_common(true, fmt, x, x_dtype, rows, k, codes, scales,
                         tensor_scale, mode, workspace, workspace_bytes, stream);
}

fp4_status fp4_quantize_noalloc(fp4_format fmt, const void* x, fp4_dtype x_dtype, int64_t rows,
                                int64_t k, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                fp4_tscale_mode mode, void* stream) {
  fp4_status s = check_quantize(fmt, x, x_dtype, rows, k, codes, scales, tensor_scale, mode,
                                nullptr, 0, false);
  if (s != FP4_OK || rows == 0) return s;
  const bool compute = fmt == FP4_NVFP4 && mode == FP4_TSCALE_COMPUTE;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (compute) {
    const hipError_t e = quantize_static_scratch(&scratch, &scratch_bytes);
    if (e != hipSuccess) return from_hip(e);
    // the compute-mode max pass writes at most this many bytes for any size
    if (scratch_bytes < quantize_workspace_bytes((int)fmt, true)) return FP4_EUNSUPPORTED;
  }
  return from_hip(launch_quantize((int)fmt, false, x, (int)x_dtype, rows * k, codes, scales,
                                  tensor_scale, compute, scratch, static_cast<hipStream_t>(stream)));
}

fp4_status fp4_quantize_mse(const void* x, fp4_dtype x_dtype, int64_t rows, int64_t k,
                            uint8_t* codes, uint8_t* scales, float* tensor_scale,
                            fp4_tscale_mode mode, void* workspace, size_t workspace_bytes,
                            void* stream) {
  fp4_status s = check_quantize(FP4_NVFP4, x, x_dtype, rows, k, codes, scales, tensor_scale,
                                mode, workspace, workspace_bytes);
  if (s != FP4_OK || rows == 0) return s;
  return from_hip(launch_quantize_mse(x, (int)x_dtype, rows * k, codes, scales, tensor_scale,
                                      mode == FP4_TSCALE_COMPUTE, workspace,
                                      static_cast<hipStream_t>(stream)));
}

fp4_status fp4_dequantize(fp4_format fmt, const uint8_t* codes,
                          const uint8_t* scales, const float* tensor_scale,
                          int64_t rows, int64_t k, void* out,
                          fp4_dtype out_dtype, void* stream) {
  if (!valid_format(fmt)) return FP4_EINVAL;
  if (out_dtype != FP4_F32 && out_dtype != FP4_BF16 && out_dtype != FP4_F16 &&
      out_dtype != FP4_E4M3)
    return FP4_EINVAL;
  if (rows < 0 || k <= 0 || k % block_of(fmt) != 0) return FP4_EINVAL;
  if (rows > 0 && k > kMaxElements / rows) return FP4_EINVAL;
  if (rows == 0) return FP4_OK;
  if (!codes || !scales || !out) return FP4_EINVAL;
  if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(out, 16)) return FP4_EINVAL;
  if (fmt == FP4_NVFP4) {
    if (!tensor_scale || !aligned(tensor_scale, 4)) return FP4_EINVAL;
  } else if (tensor_scale) {
    return FP4_EINVAL;
  }
  return from_hip(launch_dequantize((int)fmt, codes, scales, tensor_scale, rows * k,
                                    out, (int)out_dtype,
                                    static_cast<hipStream_t>(stream)));
}

size_t fp4_gemm_workspace_size(fp4_format fmt, int64_t m, int64_t n, int64_t k) {
  if (!valid_format(fmt)) return 0;
  return gemm_workspace_bytes((int)fmt, m, n, k);
}

fp4_status fp4_gemm(fp4_format fmt, int64_t m, int64_t n, int64_t k,
                    const uint8_t* a_codes, const uint8_t* a_scales,
                    const float* a_tscale, const uint8_t* b_codes,
                    const uint8_t* b_scales, const float* b_tscale, void* c,
                    fp4_dtype c_dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!valid_format(fmt)) return FP4_EINVAL;
  if (c_dtype != FP4_F32 && c_dtype != FP4_BF16) {
    return (c_dtype == FP4_F16 || c_dtype == FP4_E4M3) ? FP4_EUNSUPPORTED : FP4_EINVAL;
  }
  if (m < 0 || n < 0 || k <= 0 || k % 32 != 0) return FP4_EINVAL;
  if ((m > 0 && k > kMaxElements / m) || (n > 0 && k > kMaxElements / n)) return FP4_EINVAL;
  if (m > 0 && n > kMaxElements / m) return FP4_EINVAL;
  if (m == 0 || n == 0) return FP4_OK;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return FP4_EINVAL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(c, 16))
    return FP4_EINVAL;
  if (fmt == FP4_NVFP4) {
    if (!a_tscale || !b_tscale || !aligned(a_tscale, 4) || !aligned(b_tscale, 4)) return FP4_EINVAL;
  } else if (a_tscale || b_tscale) {
    return FP4_EINVAL;
  }
  const size_t need = gemm_workspace_bytes((int)fmt, m, n, k);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16))) return FP4_EINVAL;
  return from_hip(launch_gemm((int)fmt, m, n, k, a_codes, a_scales, a_tscale,
                              b_codes, b_scales, b_tscale, c, (int)c_dtype,
                              workspace, static_cast<hipStream_t>(stream)));
}

size_t fp4_gemm_w4a16_workspace_size(fp4_format fmt, int64_t m, int64_t n, int64_t k) {
  if (!valid_format(fmt)) return 0;
  return fmt == FP4_MXFP4 ? gemm_mx_stream_workspace_bytes(m, n, k) : gemm_w4a16_workspace_bytes((int)fmt, m, n, k);
}

fp4_status fp4_gemm_w4a16(fp4_format fmt, const void* x, fp4_dtype x_dtype, int64_t m, int64_t n,
                          int64_t k, const uint8_t* b_codes, const uint8_t* b_scales,
                          const float* b_tscale, void* c, fp4_dtype c_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!valid_format(fmt)) return FP4_EINVAL;
  if (x_dtype != FP4_F32 && x_dtype != FP4_BF16 && x_dtype != FP4_F16) return FP4_EINVAL;
  if (c_dtype != FP4_F32 && c_dtype != FP4_BF16) {
    return (c_dtype == FP4_F16 || c_dtype == FP4_E4M3) ? FP4_EUNSUPPORTED : FP4_EINVAL;
  }
  if (m < 0 || n < 0 || k <= 0 || k % block_of(fmt) != 0) return FP4_EINVAL;
  if ((m > 0 && k > kMaxElements / m) || (n > 0 && k > kMaxElements / n)) return FP4_EINVAL;
  if (m > 0 && n > kMaxElements / m) return FP4_EINVAL;
  if (m == 0 || n == 0) return FP4_OK;
  if (!x || !b_codes || !b_scales || !c) return FP4_EINVAL;
  const int xs = x_dtype == FP4_F32 ? 4 : 2;
  if (!aligned(x, xs) || !aligned(b_codes, 4) || !aligned(c, c_dtype == FP4_F32 ? 4 : 2)) return FP4_EINVAL;
  if (fmt == FP4_NVFP4) {
    if (!b_tscale || !aligned(b_tscale, 4)) return FP4_EINVAL;
  } else if (b_tscale) {
    return FP4_EINVAL;
  }
  const size_t need = fp4_gemm_w4a16_workspace_size(fmt, m, n, k);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16))) return FP4_EINVAL;
  if (fmt == FP4_MXFP4 && x_dtype == FP4_BF16) {
    hipError_t e = hipSuccess;
    if (launch_gemm_w4a16_mx(m, n, k, x, b_codes, b_scales, c, (int)c_dtype, workspace,
                             static_cast<hipStream_t>(stream), &e))
      return from_hip(e);
  }
  return from_hip(launch_gemm_w4a16((int)fmt, m, n, k, x, (int)x_dtype, b_codes, b_scales,
                                    b_tscale, c, (int)c_dtype, workspace,
                                    static_cast<hipStream_t>(stream)));
}

size_t fp4_quantize_gemm_workspace_size(fp4_format fmt, int64_t m, int64_t n, int64_t k) {
  if (!valid_format(fmt)) return 0;
  const size_t q = fp4_quantize_workspace_size(fmt, FP4_TSCALE_COMPUTE, m, k);
  const size_t g = gemm_workspace_bytes((int)fmt, m, n, k);
  return q > g ? q : g;
}

fp4_status fp4_quantize_gemm(fp4_format fmt, const void* x, fp4_dtype x_dtype,
                             int64_t m, int64_t n, int64_t k, uint8_t* a_codes,
                             uint8_t* a_scales, float* a_tscale,
                             const uint8_t* b_codes, const uint8_t* b_scales,
                             const float* b_tscale, void* c, fp4_dtype c_dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  // Both calls' checks first, so a rejected call enqueues nothing.
  fp4_status s = check_quantize(fmt, x, x_dtype, m, k, a_codes, a_scales, a_tscale,
                                FP4_TSCALE_COMPUTE, workspace, workspace_bytes);
  if (s != FP4_OK) return s;
  if (!valid_format(fmt)) return FP4_EINVAL;
  if (c_dtype != FP4_F32 && c_dtype != FP4_BF16) {
    return (c_dtype == FP4_F16 || c_dtype == FP4_E4M3) ? FP4_EUNSUPPORTED : FP4_EINVAL;
  }
  if (n < 0 || k % 32 != 0) return FP4_EINVAL;
  if ((n > 0 && k > kMaxElements / n) || (m > 0 && n > kMaxElements / m)) return FP4_EINVAL;
  if (m == 0) return FP4_OK;
  if (n > 0) {
    if (!b_codes || !b_scales || !c) return FP4_EINVAL;
    if (!aligned(b_codes, 16) || !aligned(b_scales, 4) || !aligned(c, 16)) return FP4_EINVAL;
    if (fmt == FP4_NVFP4) {
      if (!b_tscale || !aligned(b_tscale, 4)) return FP4_EINVAL;
    } else if (b_tscale) {
      return FP4_EINVAL;
    }
    const size_t need = gemm_workspace_bytes((int)fmt, m, n, k);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16))) return FP4_EINVAL;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fmt == FP4_NVFP4 && x_dtype == FP4_BF16 && n > 0) {
    hipError_t e = hipSuccess;
    if (launch_quantize_gemm_decode(m, n, k, x, a_codes, a_scales, a_tscale, b_codes, b_scales,
                                    b_tscale, c, (int)c_dtype, st, &e))
      return from_hip(e);
  }
  if (fmt == FP4_MXFP4 && x_dtype == FP4_BF16 && n > 0) {
    hipError_t e = hipSuccess;
    if (launch_quantize_gemm_mx_decode(m, n, k, x, a_codes, a_scales, b_codes, b_scales, c, (int)c_dtype,
                                       workspace, st, &e))
      return from_hip(e);
  }
  s = quantize_common(false, fmt, x, x_dtype, m, k, a_codes, a_scales, a_tscale,
                      FP4_TSCALE_COMPUTE, workspace, workspace_bytes, stream);
  if (s != FP4_OK || n == 0) return s;
  return from_hip(launch_gemm((int)fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes,
                              b_scales, b_tscale, c, (int)c_dtype, workspace, st));
}

fp4_status fp4_kv_append(fp4_format fmt, const void* x, fp4_dtype x_dtype, int64_t batch,
                         int64_t heads, int64_t t_new, int64_t k, const int32_t* positions,
                         uint8_t* codes, uint8_t* scales, const float* tensor_scale,
                         int64_t t_max, void* stream) {
  if (!valid_format(fmt)) return FP4_EINVAL;
  if (x_dtype != FP4_F32 && x_dtype != FP4_BF16 && x_dtype != FP4_F16) return FP4_EINVAL;
  if (batch < 0 || heads < 0 || t_new < 0 || t_max <= 0) return FP4_EINVAL;
  if (k <= 0 || k % block_of(fmt) != 0) return FP4_EINVAL;
  if (batch > 0 && heads > kMaxElements / batch) return FP4_EINVAL;
  const int64_t bh = batch * heads;
  if (bh > 0 && (t_max > kMaxElements / bh || t_new > kMaxElements / bh)) return FP4_EINVAL;
  if (bh > 0 && (k > kMaxElements / (bh * t_max) || (t_new > 0 && k > kMaxElements / (bh * t_new))))
    return FP4_EINVAL;
  if (bh == 0 || t_new == 0) return FP4_OK;
  if (bh * t_new > (int64_t(1) << 31) / (k / 8) - 1) return FP4_EUNSUPPORTED;
  if (!x || !positions || !codes || !scales) return FP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(positions, 4))
    return FP4_EINVAL;
  if (fmt == FP4_NVFP4) {
    if (!tensor_scale || !aligned(tensor_scale, 4)) return FP4_EINVAL;
  } else if (tensor_scale) {
    return FP4_EINVAL;
  }
  return from_hip(launch_kv_append((int)fmt, x, (int)x_dtype, batch, heads, t_new, k, positions,
                                   t_max, codes, scales, tensor_scale,
                                   static_cast<hipStream_t>(stream)));
}

size_t fp4_attention_workspace_size(int64_t batch, int64_t q_heads, int64_t kv_heads,
                                    int64_t head_dim, int64_t t_max) {
  if (batch <= 0 || kv_heads <= 0 || q_heads <= 0 || q_heads % kv_heads != 0 || t_max <= 0 ||
      head_dim != 128 || q_heads / kv_heads > 16 || t_max > (int64_t(1) << 26))
    return 0;
  return attention_workspace_bytes(batch, q_heads, kv_heads, t_max);
}

fp4_status fp4_attention_decode(fp4_format fmt, const void* q, fp4_dtype q_dtype,
                                int64_t batch, int64_t q_heads, int64_t kv_heads,
                                int64_t head_dim, const uint8_t* k_codes,
                                const uint8_t* k_scales, const float* k_tscale,
                                const uint8_t* v_codes, const uint8_t* v_scales,
                                const float* v_tscale, int64_t t_max, const int32_t* seq_lens,
                                float softmax_scale, void* out, fp4_dtype out_dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_format(fmt)) return FP4_EINVAL;
  if (q_dtype != FP4_BF16 && q_dtype != FP4_F16) {
    return q_dtype == FP4_F32 ? FP4_EUNSUPPORTED : FP4_EINVAL;
  }
  if (out_dtype != FP4_F32 && out_dtype != FP4_BF16) {
    return (out_dtype == FP4_F16 || out_dtype == FP4_E4M3) ? FP4_EUNSUPPORTED : FP4_EINVAL;
  }
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || t_max <= 0 || head_dim <= 0) return FP4_EINVAL;
  if (q_heads % kv_heads != 0 || head_dim % block_of(fmt) != 0) return FP4_EINVAL;
  if (head_dim != 128 || q_heads / kv_heads > 16 || t_max > (int64_t(1) << 26)) return FP4_EUNSUPPORTED;
  if (q_heads > (int64_t(1) << 20) || kv_heads > (int64_t(1) << 20)) return FP4_EINVAL;
  if (batch > 0 && (kv_heads > kMaxElements / batch || q_heads > kMaxElements / batch))
    return FP4_EINVAL;
  if (batch > 0 && t_max > kMaxElements / (batch * kv_heads * head_dim)) return FP4_EINVAL;
  if (batch > (int64_t(1) << 31) / kv_heads || batch > (int64_t(1) << 31) / q_heads) return FP4_EINVAL;
  if (batch == 0) return FP4_OK;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !seq_lens || !out) return FP4_EINVAL;
  if (!aligned(q, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_scales, 4) ||
      !aligned(v_scales, 4) || !aligned(seq_lens, 4) || !aligned(out, 16))
    return FP4_EINVAL;
  if (fmt == FP4_NVFP4) {
    if (!k_tscale || !v_tscale || !aligned(k_tscale, 4) || !aligned(v_tscale, 4)) return FP4_EINVAL;
  } else if (k_tscale || v_tscale) {
    return FP4_EINVAL;
  }
  const size_t need = attention_workspace_bytes(batch, q_heads, kv_heads, t_max);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return FP4_EINVAL;
  return from_hip(launch_attention_decode((int)fmt, q, (int)q_dtype, batch, q_heads, kv_heads,
                                          k_codes, k_scales, k_tscale, v_codes, v_scales,
                                          v_tscale, t_max, seq_lens, softmax_scale, out,
                                          (int)out_dtype, workspace,
                                          static_cast<hipStream_t>(stream)));
}

size_t fp4_gptq_workspace_size(int64_t n, int64_t k, int64_t n_calib) {
  if (n <= 0 || k <= 0 || n_calib <= 0 || k % 128 != 0 || k > 16384) return 0;
  if (n > kMaxElements / k || n_calib > kMaxElements / k) return 0;
  return gptq_workspace_bytes(n, k, n_calib);
}

fp4_status fp4_gptq_quantize(fp4_format fmt, const void* w, fp4_dtype w_dtype, int64_t n,
                             int64_t k, const void* x, fp4_dtype x_dtype, int64_t n_calib,
                             double damp, int rotate, uint8_t* codes, uint8_t* scales,
                             float* tensor_scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!valid_format(fmt)) return FP4_EINVAL;
  if (w_dtype != FP4_F32 && w_dtype != FP4_BF16 && w_dtype != FP4_F16) return FP4_EINVAL;
  if (x_dtype != FP4_F32 && x_dtype != FP4_BF16 && x_dtype != FP4_F16) return FP4_EINVAL;
  if (n <= 0 || k <= 0 || n_calib <= 0 || k % 128 != 0) return FP4_EINVAL;
  if (!(damp >= 0.0) || damp > 1e30) return FP4_EINVAL;
  if (k > 16384) return FP4_EUNSUPPORTED;
  if (n > kMaxElements / k || n_calib > kMaxElements / k) return FP4_EINVAL;
  if ((n + 63) / 64 > (int64_t(1) << 31) || n * k / 8 > (int64_t(1) << 31) * 256 ||
      n_calib * k / 8 > (int64_t(1) << 31) * 256)
    return FP4_EUNSUPPORTED;
  if (!w || !x || !codes || !scales || !workspace) return FP4_EINVAL;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) ||
      !aligned(workspace, 16))
    return FP4_EINVAL;
  if (fmt == FP4_NVFP4) {
    if (!tensor_scale || !aligned(tensor_scale, 4)) return FP4_EINVAL;
  } else if (tensor_scale) {
    return FP4_EINVAL;
  }
  if (workspace_bytes < gptq_workspace_bytes(n, k, n_calib)) return FP4_EINVAL;
  return from_hip(launch_gptq((int)fmt, w, (int)w_dtype, n, k, x, (int)x_dtype, n_calib, damp,
                              rotate != 0, codes, scales, tensor_scale, workspace,
                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"

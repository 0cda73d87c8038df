// fp4_gemm dispatch: picks a kernel by format and shape.
#include "launch.hpp"

hipError_t launch_gemm_simple(int fmt, int64_t m, int64_t n, int64_t k,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_tscale, const uint8_t* b_codes,
                              const uint8_t* b_scales, const float* b_tscale,
                              void* c, int c_dtype, hipStream_t stream);

hipError_t launch_gemm_skinny(int fmt, int64_t m, int64_t n, int64_t k,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_tscale, const uint8_t* b_codes,
                              const uint8_t* b_scales, const float* b_tscale,
                              void* c, int c_dtype, hipStream_t stream);

bool gemm_large_supported(int fmt, int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_large(int fmt, int64_t m, int64_t n, int64_t k,
                             const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tscale, const uint8_t* b_codes,
                             const uint8_t* b_scales, const float* b_tscale,
                             void* c, int c_dtype, hipStream_t stream);

size_t gemm_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
  (void)fmt;
  (void)m;
  (void)n;
  (void)k;
  return 0;
}

hipError_t launch_gemm(int fmt, int64_t m, int64_t n, int64_t k,
                       const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_tscale, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_tscale, void* c,
                       int c_dtype, void* workspace, hipStream_t stream) {
  (void)workspace;
  if (m <= 16) {
    return launch_gemm_skinny(fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes,
                              b_scales, b_tscale, c, c_dtype, stream);
  }
  if (gemm_large_supported(fmt, m, n, k)) {
    return launch_gemm_large(fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                             b_tscale, c, c_dtype, stream);
  }
  return launch_gemm_simple(fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes,
                            b_scales, b_tscale, c, c_dtype, stream);
}

// fp4_gemm dispatch: picks a kernel by format and shape.
#include "launch.hpp"

hipError_t launch_gemm_simple(int fmt, int64_t m, int64_t n, int64_t k,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_tscale, const uint8_t* b_codes,
                              const uint8_t* b_scales, const float* b_tscale,
                              void* c, int c_dtype, hipStream_t stream);

size_t gemm_skinny_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_skinny(int fmt, int64_t m, int64_t n, int64_t k,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_tscale, const uint8_t* b_codes,
                              const uint8_t* b_scales, const float* b_tscale,
                              void* c, int c_dtype, void* workspace, hipStream_t stream);

bool gemm_large_supported(int fmt, int64_t m, int64_t n, int64_t k);
size_t gemm_large_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_large(int fmt, int64_t m, int64_t n, int64_t k,
                             const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tscale, const uint8_t* b_codes,
                             const uint8_t* b_scales, const float* b_tscale,
                             void* c, int c_dtype, void* workspace, hipStream_t stream);

// The large kernels split k over several workgroups per tile when the tiles
// alone would leave most CUs idle, and the decode kernels split a long k over
// workgroup rows; the slices' fp32 sums go to the workspace.
size_t gemm_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
  if (m <= 16) return fmt == kFmtMX ? gemm_mx_stream_workspace_bytes(m, n, k) : gemm_skinny_workspace_bytes(fmt, m, n, k);
  if (gemm_large_supported(fmt, m, n, k)) return gemm_large_workspace_bytes(fmt, m, n, k);
  return 0;
}

hipError_t launch_gemm(int fmt, int64_t m, int64_t n, int64_t k,
                       const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_tscale, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_tscale, void* c,
                       int c_dtype, void* workspace, hipStream_t stream) {
  if (m <= 16) {
    hipError_t e = hipSuccess;
    if (fmt == kFmtMX && launch_gemm_mx_decode(m, n, k, a_codes, a_scales, b_codes, b_scales, c, c_dtype,
                                               workspace, stream, &e))
      return e;
    return launch_gemm_skinny(fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes,
                              b_scales, b_tscale, c, c_dtype, workspace, stream);
  }
  if (gemm_large_supported(fmt, m, n, k)) {
    return launch_gemm_large(fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                             b_tscale, c, c_dtype, workspace, stream);
  }
  return launch_gemm_simple(fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes,
                            b_scales, b_tscale, c, c_dtype, stream);
}

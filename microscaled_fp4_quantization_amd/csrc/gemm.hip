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
// A small batch past 16 rows on the decode kernels, in groups of 16
// activation rows, W streamed once per group:
// - NVFP4 with one chunk of k (2048..4096 values) below 96 rows.  The
//   generic kernel took 105-207 us for 17..100 rows of a 14336x4096 weight,
//   the decode kernel 10 us per 16 rows.
// - NVFP4 with a longer k (2 to 64 chunks of the split-k decode kernel) up
//   to 64 rows.  A group costs about what 16 rows alone do (13.6 us for a
//   4096x14336 weight, 38 us for 8192x28672, 9.5 us for 4096x8192), the
//   large kernel with one row of tiles a flat 84, 146 and 55 us: four
//   groups tie or win on all three, more lose on the largest.
// - MXFP4 up to 32 rows (k as below); from 33 the large kernel (one row of
//   tiles) is as fast as two groups.
constexpr int64_t kNvLongGroupsBelow = 65;

bool nv_long_k_chunks(int64_t k) {
  const int64_t s = gemm_stream_chunks(k);
  return s >= 2 && s <= 64;
}

bool small_batch_groups(int fmt, int64_t m, int64_t n, int64_t k) {
  if (m <= 16) return false;
  if (fmt == kFmtNV) return gemm_stream_chunks(k) == 1 ? m < 96 : nv_long_k_chunks(k) && m < kNvLongGroupsBelow;
  // MXFP4: k a multiple of 2048, or a longer k than 8192 with a short last
  // chunk (32x5120x13824: 39.5 us in groups, 75 on the generic kernel;
  // 32x13824x5120: 41.5 in groups, 35 generic)
  const int64_t s = gemm_stream_chunks(k);
  return m <= 32 && s >= 1 && s <= 64 && (k % 2048 == 0 || k > 8192);
}

// NVFP4 below 128 rows past the groups (from 96 rows, or from 65 with a
// long k): the large kernel with one partly filled row of tiles (rows past m
// load zeros and are not stored), 50 us for 100 rows of a 14336x4096 weight
// against 58 us in 16-row groups.
bool large_nv_below_128(int fmt, int64_t m, int64_t n, int64_t k) {
  if (fmt != kFmtNV || m >= 128 || m <= 16 || small_batch_groups(fmt, m, n, k)) return false;
  return m >= (nv_long_k_chunks(k) ? kNvLongGroupsBelow : 96) && gemm_large_supported(fmt, 128, n, k);
}

size_t gemm_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
  if (m <= 16 || small_batch_groups(fmt, m, n, k))   // one group's, reused by the next
    return fmt == kFmtMX ? gemm_mx_stream_workspace_bytes(m, n, k)
                         : gemm_skinny_workspace_bytes(fmt, m < 16 ? m : 16, n, k);
  if (large_nv_below_128(fmt, m, n, k)) return gemm_large_workspace_bytes(fmt, m, n, k);
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
  if (small_batch_groups(fmt, m, n, k)) {
    const int64_t osz = c_dtype == kInF32 ? 4 : 2, bs = fmt == kFmtNV ? 16 : 32;
    for (int64_t i0 = 0; i0 < m; i0 += 16) {
      const int64_t mc = m - i0 < 16 ? m - i0 : 16;
      const hipError_t e = launch_gemm(fmt, mc, n, k, a_codes + i0 * (k / 2), a_scales + i0 * (k / bs), a_tscale,
                                       b_codes, b_scales, b_tscale, reinterpret_cast<char*>(c) + i0 * n * osz,
                                       c_dtype, workspace, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (gemm_large_supported(fmt, m, n, k) || large_nv_below_128(fmt, m, n, k)) {
    return launch_gemm_large(fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                             b_tscale, c, c_dtype, workspace, stream);
  }
  return launch_gemm_simple(fmt, m, n, k, a_codes, a_scales, a_tscale, b_codes,
                            b_scales, b_tscale, c, c_dtype, stream);
}

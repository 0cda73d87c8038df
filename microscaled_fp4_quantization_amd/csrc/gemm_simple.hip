// W4A4 GEMM, reference-structure kernels for gfx950 (small or odd shapes).
//
// C[m, n] = sum_k deq(A)[m, k] * deq(B)[n, k]; A = activations [m, k],
// B = weights [n, k], both quantized along k.  W4A4 as on pimento.cloud
// "FP8, NVFP4 czy AWQ?", section "Dlaczego W8A8 i W4A16 to nie to samo?"
// (both operands 4-bit, products on low-precision matrix units).
//
// MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1 and one
// E8M0 scale per lane (= per row and 32-value block), exactly the MXFP4
// block structure.
// NVFP4: the E4M3 scale is not a power of two, so the block-scaled MFMA
// cannot apply it.  Instead each E2M1 value is multiplied by its E4M3 block
// scale in fp16 (v * sb has at most 6 significant bits and lies in
// [2^-10, 2688], so the fp16 product is exact) and the exact products go
// through v_mfma_f32_16x16x32_f16 with fp32 accumulation; the two FP32
// tensor scales are applied in the epilogue.
//
// Layout: one workgroup = 4 waves in a 2 x 2 arrangement, 32 x 32 of C per
// wave (2 x 2 MFMA tiles of 16 x 16).  Each lane loads its MFMA fragments
// straight from global memory (row r = lane % 16, k-group g = lane / 16);
// rows past m or n are clamped on load and skipped on store, k-groups past
// k load zeros.
#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWaveTile = 32;
constexpr int kBlockTile = 64;

__device__ __forceinline__ void store_c(void* c, int c_dtype, int64_t n, int64_t row,
                                        int64_t col, float v) {
  if (c_dtype == kInF32) {
    reinterpret_cast<float*>(c)[row * n + col] = v;
  } else {
    __bf16 b = (__bf16)v;
    reinterpret_cast<__bf16*>(c)[row * n + col] = b;
  }
}

__global__ __launch_bounds__(256) void gemm_mx_simple(
    int64_t m, int64_t n, int64_t k, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const uint8_t* __restrict__ b,
    const uint8_t* __restrict__ bs, void* __restrict__ c, int c_dtype) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * kBlockTile + (wave >> 1) * kWaveTile;
  const int64_t n0 = (int64_t)blockIdx.x * kBlockTile + (wave & 1) * kWaveTile;
  const int64_t kb = k / 32;           // scale bytes per row
  const int64_t kbytes = k / 2;
  int64_t arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int64_t ra = m0 + 16 * i + r, rb = n0 + 16 * i + r;
    arow[i] = ra < m ? ra : m - 1;
    brow[i] = rb < n ? rb : n - 1;
  }
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < k; k0 += 128) {
    const int64_t blk = k0 / 32 + g;   // this lane's 32-value block
    const bool kin = blk < kb;
    v8i fa[2], fb[2];
    int sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint4 wa = make_uint4(0u, 0u, 0u, 0u), wb = wa;
      int ca = 127, cb = 127;
      if (kin) {
        wa = *reinterpret_cast<const uint4*>(a + arow[i] * kbytes + blk * 16);
        wb = *reinterpret_cast<const uint4*>(b + brow[i] * kbytes + blk * 16);
        ca = as[arow[i] * kb + blk];
        cb = bs[brow[i] * kb + blk];
      }
      fa[i] = (v8i){(int)wa.x, (int)wa.y, (int)wa.z, (int)wa.w, 0, 0, 0, 0};
      fb[i] = (v8i){(int)wb.x, (int)wb.y, (int)wb.z, (int)wb.w, 0, 0, 0, 0};
      sa[i] = ca;
      sb[i] = cb;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fa[i], fb[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
  }
  // D layout: lane holds rows 4*(lane/16) + e, column lane % 16.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + 16 * i + 4 * g + e, col = n0 + 16 * j + r;
        if (row < m && col < n) store_c(c, c_dtype, n, row, col, acc[i][j][e]);
      }
}

// 8 E2M1 codes (one dword) times an fp16 block scale -> 8 exact fp16 values.
__device__ __forceinline__ v8h dequant8_f16(uint32_t w, _Float16 s) {
  const v2h sv = {s, s};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sv;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sv;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sv;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sv;
  return (v8h){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__global__ __launch_bounds__(256) void gemm_nv_simple(
    int64_t m, int64_t n, int64_t k, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const float* __restrict__ at,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs,
    const float* __restrict__ bt, void* __restrict__ c, int c_dtype) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * kBlockTile + (wave >> 1) * kWaveTile;
  const int64_t n0 = (int64_t)blockIdx.x * kBlockTile + (wave & 1) * kWaveTile;
  const int64_t kb = k / 16;
  const int64_t kbytes = k / 2;
  int64_t arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int64_t ra = m0 + 16 * i + r, rb = n0 + 16 * i + r;
    arow[i] = ra < m ? ra : m - 1;
    brow[i] = rb < n ? rb : n - 1;
  }
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < k; k0 += 32) {
    const int64_t kk = k0 + 8 * g;     // this lane's 8 values
    const bool kin = kk < k;
    v8h fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t wa = 0u, wb = 0u, ca = 0u, cb = 0u;
      if (kin) {
        wa = *reinterpret_cast<const uint32_t*>(a + arow[i] * kbytes + kk / 2);
        wb = *reinterpret_cast<const uint32_t*>(b + brow[i] * kbytes + kk / 2);
        ca = as[arow[i] * kb + kk / 16];
        cb = bs[brow[i] * kb + kk / 16];
      }
      fa[i] = dequant8_f16(wa, (_Float16)e4m3_decode(ca));
      fb[i] = dequant8_f16(wb, (_Float16)e4m3_decode(cb));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }
  const float ts = (*at) * (*bt);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + 16 * i + 4 * g + e, col = n0 + 16 * j + r;
        if (row < m && col < n) store_c(c, c_dtype, n, row, col, acc[i][j][e] * ts);
      }
}

}  // namespace

hipError_t launch_gemm_simple(int fmt, int64_t m, int64_t n, int64_t k,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_tscale, const uint8_t* b_codes,
                              const uint8_t* b_scales, const float* b_tscale,
                              void* c, int c_dtype, hipStream_t stream) {
  const dim3 grid((unsigned)((n + kBlockTile - 1) / kBlockTile),
                  (unsigned)((m + kBlockTile - 1) / kBlockTile));
  if (fmt == kFmtMX) {
    hipLaunchKernelGGL(gemm_mx_simple, grid, dim3(256), 0, stream, m, n, k,
                       a_codes, a_scales, b_codes, b_scales, c, c_dtype);
  } else {
    hipLaunchKernelGGL(gemm_nv_simple, grid, dim3(256), 0, stream, m, n, k,
                       a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale,
                       c, c_dtype);
  }
  return hipGetLastError();
}

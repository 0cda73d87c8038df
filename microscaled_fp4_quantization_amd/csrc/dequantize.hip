// FP4 dequantization kernel for gfx950: packed E2M1 codes + block scales
// (+ FP32 tensor scale) -> fp32 / bf16 / fp16 / FP8 E4M3.
//
// The FP8 E4M3 output is the form the hyper.ai story on the NVFP4 KV cache
// describes: cached K/V are dequantized to FP8 before attention.  Formats as
// in aisyndicate.ch "FP4 auf Blackwell" (section "Was NVFP4 von frueheren
// 4-Bit-Formaten unterscheidet") and pimento.cloud "FP8, NVFP4 czy AWQ?"
// (section "Czym roznia sie FP8, NVFP4, MXFP4 i AWQ?").
//
// NVFP4: y = fp32(fp32(v * E4M3(sb)) * s_t); the first product is exact (at
// most 6 significant bits), so y is the exact value rounded once.  MXFP4:
// y = v * 2^(c-127), exact.  Conversion: bf16 / fp16 round to nearest even;
// FP8 rounds to nearest even after a clamp to +-448 (the hardware conversion
// rounds correctly inside that range but returns NaN beyond it).
//
// Lane t owns chunk base + t of 8 elements: one dword of codes in, 8 values
// out (8 bytes FP8, 16 bytes bf16/fp16, 32 bytes fp32).
#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kChunksPerTrip = kThreads * kUnroll;
constexpr int kMaxGrid = 4096;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The fp32 value must exist before the narrowing: without the empty asm the
// compiler fuses "t * s_t then narrow" into one mixed-precision FMA, which
// rounds once instead of twice and turns -0 into +0.
__device__ __forceinline__ float materialize(float v) {
  __asm__ volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)materialize(a), y = (__bf16)materialize(b);
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  _Float16 x = (_Float16)materialize(a), y = (_Float16)materialize(b);
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ uint32_t pack_e4m3x4(const float* y) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_fmed3f(y[i], -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  return (uint32_t)w;
}

template <int FMT, int OUT>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, int64_t nchunks, void* __restrict__ out) {
  const float s_t = (FMT == kFmtNV) ? *tscale : 1.0f;
  for (int64_t base = (int64_t)blockIdx.x * kChunksPerTrip; base < nchunks;
       base += (int64_t)gridDim.x * kChunksPerTrip) {
    uint32_t w[kUnroll], sb[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = base + j * kThreads + threadIdx.x;
      w[j] = 0u;
      sb[j] = 0u;
      if (c < nchunks) {
        w[j] = __builtin_nontemporal_load(codes + c);
        sb[j] = scales[FMT == kFmtNV ? (c >> 1) : (c >> 2)];
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = base + j * kThreads + threadIdx.x;
      if (c >= nchunks) continue;
      float sv;
      if (FMT == kFmtNV) {
        sv = e4m3_decode_pos(sb[j] & 0x7Fu);
        if (sb[j] & 0x80u) sv = -sv;
      } else {
        sv = sb[j] ? as_f(sb[j] << 23) : as_f(0x00400000u);  // 2^(c-127); c = 0 is 2^-127
      }
      float y[8];
      const v2f p0 = e2m1_unpack2<0>(w[j]), p1 = e2m1_unpack2<1>(w[j]);
      const v2f p2 = e2m1_unpack2<2>(w[j]), p3 = e2m1_unpack2<3>(w[j]);
      y[0] = p0.x; y[1] = p0.y; y[2] = p1.x; y[3] = p1.y;
      y[4] = p2.x; y[5] = p2.y; y[6] = p3.x; y[7] = p3.y;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (FMT == kFmtNV) {
          const float t = y[i] * sv;   // exact
          y[i] = t * s_t;
        } else {
          y[i] = y[i] * sv;            // exact
        }
      }
      if (OUT == kInF32) {
        f32x4* o = reinterpret_cast<f32x4*>(out) + 2 * c;
        __builtin_nontemporal_store((f32x4){y[0], y[1], y[2], y[3]}, o);
        __builtin_nontemporal_store((f32x4){y[4], y[5], y[6], y[7]}, o + 1);
      } else if (OUT == kInBF16) {
        u32x4 o = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                   pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out) + c);
      } else if (OUT == kInF16) {
        u32x4 o = {pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3]),
                   pack_f16x2(y[4], y[5]), pack_f16x2(y[6], y[7])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out) + c);
      } else {
        u32x2 o = {pack_e4m3x4(y), pack_e4m3x4(y + 4)};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(out) + c);
      }
    }
  }
}

template <int FMT>
hipError_t launch_fmt(const uint8_t* codes, const uint8_t* scales,
                      const float* tscale, int64_t nchunks, void* out,
                      int out_dtype, hipStream_t stream) {
  const int64_t trips = (nchunks + kChunksPerTrip - 1) / kChunksPerTrip;
  const dim3 grid((unsigned)(trips < kMaxGrid ? trips : kMaxGrid));
  const uint32_t* c32 = reinterpret_cast<const uint32_t*>(codes);
  switch (out_dtype) {
    case kInF32:
      hipLaunchKernelGGL((dequantize_kernel<FMT, kInF32>), grid, dim3(kThreads), 0, stream, c32, scales, tscale, nchunks, out);
      break;
    case kInBF16:
      hipLaunchKernelGGL((dequantize_kernel<FMT, kInBF16>), grid, dim3(kThreads), 0, stream, c32, scales, tscale, nchunks, out);
      break;
    case kInF16:
      hipLaunchKernelGGL((dequantize_kernel<FMT, kInF16>), grid, dim3(kThreads), 0, stream, c32, scales, tscale, nchunks, out);
      break;
    default:
      hipLaunchKernelGGL((dequantize_kernel<FMT, kOutE4M3>), grid, dim3(kThreads), 0, stream, c32, scales, tscale, nchunks, out);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(int fmt, const uint8_t* codes,
                             const uint8_t* scales, const float* tscale,
                             int64_t n, void* out, int out_dtype,
                             hipStream_t stream) {
  const int64_t nchunks = n / 8;
  return fmt == kFmtNV
             ? launch_fmt<kFmtNV>(codes, scales, tscale, nchunks, out, out_dtype, stream)
             : launch_fmt<kFmtMX>(codes, scales, tscale, nchunks, out, out_dtype, stream);
}

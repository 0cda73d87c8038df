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
// Lane t owns chunks 2p and 2p + 1 (16 elements, one NVFP4 block, half an
// MXFP4 block): 8 bytes of codes and one scale byte in, 16 values out (16
// bytes FP8, 32 bytes bf16/fp16, 64 bytes fp32), so the wave instructions
// of the FP8 path read and write contiguous memory.
#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr int kUnrollP = 4;          // chunk pairs per thread per loop trip

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

// Chunk c (8 values, code word w, scale byte sbyte) -> out.
template <int FMT, int OUT>
__device__ __forceinline__ void dequant_chunk(uint32_t w, uint32_t sbyte, float s_t, int64_t c,
                                              void* __restrict__ out) {
  const float sv = block_scale_value<FMT == kFmtNV>(sbyte);
  float y[8];
  const v2f p0 = e2m1_unpack2<0>(w), p1 = e2m1_unpack2<1>(w);
  const v2f p2 = e2m1_unpack2<2>(w), p3 = e2m1_unpack2<3>(w);
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

// Chunk (code word w, scale byte sbyte) -> 8 FP8 E4M3 bytes.
template <int FMT>
__device__ __forceinline__ u32x2 dequant_e4m3(uint32_t w, uint32_t sbyte, float s_t) {
  const float sv = block_scale_value<FMT == kFmtNV>(sbyte);
  float y[8];
  const v2f p0 = e2m1_unpack2<0>(w), p1 = e2m1_unpack2<1>(w);
  const v2f p2 = e2m1_unpack2<2>(w), p3 = e2m1_unpack2<3>(w);
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
  return (u32x2){pack_e4m3x4(y), pack_e4m3x4(y + 4)};
}

// An odd last chunk goes alone.
template <int FMT, int OUT>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, int64_t nchunks, void* __restrict__ out) {
  const float s_t = (FMT == kFmtNV) ? *tscale : 1.0f;
  const int64_t npairs = nchunks >> 1;
  const u32x2* codes2 = reinterpret_cast<const u32x2*>(codes);
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnrollP; base < npairs;
       base += (int64_t)gridDim.x * kThreads * kUnrollP) {
    u32x2 w[kUnrollP];
    uint32_t sb[kUnrollP];
#pragma unroll
    for (int j = 0; j < kUnrollP; ++j) {
      const int64_t p = base + j * kThreads + threadIdx.x;
      w[j] = (u32x2){0u, 0u};
      sb[j] = 0u;
      if (p < npairs) {
        w[j] = __builtin_nontemporal_load(codes2 + p);
        sb[j] = scales[FMT == kFmtNV ? p : (p >> 1)];
      }
    }
#pragma unroll
    for (int j = 0; j < kUnrollP; ++j) {
      const int64_t p = base + j * kThreads + threadIdx.x;
      if (p >= npairs) continue;
      if (OUT == kOutE4M3) {
        const u32x2 a = dequant_e4m3<FMT>(w[j][0], sb[j], s_t);
        const u32x2 b = dequant_e4m3<FMT>(w[j][1], sb[j], s_t);
        __builtin_nontemporal_store((u32x4){a.x, a.y, b.x, b.y}, reinterpret_cast<u32x4*>(out) + p);
      } else {
        dequant_chunk<FMT, OUT>(w[j][0], sb[j], s_t, 2 * p, out);
        dequant_chunk<FMT, OUT>(w[j][1], sb[j], s_t, 2 * p + 1, out);
      }
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && (nchunks & 1)) {
    const int64_t c = nchunks - 1;
    dequant_chunk<FMT, OUT>(codes[c], scales[FMT == kFmtNV ? (c >> 1) : (c >> 2)], s_t, c, out);
  }
}

template <int FMT>
hipError_t launch_fmt(const uint8_t* codes, const uint8_t* scales,
                      const float* tscale, int64_t nchunks, void* out,
                      int out_dtype, hipStream_t stream) {
  // one trip per workgroup (a grid-stride cap cost bandwidth on long tensors)
  const int64_t trips = (nchunks / 2 + kThreads * kUnrollP - 1) / (kThreads * kUnrollP);
  const dim3 grid((unsigned)(trips < 1 ? 1 : trips));
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

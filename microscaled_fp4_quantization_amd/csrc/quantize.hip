// Block-scaled FP4 quantization kernels for gfx950: NVFP4 (16-element blocks,
// E4M3 scale, FP32 tensor scale) and MXFP4 (32-element blocks, E8M0 scale),
// optionally preceded by the blockwise Hadamard rotation of MR-GPTQ.
//
// Formats: aisyndicate.ch "FP4 auf Blackwell", section "Was NVFP4 von
// frueheren 4-Bit-Formaten unterscheidet"; pimento.cloud "FP8, NVFP4 czy
// AWQ?", section "Czym roznia sie FP8, NVFP4, MXFP4 i AWQ?".  Rotation:
// hyper.ai, paper 2509.23202, Abstract (blockwise Hadamard transforms,
// computed online for activations).
//
// Work decomposition.  A [rows, k] tensor with k a multiple of the block size
// is a flat run of blocks.  The bulk kernels (blocks_kernel and its max pass)
// give each lane one whole block: its 16 or 32 contiguous values in 16-byte
// loads, the rotation's butterfly stages inside the lane, the block's scale
// arithmetic once per block, its codes as one 8- or 16-byte store and its
// scale byte.  The kernels for short inputs (the single-workgroup
// compute-mode kernel for decode activations, the KV append, the rotation
// alone) cut the elements into chunks of 8 instead: lane t of a wave owns
// chunk base + t, an NVFP4 block is a lane pair (t, t^1), an MXFP4 block a
// lane quad, and the block max and the cross-lane butterfly stages use DPP
// quad permutes.  Both orders of arithmetic are the same, so both give the
// same bits.
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;        // 4 waves of 64
constexpr int kMaxPartials = 1024;   // amax partials (workspace floats)
static_assert(kMaxPartials % kThreads == 0, "partials per thread");

typedef uint32_t u32x4e __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2e __attribute__((ext_vector_type(2)));
typedef float f32x4e __attribute__((ext_vector_type(4)));

// 8 elements of chunk c widened to fp32 (exact); zeros when !valid.
template <int DT>
__device__ __forceinline__ void load_chunk(const void* __restrict__ x, int64_t c,
                                           bool valid, float v[8]) {
  if (DT == kInF32) {
    // the input is read once: nontemporal loads
    const f32x4e* p = reinterpret_cast<const f32x4e*>(x) + 2 * c;
    f32x4e a = {0.f, 0.f, 0.f, 0.f}, b = a;
    if (valid) { a = __builtin_nontemporal_load(p); b = __builtin_nontemporal_load(p + 1); }
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const u32x4e* p = reinterpret_cast<const u32x4e*>(x) + c;
    u32x4e w = {0u, 0u, 0u, 0u};
    if (valid) w = __builtin_nontemporal_load(p);
    const uint32_t ws[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (DT == kInBF16) {
        v[2 * i] = bf16_lo(ws[i]);
        v[2 * i + 1] = bf16_hi(ws[i]);
      } else {
        v2h h = __builtin_bit_cast(v2h, ws[i]);
        v[2 * i] = (float)h.x;
        v[2 * i + 1] = (float)h.y;
      }
    }
  }
}

// In-place blockwise Hadamard of the 8 values a lane holds, for blocks of B
// (16: lane pair, 32: lane quad).  Butterfly stages h = 1, 2, 4 inside the
// lane, h = 8 with lane ^ 1, h = 16 with lane ^ 2; each stage turns the pair
// (lower, upper) into (lower + upper, lower - upper) in fp32.  Then one
// multiply by fp32(1/sqrt(B)).
template <int B>
__device__ __forceinline__ void fwht_chunk(float v[8], int lane) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2) {
#pragma unroll
    for (int s = 0; s < 8; s += 2 * h) {
#pragma unroll
      for (int j = s; j < s + h; ++j) {
        float u = v[j], w = v[j + h];
        v[j] = u + w;
        v[j + h] = u - w;
      }
    }
  }
  const bool up1 = (lane & 1) != 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float p = dpp_f<kDppXor1>(v[j]);
    v[j] = up1 ? (p - v[j]) : (v[j] + p);
  }
  if (B == 32) {
    const bool up2 = (lane & 2) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float p = dpp_f<kDppXor2>(v[j]);
      v[j] = up2 ? (p - v[j]) : (v[j] + p);
    }
  }
  const float cb = (B == 16) ? 0.25f : __uint_as_float(0x3E3504F3u);  // fp32(1/sqrt(32))
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = v[j] * cb;
}

__device__ __forceinline__ float amax8(const float v[8]) {
  float a = fmaxf(fabsf(v[0]), fabsf(v[1]));
  a = fmaxf(a, fmaxf(fabsf(v[2]), fabsf(v[3])));
  a = fmaxf(a, fmaxf(fabsf(v[4]), fabsf(v[5])));
  return fmaxf(a, fmaxf(fabsf(v[6]), fabsf(v[7])));
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  return m;
}

// Max over a workgroup of NT threads; every thread gets the result.
template <int NT = kThreads>
__device__ __forceinline__ float block_max(float m) {
  __shared__ float red[NT / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  // LDS only: barriers that leave the wave's global loads in flight
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __asm__ volatile("s_barrier" ::: "memory");
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  __asm__ volatile("s_barrier" ::: "memory");
  return r;
}

// One chunk (8 values, already rotated when the rotation applies) of lane
// `lane` to codes and, from the first lane of its block, the scale byte.
// NVFP4: s_t is the tensor scale and d = 6 s_t.
template <int FMT>
__device__ __forceinline__ void quantize_chunk(const float v[8], int lane, float s_t, float d,
                                               int64_t c, bool valid, uint32_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales) {
  float a = amax8(v);
  a = fmaxf(a, dpp_f<kDppXor1>(a));
  float r;
  uint32_t sbyte;
  if (FMT == kFmtNV) {
    const float u = a / d;
    sbyte = e4m3_encode_pos(u);
    const float S = e4m3_decode_pos(sbyte) * s_t;
    r = 1.0f / S;
    // S == 0 (zero block) or an overflowing reciprocal: sign bits only.
    if (!(S != 0.0f && r < __builtin_inff())) r = 0.0f;
  } else {
    a = fmaxf(a, dpp_f<kDppXor2>(a));
    const int kx = mx_block_exponent(a);
    sbyte = (uint32_t)(kx + 127);
    r = as_f((uint32_t)(127 - kx) << 23);  // 2^-k, a normal float for k in [-127, 126]
  }
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = v[i] * r;
  uint32_t w = e2m1_pack2<0>(0u, q[0], q[1]);
  w = e2m1_pack2<1>(w, q[2], q[3]);
  w = e2m1_pack2<2>(w, q[4], q[5]);
  w = e2m1_pack2<3>(w, q[6], q[7]);
  if (valid) {
    __builtin_nontemporal_store(w, codes + c);
    if (FMT == kFmtNV) {
      if ((lane & 1) == 0) scales[c >> 1] = (uint8_t)sbyte;
    } else {
      if ((lane & 3) == 0) scales[c >> 2] = (uint8_t)sbyte;
    }
  }
}

// ---- block-per-lane kernels ----------------------------------------------
// The bulk quantize path: lane l of a wave owns one whole block (BS = 16
// NVFP4 or 32 MXFP4 values, BS * element-size bytes of contiguous input),
// so the rotation's butterfly stages all run inside the lane and the block's
// scale arithmetic (two IEEE divisions for NVFP4) runs once per block.  The
// arithmetic, and its order, is that of quantize_chunk / fwht_chunk.

// 16-byte pieces of one block of BS values of type DT
template <int DT, int BS>
constexpr int block_pieces() { return BS * (DT == kInF32 ? 4 : 2) / 16; }

// The raw pieces of block b.  A block past the end loads block 0 instead (it
// exists whenever the kernel runs): counted once more in a maximum it changes
// nothing, and it is never stored.  No branch and no select around the
// loads, so a wait for an earlier load does not wait for these.
template <int DT, int BS, bool NT>
__device__ __forceinline__ void load_block(const void* __restrict__ x, int64_t b, bool valid,
                                           u32x4e (&w)[block_pieces<DT, BS>()]) {
  constexpr int L = block_pieces<DT, BS>();
  const u32x4e* p = reinterpret_cast<const u32x4e*>(x) + (valid ? b : 0) * L;
#pragma unroll
  for (int i = 0; i < L; ++i) w[i] = NT ? __builtin_nontemporal_load(p + i) : p[i];
}

// The pieces widened exactly to fp32.
template <int DT, int BS>
__device__ __forceinline__ void widen_block(const u32x4e (&w)[block_pieces<DT, BS>()], float v[BS]) {
  constexpr int L = block_pieces<DT, BS>();
#pragma unroll
  for (int i = 0; i < L; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (DT == kInF32) {
        v[4 * i + j] = as_f(w[i][j]);
      } else if (DT == kInBF16) {
        v[8 * i + 2 * j] = bf16_lo(w[i][j]);
        v[8 * i + 2 * j + 1] = bf16_hi(w[i][j]);
      } else {
        // through a scalar: clang's bit cast of a vector-element lvalue reads
        // the vector's first element whatever the index
        const uint32_t wd = w[i][j];
        const v2h h = __builtin_bit_cast(v2h, wd);
        v[8 * i + 2 * j] = (float)h.x;
        v[8 * i + 2 * j + 1] = (float)h.y;
      }
    }
  }
}

// Block b widened, zeros past the end (the given-scale path: nothing waits
// between its loads, and this form streams faster there).
template <int DT, int BS>
__device__ __forceinline__ void load_widen_block(const void* __restrict__ x, int64_t b, bool valid,
                                                 float v[BS]) {
  constexpr int L = block_pieces<DT, BS>();
  const u32x4e* p = reinterpret_cast<const u32x4e*>(x) + b * L;
  u32x4e w[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    w[i] = (u32x4e){0u, 0u, 0u, 0u};
    if (valid) w[i] = p[i];
  }
  widen_block<DT, BS>(w, v);
}

// Blockwise Hadamard of one whole block in the lane: stages h = 1, 2, 4, ...,
// BS/2, each pair (j, j + h) -> (lower + upper, lower - upper), then one
// multiply by fp32(1/sqrt(BS)).
template <int BS>
__device__ __forceinline__ void fwht_block(float v[BS]) {
#pragma unroll
  for (int h = 1; h < BS; h *= 2) {
#pragma unroll
    for (int s = 0; s < BS; s += 2 * h) {
#pragma unroll
      for (int j = s; j < s + h; ++j) {
        const float u = v[j], w = v[j + h];
        v[j] = u + w;
        v[j + h] = u - w;
      }
    }
  }
  const float cb = (BS == 16) ? 0.25f : __uint_as_float(0x3E3504F3u);  // fp32(1/sqrt(32))
#pragma unroll
  for (int j = 0; j < BS; ++j) v[j] = v[j] * cb;
}

template <int BS>
__device__ __forceinline__ float amax_block(const float v[BS]) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < BS; j += 2) a = fmaxf(a, fmaxf(fabsf(v[j]), fabsf(v[j + 1])));
  return a;
}

// One block to its BS/8 code dwords and scale byte (arithmetic as in
// quantize_chunk).
template <int FMT, int BS>
__device__ __forceinline__ void quantize_block(const float v[BS], float s_t, float d,
                                               uint32_t w[BS / 8], uint32_t& sbyte) {
  const float a = amax_block<BS>(v);
  float r;
  if (FMT == kFmtNV) {
    const float u = a / d;
    sbyte = e4m3_encode_pos(u);
    const float S = e4m3_decode_pos(sbyte) * s_t;
    r = 1.0f / S;
    // S == 0 (zero block) or an overflowing reciprocal: sign bits only.
    if (!(S != 0.0f && r < __builtin_inff())) r = 0.0f;
  } else {
    const int kx = mx_block_exponent(a);
    sbyte = (uint32_t)(kx + 127);
    r = as_f((uint32_t)(127 - kx) << 23);  // 2^-k, a normal float for k in [-127, 126]
  }
#pragma unroll
  for (int i = 0; i < BS / 8; ++i) {
    const float* q = v + 8 * i;
    uint32_t t = e2m1_pack2<0>(0u, q[0] * r, q[1] * r);
    t = e2m1_pack2<1>(t, q[2] * r, q[3] * r);
    t = e2m1_pack2<2>(t, q[4] * r, q[5] * r);
    w[i] = e2m1_pack2<3>(t, q[6] * r, q[7] * r);
  }
}

template <int FMT>
constexpr int blocks_per_thread() { return FMT == kFmtNV ? 4 : 2; }

// Pass 1 of dynamic NVFP4 scaling: per-workgroup max |x| (of the rotated
// values when HAD > 0) into partials[blockIdx.x].  The same block -> thread
// mapping as blocks_kernel, and ordinary (cached) loads, so that the second
// pass finds much of x in the caches of the same XCD.
template <int DT, int HAD>
__global__ __launch_bounds__(kThreads) void amax_blocks_kernel(const void* __restrict__ x,
                                                               int64_t nblocks,
                                                               float* __restrict__ partials) {
  constexpr int BS = 16, U = blocks_per_thread<kFmtNV>();
  float m = 0.0f;
  // one trip per workgroup unless the tensor needs more than kMaxPartials
  for (int64_t base = (int64_t)blockIdx.x * (U * kThreads) + threadIdx.x; base < nblocks + threadIdx.x;
       base += (int64_t)gridDim.x * (U * kThreads)) {
    u32x4e w[U][block_pieces<DT, BS>()];
#pragma unroll
    for (int j = 0; j < U; ++j) load_block<DT, BS, false>(x, base + j * kThreads, base + j * kThreads < nblocks, w[j]);
    __builtin_amdgcn_sched_barrier(0);        // every load issued before the first wait
    float v[U][BS];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      widen_block<DT, BS>(w[j], v[j]);
      if (HAD) fwht_block<BS>(v[j]);
      m = fmaxf(m, amax_block<BS>(v[j]));
    }
  }
  m = block_max(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Quantize, one block per lane, U blocks per thread.  COMPUTE (NVFP4):
// reduce the npartials maxima of amax_blocks_kernel to s_t (every workgroup,
// redundantly) and let workgroup 0 publish it; otherwise read s_t.
template <int FMT, int DT, int HAD, bool COMPUTE>
__global__ __launch_bounds__(kThreads) void blocks_kernel(
    const void* __restrict__ x, int64_t nblocks, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tscale, const float* __restrict__ partials,
    int npartials) {
  constexpr int BS = FMT == kFmtNV ? 16 : 32, U = blocks_per_thread<FMT>();
  const int64_t base = (int64_t)blockIdx.x * (U * kThreads) + threadIdx.x;
  // the partial maxima first, all in flight at once: loads return in order,
  // and queued behind the block loads they would hold the whole workgroup up
  // for one more trip
  constexpr int PP = (FMT == kFmtNV && COMPUTE) ? kMaxPartials / kThreads : 1;
  float pv[PP];
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    pv[i] = (FMT == kFmtNV && COMPUTE && idx < npartials) ? partials[idx] : 0.0f;
  }
  // given scale: cached loads (a lane's two 16-byte pieces share lines with
  // its neighbours' and are requested by two instructions)
  // COMPUTE: nontemporal loads (x is read a second time), every one issued
  // before the first wait (the partial maxima come first); widened later
  u32x4e raw[U][COMPUTE ? block_pieces<DT, BS>() : 1];
  float vg[U][COMPUTE ? 1 : BS];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t b = base + j * kThreads;
    if constexpr (COMPUTE) load_block<DT, BS, true>(x, b, b < nblocks, raw[j]);
    else load_widen_block<DT, BS>(x, b, b < nblocks, vg[j]);
  }
  if (COMPUTE) __builtin_amdgcn_sched_barrier(0);
  float s_t = 1.0f, d = 6.0f;
  if (FMT == kFmtNV) {
    if (COMPUTE) {
      float m = pv[0];
#pragma unroll
      for (int i = 1; i < PP; ++i) m = fmaxf(m, pv[i]);
      const float A = block_max(m);
      s_t = A / 2688.0f;                       // 6 * 448
      if (s_t == 0.0f) s_t = 1.0f;
      if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = s_t;
    } else {
      s_t = *tscale;
    }
    d = 6.0f * s_t;
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t b = base + j * kThreads;
    float v[BS];
    if constexpr (COMPUTE) {
      widen_block<DT, BS>(raw[j], v);
    } else {
#pragma unroll
      for (int e = 0; e < BS; ++e) v[e] = vg[j][e];
    }
    if (HAD) fwht_block<BS>(v);
    uint32_t w[BS / 8], sbyte;
    quantize_block<FMT, BS>(v, s_t, d, w, sbyte);
    if (b < nblocks) {
      if (BS == 16) {
        __builtin_nontemporal_store(((u32x2e){w[0], w[1 % (BS / 8)]}),
                                    reinterpret_cast<u32x2e*>(codes) + b);
      } else {
        __builtin_nontemporal_store(((u32x4e){w[0], w[1 % (BS / 8)], w[2 % (BS / 8)], w[3 % (BS / 8)]}),
                                    reinterpret_cast<u32x4e*>(codes) + b);
      }
      scales[b] = (uint8_t)sbyte;
    }
  }
}

// KV cache append (hyper.ai story on the NVFP4 KV cache: new K/V vectors are
// written into the cache in 4-bit form).  The rows of x [batch, heads,
// t_new, k] are quantized exactly as quantize_kernel quantizes them (NVFP4
// with the given tensor scale) and row (b, h, i) is stored at position
// positions[b] + i of the [batch, heads, t_max, ...] cache; a position
// outside [0, t_max) stores nothing.  k is a multiple of 16 (32 for
// MXFP4), so cpr = k / 8 keeps a block's lane pair (quad) and the parity of
// the chunk index from source to destination.
template <int FMT, int DT>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    const void* __restrict__ x, uint32_t nchunks, uint32_t cpr, uint32_t t_new, uint32_t heads,
    const int32_t* __restrict__ positions, int64_t t_max, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, const float* __restrict__ tscale) {
  // one chunk per thread: an append is a few rows, so the grid, not a loop,
  // covers it (32-bit index arithmetic: fewer than 2^31 chunks per call)
  const int lane = threadIdx.x & 63;
  float s_t = 1.0f, d = 6.0f;
  if (FMT == kFmtNV) {
    s_t = *tscale;
    d = 6.0f * s_t;
  }
  const uint32_t c = blockIdx.x * (uint32_t)kThreads + threadIdx.x;
  float v[8];
  load_chunk<DT>(x, c, c < nchunks, v);
  int64_t cdst = 0;
  bool ok = false;
  if (c < nchunks) {
    const uint32_t row = c / cpr, cr = c - row * cpr;
    const uint32_t bh = row / t_new, i = row - bh * t_new;
    const int64_t p = (int64_t)positions[bh / heads] + i;
    ok = p >= 0 && p < t_max;
    cdst = ((int64_t)bh * t_max + (ok ? p : 0)) * cpr + cr;
  }
  quantize_chunk<FMT>(v, lane, s_t, d, cdst, ok, codes, scales);
}

// Blockwise Hadamard rotation alone (HAD = 16 or 32; 0 copies), fp32
// arithmetic exactly as in the fused quantizer, widened to fp64: the
// rotated weights and calibration activations of GPTQ.
template <int DT, int HAD>
__global__ __launch_bounds__(kThreads) void rotate_f64_kernel(const void* __restrict__ x,
                                                              int64_t nchunks,
                                                              double* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  float v[8];
  load_chunk<DT>(x, c, c < nchunks, v);
  if (HAD) fwht_chunk<HAD>(v, lane);
  if (c < nchunks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[8 * c + i] = (double)v[i];
  }
}

// NVFP4 with the tensor scale computed from the data, for small tensors
// (decode activations): one workgroup holds the whole tensor in registers,
// reduces its max |x| and quantizes, in a single launch instead of two.
constexpr int kSmallThreads = 1024;
constexpr int kSmallPer = 4;                                  // chunks per thread
constexpr int64_t kSmallChunks = (int64_t)kSmallThreads * kSmallPer;   // 32 Ki values

template <int DT, int HAD>
__global__ __launch_bounds__(kSmallThreads) void quantize_small_kernel(
    const void* __restrict__ x, int64_t nchunks, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tscale) {
  const int lane = threadIdx.x & 63;
  float v[kSmallPer][8];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kSmallPer; ++j) {
    // chunk j * 1024 + tid: lane t of a wave still owns chunk = t (mod 64)
    const int64_t c = (int64_t)j * kSmallThreads + threadIdx.x;
    load_chunk<DT>(x, c, c < nchunks, v[j]);
    if (HAD) fwht_chunk<HAD>(v[j], lane);
    m = fmaxf(m, amax8(v[j]));
  }
  const float A = block_max<kSmallThreads>(m);
  float s_t = A / 2688.0f;                     // 6 * 448
  if (s_t == 0.0f) s_t = 1.0f;
  if (threadIdx.x == 0) *tscale = s_t;
  const float d = 6.0f * s_t;
#pragma unroll
  for (int j = 0; j < kSmallPer; ++j) {
    const int64_t c = (int64_t)j * kSmallThreads + threadIdx.x;
    quantize_chunk<kFmtNV>(v[j], lane, s_t, d, c, c < nchunks, codes, scales);
  }
}

// NVFP4 with the block scale of least squared error (aisyndicate.ch "FP4 auf
// Blackwell", section "Was NVFP4 von frueheren 4-Bit-Formaten
// unterscheidet": the E4M3 block scale is the factor that minimizes the mean
// squared error over the block's 16 values).  A thread owns one block and
// tries every positive finite E4M3 byte, 1 .. 126, in ascending order: each
// quantizes the block as quantize_chunk does for that byte, its error
// sum_i (x_i - v_i S_b)^2 is accumulated in fp64 in element order (v_i S_b is
// exact in fp64, every other step rounds once), and only a strictly smaller
// error replaces the best, so ties keep the smaller scale.  A block whose max
// |x| is 0 keeps byte 0 and the sign bits, as in quantize_chunk.  The search
// is compute-bound (about 10^4 fp64 operations per block); it is meant for
// weights quantized once.
constexpr int kMseThreads = 256;

template <int DT, bool COMPUTE>
__global__ __launch_bounds__(kMseThreads) void quantize_mse_kernel(
    const void* __restrict__ x, int64_t nblocks, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tscale,
    const float* __restrict__ partials, int npartials) {
  float s_t;
  if (COMPUTE) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < npartials; i += kMseThreads) m = fmaxf(m, partials[i]);
    const float A = block_max<kMseThreads>(m);
    s_t = A / 2688.0f;                         // 6 * 448
    if (s_t == 0.0f) s_t = 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = s_t;
  } else {
    s_t = *tscale;
  }
  const int64_t b = (int64_t)blockIdx.x * kMseThreads + threadIdx.x;
  const bool valid = b < nblocks;
  float v[16];
  load_chunk<DT>(x, 2 * b, valid, v);
  load_chunk<DT>(x, 2 * b + 1, valid, v + 8);
  const float a = fmaxf(amax8(v), amax8(v + 8));

  // byte 0 / sign bits for a zero block (and the start of the search)
  uint32_t best_c = 0;
  uint32_t best_w0 = e2m1_pack2<3>(e2m1_pack2<2>(e2m1_pack2<1>(e2m1_pack2<0>(0u, v[0] * 0.0f, v[1] * 0.0f),
                                                              v[2] * 0.0f, v[3] * 0.0f),
                                                 v[4] * 0.0f, v[5] * 0.0f),
                                    v[6] * 0.0f, v[7] * 0.0f);
  uint32_t best_w1 = e2m1_pack2<3>(e2m1_pack2<2>(e2m1_pack2<1>(e2m1_pack2<0>(0u, v[8] * 0.0f, v[9] * 0.0f),
                                                              v[10] * 0.0f, v[11] * 0.0f),
                                                 v[12] * 0.0f, v[13] * 0.0f),
                                    v[14] * 0.0f, v[15] * 0.0f);
  if (a != 0.0f) {
    double best = __builtin_inf();
    for (uint32_t c = 1; c < 127; ++c) {
      const float S = e4m3_decode_pos(c) * s_t;
      const float r = 1.0f / S;
      if (!(S != 0.0f && r < __builtin_inff())) continue;     // uniform
      float q[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = v[i] * r;
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t t = e2m1_pack2<0>(0u, q[8 * h], q[8 * h + 1]);
        t = e2m1_pack2<1>(t, q[8 * h + 2], q[8 * h + 3]);
        t = e2m1_pack2<2>(t, q[8 * h + 4], q[8 * h + 5]);
        w[h] = e2m1_pack2<3>(t, q[8 * h + 6], q[8 * h + 7]);
      }
      const double Sd = (double)S;
      double err = 0.0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v2f p0 = e2m1_unpack2<0>(w[h]), p1 = e2m1_unpack2<1>(w[h]);
        const v2f p2 = e2m1_unpack2<2>(w[h]), p3 = e2m1_unpack2<3>(w[h]);
        const float dv[8] = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // v - dv S rounded once: dv S is exact in fp64 (at most 2 + 24
          // significant bits), so the fused form gives the same bits as the
          // product followed by the subtraction
          const double d = __builtin_fma(-(double)dv[i], Sd, (double)v[8 * h + i]);
          err = err + d * d;
        }
      }
      if (err < best) {
        best = err;
        best_c = c;
        best_w0 = w[0];
        best_w1 = w[1];
      }
    }
  }
  if (valid) {
    codes[b] = make_uint2(best_w0, best_w1);
    scales[b] = (uint8_t)best_c;
  }
}

template <int DT>
hipError_t launch_mse_typed(const void* x, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                            float* tscale, bool compute, void* workspace, hipStream_t stream) {
  const int grid = (int)((nblocks + kMseThreads - 1) / kMseThreads);
  uint2* codes64 = reinterpret_cast<uint2*>(codes);
  if (compute) {
    const int64_t per_wg = (int64_t)blocks_per_thread<kFmtNV>() * kThreads;
    const int64_t trips = (nblocks + per_wg - 1) / per_wg;
    const int g = (int)(trips < kMaxPartials ? trips : kMaxPartials);
    float* partials = reinterpret_cast<float*>(workspace);
    hipLaunchKernelGGL((amax_blocks_kernel<DT, 0>), dim3(g), dim3(kThreads), 0, stream, x, nblocks,
                       partials);
    hipLaunchKernelGGL((quantize_mse_kernel<DT, true>), dim3(grid), dim3(kMseThreads), 0, stream, x,
                       nblocks, codes64, scales, tscale, (const float*)partials, g);
  } else {
    hipLaunchKernelGGL((quantize_mse_kernel<DT, false>), dim3(grid), dim3(kMseThreads), 0, stream, x,
                       nblocks, codes64, scales, tscale, (const float*)nullptr, 0);
  }
  return hipGetLastError();
}

template <int FMT, int DT, int HAD>
hipError_t launch_typed(const void* x, int64_t nchunks, uint8_t* codes,
                        uint8_t* scales, float* tscale, bool compute,
                        void* workspace, hipStream_t stream) {
  constexpr int BS = FMT == kFmtNV ? 16 : 32;
  const int64_t nblocks = nchunks / (BS / 8);
  const int64_t per_wg = (int64_t)blocks_per_thread<FMT>() * kThreads;
  const int64_t grid = (nblocks + per_wg - 1) / per_wg;      // at most 2^30 / 4 workgroups
  if (FMT == kFmtNV && compute && nchunks <= kSmallChunks) {
    hipLaunchKernelGGL((quantize_small_kernel<DT, HAD>), dim3(1), dim3(kSmallThreads), 0, stream,
                       x, nchunks, reinterpret_cast<uint32_t*>(codes), scales, tscale);
  } else if (FMT == kFmtNV && compute) {
    float* partials = reinterpret_cast<float*>(workspace);
    const int g = (int)(grid < kMaxPartials ? grid : kMaxPartials);
    hipLaunchKernelGGL((amax_blocks_kernel<DT, HAD>), dim3(g), dim3(kThreads), 0, stream, x, nblocks,
                       partials);
    hipLaunchKernelGGL((blocks_kernel<FMT, DT, HAD, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       stream, x, nblocks, codes, scales, tscale, (const float*)partials, g);
  } else {
    hipLaunchKernelGGL((blocks_kernel<FMT, DT, HAD, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                       stream, x, nblocks, codes, scales, tscale, (const float*)nullptr, 0);
  }
  return hipGetLastError();
}

template <int FMT, int HAD>
hipError_t launch_dtype(int dtype, const void* x, int64_t nchunks, uint8_t* codes,
                        uint8_t* scales, float* tscale, bool compute,
                        void* workspace, hipStream_t stream) {
  switch (dtype) {
    case kInF32:
      return launch_typed<FMT, kInF32, HAD>(x, nchunks, codes, scales, tscale, compute, workspace, stream);
    case kInBF16:
      return launch_typed<FMT, kInBF16, HAD>(x, nchunks, codes, scales, tscale, compute, workspace, stream);
    default:
      return launch_typed<FMT, kInF16, HAD>(x, nchunks, codes, scales, tscale, compute, workspace, stream);
  }
}

}  // namespace

// Scratch of fp4_quantize_noalloc: the partial maxima of the compute-mode
// max pass (kMaxPartials floats; the pass never writes more, whatever the
// tensor size), in device memory the library owns instead of a caller
// workspace.  Each device holds its own copy at its own address, looked up
// once per device; nothing in it needs to start at zero (every partial is
// written before it is read).
static __device__ __align__(256) float scratch[kMaxPartials];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t quantize_static_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    // the array's name is a host-side stand-in: only this address may be
    // handed to kernels
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

size_t quantize_workspace_bytes(int fmt, bool compute) {
  // the partial maxima of the tensor amax pass
  return (fmt == kFmtNV && compute) ? kMaxPartials * sizeof(float) : 0;
}

hipError_t launch_quantize(int fmt, bool hadamard, const void* x, int dtype,
                           int64_t n, uint8_t* codes, uint8_t* scales,
                           float* tscale, bool compute, void* workspace,
                           hipStream_t stream) {
  const int64_t nchunks = n / 8;
  if (fmt == kFmtNV) {
    return hadamard ? launch_dtype<kFmtNV, 16>(dtype, x, nchunks, codes, scales, tscale, compute, workspace, stream)
                    : launch_dtype<kFmtNV, 0>(dtype, x, nchunks, codes, scales, tscale, compute, workspace, stream);
  }
  return hadamard ? launch_dtype<kFmtMX, 32>(dtype, x, nchunks, codes, scales, tscale, false, workspace, stream)
                  : launch_dtype<kFmtMX, 0>(dtype, x, nchunks, codes, scales, tscale, false, workspace, stream);
}

hipError_t launch_kv_append(int fmt, const void* x, int dtype, int64_t batch, int64_t heads,
                            int64_t t_new, int64_t k, const int32_t* positions, int64_t t_max,
                            uint8_t* codes, uint8_t* scales, const float* tscale,
                            hipStream_t stream) {
  const uint32_t nchunks = (uint32_t)(batch * heads * t_new * (k / 8));
  const uint32_t grid = (nchunks + kThreads - 1) / kThreads;
  uint32_t* c32 = reinterpret_cast<uint32_t*>(codes);
  const uint32_t cpr = (uint32_t)(k / 8);
#define FP4_KV_APPEND(F, D)                                                                  \
  hipLaunchKernelGGL((kv_append_kernel<F, D>), dim3(grid), dim3(kThreads), 0, stream, x,     \
                     nchunks, cpr, (uint32_t)t_new, (uint32_t)heads, positions, t_max, c32,  \
                     scales, tscale)
  if (fmt == kFmtNV) {
    if (dtype == kInF32) FP4_KV_APPEND(kFmtNV, kInF32);
    else if (dtype == kInBF16) FP4_KV_APPEND(kFmtNV, kInBF16);
    else FP4_KV_APPEND(kFmtNV, kInF16);
  } else {
    if (dtype == kInF32) FP4_KV_APPEND(kFmtMX, kInF32);
    else if (dtype == kInBF16) FP4_KV_APPEND(kFmtMX, kInBF16);
    else FP4_KV_APPEND(kFmtMX, kInF16);
  }
#undef FP4_KV_APPEND
  return hipGetLastError();
}

hipError_t launch_rotate_f64(const void* x, int dtype, int64_t n, int hadamard, double* out,
                             hipStream_t stream) {
  const int64_t nchunks = n / 8;
  const dim3 grid((unsigned)((nchunks + kThreads - 1) / kThreads));
#define FP4_ROT(D, H) \
  hipLaunchKernelGGL((rotate_f64_kernel<D, H>), grid, dim3(kThreads), 0, stream, x, nchunks, out)
#define FP4_ROT_H(D)                    \
  if (hadamard == 16) FP4_ROT(D, 16);   \
  else if (hadamard == 32) FP4_ROT(D, 32); \
  else FP4_ROT(D, 0)
  if (dtype == kInF32) { FP4_ROT_H(kInF32); }
  else if (dtype == kInBF16) { FP4_ROT_H(kInBF16); }
  else { FP4_ROT_H(kInF16); }
#undef FP4_ROT_H
#undef FP4_ROT
  return hipGetLastError();
}

hipError_t launch_quantize_mse(const void* x, int dtype, int64_t n, uint8_t* codes,
                               uint8_t* scales, float* tscale, bool compute, void* workspace,
                               hipStream_t stream) {
  const int64_t nblocks = n / 16;
  switch (dtype) {
    case kInF32:
      return launch_mse_typed<kInF32>(x, nblocks, codes, scales, tscale, compute, workspace, stream);
    case kInBF16:
      return launch_mse_typed<kInBF16>(x, nblocks, codes, scales, tscale, compute, workspace, stream);
    default:
      return launch_mse_typed<kInF16>(x, nblocks, codes, scales, tscale, compute, workspace, stream);
  }
}

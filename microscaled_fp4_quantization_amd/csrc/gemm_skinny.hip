// W4A4 GEMM for few activation rows (m <= 16, the decode shape): a weight
// stream.  C[m, n] = sum_k deq(X)[m, k] deq(W)[n, k].
//
// pimento.cloud "FP8, NVFP4 czy AWQ?", section "Dlaczego W8A8 i W4A16 to nie
// to samo?": token-by-token generation is bound by reading the weights, so
// this kernel is built to stream W once at full HBM rate.
//
// One workgroup owns 16 weight rows; its 4 waves split k into quarters and
// add their partial tiles through LDS at the end.  Lane l works on weight
// row n0 + l % 16 and activation row l % 16 (zero when >= m); per trip it
// loads 16 bytes (32 values) of its weight row and the same 32 positions of
// its activation row.  Because a dot product may visit k in any order, the
// MFMA k-slots are filled with whatever 8 consecutive values a lane holds,
// identically for both operands.
//   NVFP4: v_mfma_f32_16x16x32_f16 on exact fp16 products v * E4M3(sb)
//          (at most 6 significant bits, range [2^-10, 2688]); tensor scales
//          in the epilogue.
//   MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1 and
//          the E8M0 block scale of each lane's 32 values.
#include <cstddef>

#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Scalars for LDS bytes written and read at different widths: without
// may_alias, type-based alias analysis lets a 16-bit read move above the
// 32-bit write of the same bytes.
typedef uint32_t __attribute__((may_alias)) u32_alias;
typedef uint16_t __attribute__((may_alias)) u16_alias;

constexpr int kWaves = 4;
constexpr int kRows = 16;

__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t c) {
  return (_Float16)e4m3_decode(c);
}

__device__ __forceinline__ v8h dequant8(uint32_t w, _Float16 s) {
  const v2h sv = {s, s};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sv;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sv;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sv;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sv;
  return (v8h){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ void store_out(void* c, int c_dtype, int64_t idx, float v) {
  if (c_dtype == kInF32) {
    reinterpret_cast<float*>(c)[idx] = v;
  } else {
    reinterpret_cast<__bf16*>(c)[idx] = (__bf16)v;
  }
}

// Adds the 4 waves' 16x16 partial tiles; wave 0 stores C[m, n0 + ...].
__device__ __forceinline__ void reduce_store(v4f acc, float scale, int64_t m, int64_t n,
                                             int64_t n0, void* c, int c_dtype) {
  __shared__ v4f part[kWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    v4f s = part[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += part[w][lane];
    // D layout: lane holds rows 4*(lane/16) + e (weight rows), column lane % 16 (activation row)
    const int64_t mi = lane & 15;
    if (mi < m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ni = n0 + 4 * (lane >> 4) + e;
        if (ni < n) store_out(c, c_dtype, mi * n + ni, s[e] * scale);
      }
    }
  }
}

template <int UNROLL>
__global__ __launch_bounds__(256) void gemm_nv_skinny(
    int64_t m, int64_t n, int64_t k, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const float* __restrict__ at,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs,
    const float* __restrict__ bt, void* __restrict__ c, int c_dtype) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t wrow = (n0 + r < n) ? n0 + r : n - 1;
  const bool arow_ok = r < m;
  const int64_t arow = arow_ok ? r : 0;
  const int64_t kbytes = k / 2, kblocks = k / 16, k32 = k / 32;
  // a trip covers 128 values; lane group g owns the 32 values at 128*ch + 32*g
  const int64_t nchunks = (k + 127) / 128;
  const int64_t per_wave = (nchunks + kWaves - 1) / kWaves;
  const int64_t c0 = wave * per_wave;
  const int64_t c1 = (c0 + per_wave < nchunks) ? c0 + per_wave : nchunks;
  const uint8_t* wp = b + wrow * kbytes + 16 * g;
  const uint8_t* ap = a + arow * kbytes + 16 * g;
  const uint8_t* wsp = bs + wrow * kblocks + 2 * g;
  const uint8_t* asp = as + arow * kblocks + 2 * g;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t ch = c0; ch < c1; ch += UNROLL) {
    u32x4 wv[UNROLL], av[UNROLL];
    uint32_t wsv[UNROLL], asv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      // lanes past k load nothing (their 32 values may lie past the row, or
      // past the buffer) and take zero codes with a zero scale: a scale byte
      // from elsewhere could be NaN, and NaN * 0 is NaN
      const bool ok = (ch + u < c1) && ((ch + u) * 4 + g < k32);
      const int64_t cc = ch + u;
      wv[u] = (u32x4){0u, 0u, 0u, 0u};
      av[u] = (u32x4){0u, 0u, 0u, 0u};
      wsv[u] = 0u;
      asv[u] = 0u;
      if (ok) {
        wv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + cc * 64));
        wsv[u] = *reinterpret_cast<const uint16_t*>(wsp + cc * 8);
        if (arow_ok) {
          av[u] = *reinterpret_cast<const u32x4*>(ap + cc * 64);
          asv[u] = *reinterpret_cast<const uint16_t*>(asp + cc * 8);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const _Float16 ws0 = e4m3_to_f16(wsv[u] & 0xFFu), ws1 = e4m3_to_f16((wsv[u] >> 8) & 0xFFu);
      const _Float16 as0 = e4m3_to_f16(asv[u] & 0xFFu), as1 = e4m3_to_f16((asv[u] >> 8) & 0xFFu);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8h fw = dequant8(wv[u][j], j < 2 ? ws0 : ws1);
        const v8h fa = dequant8(av[u][j], j < 2 ? as0 : as1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw, fa, acc, 0, 0, 0);
      }
    }
  }
  reduce_store(acc, (*at) * (*bt), m, n, n0, c, c_dtype);
}

template <int UNROLL>
__global__ __launch_bounds__(256) void gemm_mx_skinny(
    int64_t m, int64_t n, int64_t k, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const uint8_t* __restrict__ b,
    const uint8_t* __restrict__ bs, void* __restrict__ c, int c_dtype) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t wrow = (n0 + r < n) ? n0 + r : n - 1;
  const bool arow_ok = r < m;
  const int64_t arow = arow_ok ? r : 0;
  const int64_t kbytes = k / 2, kblocks = k / 32;
  // a trip covers 128 values = 4 blocks of 32; lane group g owns block g
  const int64_t nchunks = (k + 127) / 128;
  const int64_t per_wave = (nchunks + kWaves - 1) / kWaves;
  const int64_t c0 = wave * per_wave;
  const int64_t c1 = (c0 + per_wave < nchunks) ? c0 + per_wave : nchunks;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t ch = c0; ch < c1; ch += UNROLL) {
    u32x4 wv[UNROLL], av[UNROLL];
    int wsv[UNROLL], asv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t blk = (ch + u) * 4 + g;
      // lanes past k (and rows past m) take zero codes with scale 2^0
      const bool ok = (ch + u < c1) && blk < kblocks;
      wv[u] = (u32x4){0u, 0u, 0u, 0u};
      av[u] = (u32x4){0u, 0u, 0u, 0u};
      wsv[u] = 127;
      asv[u] = 127;
      if (ok) {
        wv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + wrow * kbytes + blk * 16));
        wsv[u] = bs[wrow * kblocks + blk];
        if (arow_ok) {
          av[u] = *reinterpret_cast<const u32x4*>(a + arow * kbytes + blk * 16);
          asv[u] = as[arow * kblocks + blk];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const v8i fw = {(int)wv[u][0], (int)wv[u][1], (int)wv[u][2], (int)wv[u][3], 0, 0, 0, 0};
      const v8i fa = {(int)av[u][0], (int)av[u][1], (int)av[u][2], (int)av[u][3], 0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw, fa, acc, 4, 4, 0, wsv[u], 0, asv[u]);
    }
  }
  reduce_store(acc, 1.0f, m, n, n0, c, c_dtype);
}


// ---- NVFP4 decode fast path (m <= 8, k % KC == 0) --------------------------
// One workgroup = 32 weight rows = 2 row tiles x 2 k-halves (one wave each),
// k processed in chunks of KC values with a two-stage LDS ring:
//  * weight codes and scales of a chunk are read with fully coalesced
//    16-byte loads (a wave instruction covers whole 128-byte lines) and
//    written to LDS, where 16-byte chunk c of row r sits at c ^ (r & 15) so
//    the 16-row MFMA fragment reads do not collide in a bank;
//  * the chunk's activations are dequantized once per workgroup to exact fp16
//    in LDS (same swizzle);
//  * loads of chunk c+1 are in flight while chunk c is multiplied.
constexpr int kDecRows = 32;
constexpr int kDecKC = 1024;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 15); }

// Activation layout: 16-byte chunk c of row r sits at c ^ ((r & 3) << 2 | (c >> 4) & 3).
// Both the dequantizing writes (2 rows x 32 items per wave instruction) and
// the fragment reads (8 rows x 4 lane groups) then spread evenly over the
// 16 bank groups.
__device__ __forceinline__ int xswz(int row, int chunk) {
  return chunk ^ (((row & 3) << 2) | ((chunk >> 4) & 3));
}

template <int KC>
struct DecodeStage {
  uint8_t w[kDecRows][KC / 2];        // weight codes
  uint8_t s[kDecRows][KC / 16 + 16];  // weight scale bytes (row padded against bank conflicts)
  _Float16 x[8][KC];                  // dequantized activations
};

template <int KC, int NCH>
__global__ __launch_bounds__(256) void gemm_nv_decode(
    int m, int64_t n, int k, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const float* __restrict__ at,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs,
    const float* __restrict__ bt, void* __restrict__ c, int c_dtype) {
  constexpr int WCH = KC / 32;                          // 16-byte code chunks per row
  constexpr int WLD = kDecRows * WCH / 256;             // code loads per thread
  constexpr int SB = kDecRows * (KC / 16) / 256;        // scale bytes per thread
  static_assert(WLD >= 1 && SB == 8 && 8 * KC / 32 == 256, "chunk shape");
  __shared__ DecodeStage<KC> st[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nbase = (int64_t)blockIdx.x * kDecRows;
  const int nchunks = k / KC;

  // Per-thread global sources, NCH chunks in flight at once.  Every load is
  // unconditional (indices are clamped instead), so the compiler can wait for
  // one chunk's loads while the later chunks are still arriving.
  u32x4 wreg[NCH][WLD], xreg[NCH];
  u32x2 sreg[NCH];
  uint32_t xsreg[NCH];
  const int xrow_ld = tid / (KC / 32);                  // activation row this thread dequantizes
  const int64_t xr_src = xrow_ld < m ? xrow_ld : 0;
  auto load_chunk = [&](int ch, int slot) {
    const int64_t kb = (int64_t)(ch < nchunks ? ch : nchunks - 1) * KC;
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int idx = tid + 256 * i, row = idx / WCH, cc = idx % WCH;
      const int64_t gr = (nbase + row < n) ? nbase + row : n - 1;
      wreg[slot][i] = *(reinterpret_cast<const u32x4*>(b + gr * (k / 2) + kb / 2) + cc);
    }
    {
      const int row = tid / (KC / 16 / SB), cc = tid % (KC / 16 / SB);
      const int64_t gr = (nbase + row < n) ? nbase + row : n - 1;
      sreg[slot] = *(reinterpret_cast<const u32x2*>(bs + gr * (k / 16) + kb / 16) + cc);
    }
    {
      const int item = tid % (KC / 32);
      xreg[slot] = *reinterpret_cast<const u32x4*>(a + xr_src * (k / 2) + kb / 2 + item * 16);
      xsreg[slot] = *reinterpret_cast<const uint16_t*>(as + xr_src * (k / 16) + kb / 16 + item * 2);
    }
  };
  auto store_chunk = [&](DecodeStage<KC>& S, int slot) {
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int idx = tid + 256 * i, row = idx / WCH, cc = idx % WCH;
      *reinterpret_cast<u32x4*>(&S.w[row][swz(row, cc) * 16]) = wreg[slot][i];
    }
    {
      const int row = tid / (KC / 16 / SB), cc = tid % (KC / 16 / SB);
      *reinterpret_cast<u32x2*>(&S.s[row][cc * SB]) = sreg[slot];
    }
    {
      const int item = tid % (KC / 32);
      const bool live = xrow_ld < m;
      const v2h s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(live ? xsreg[slot] : 0u, 1.0f, false);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8h f = dequant8(live ? xreg[slot][j] : 0u, j < 2 ? s2.x : s2.y);
        *reinterpret_cast<v8h*>(&S.x[xrow_ld][xswz(xrow_ld, item * 4 + j) * 8]) = f;
      }
    }
  };

  const int r = lane & 15, g = lane >> 4;
  const int rt = wave & 1, kh = wave >> 1;
  const int wr = rt * 16 + r;                           // weight row in the tile
  const bool xrow = r < m;
  v4f acc = {0.f, 0.f, 0.f, 0.f}, acc1 = acc;

  // Chunks go in groups of NCH: all loads of a group are issued before the
  // first of its chunks is stored to LDS and multiplied.
  for (int g0 = 0; g0 < nchunks; g0 += NCH) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) load_chunk(g0 + u, u);
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int ch = g0 + u;
      if (ch >= nchunks) break;
      DecodeStage<KC>& S = st[u & 1];
      store_chunk(S, u);
      __syncthreads();
      // this wave: k-half kh of the chunk, lane group g owns KC/8 contiguous values
      constexpr int PER = KC / 8;
      static_assert(PER == 128, "one 8-byte scale read per chunk");
      const int v0 = kh * (KC / 2) + g * PER;
      const uint2 scb = *reinterpret_cast<const uint2*>(&S.s[wr][v0 / 16]);   // 8 blocks
#pragma unroll
      for (int q = 0; q < PER / 32; ++q) {              // 32 values = 16 code bytes = 2 blocks
        const int vq = v0 + q * 32;
        const u32x4 wc = *reinterpret_cast<const u32x4*>(&S.w[wr][swz(wr, vq / 32) * 16]);
        const uint32_t sw = (q < 2) ? scb.x : scb.y;
        const v2h s2 = (q & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)
                               : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v8h fw = dequant8(wc[j], j < 2 ? s2.x : s2.y);
          v8h fx = {0, 0, 0, 0, 0, 0, 0, 0};
          if (xrow) fx = *reinterpret_cast<const v8h*>(&S.x[r][xswz(r, vq / 8 + j) * 8]);
          if (j & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw, fx, acc1, 0, 0, 0);
          else acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw, fx, acc, 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // add the two k-halves and store
  acc += acc1;
  v4f* part = reinterpret_cast<v4f*>(&st[0]);
  if (kh == 1) part[rt * 64 + lane] = acc;
  __syncthreads();
  if (kh == 0) {
    acc += part[rt * 64 + lane];
    const float scale = (*at) * (*bt);
    if (r < m) {
      const int64_t n0 = nbase + rt * 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ni = n0 + 4 * g + e;
        if (ni < n) store_out(c, c_dtype, (int64_t)r * n + ni, acc[e] * scale);
      }
    }
  }
}


// ---- NVFP4 weight-stream kernel (m <= 16, k in chunks of 2048 or 4096) -------
// The weight rows are dealt out evenly: one workgroup of 16 waves per
// CU-share of R = ceil(n / 256) rows (at most 64: up to four 16-row MFMA
// tiles, the last possibly partial), so every CU streams the same number of
// bytes.  The 16 waves split a chunk of 2048 NSTEP values of k (NSTEP = 1 or
// 2; k in one chunk, or split over workgroup rows): wave w takes the slice
// of NSTEP steps of 128 values at 128 NSTEP w, for all its tiles, and issues
// all its loads at once.  Requests are not served in issue order (a wave's
// data tends to arrive in one burst at any time during the stream), so each
// wave depends only on its own loads: it dequantizes its activation slice and
// stores its scale slices in LDS regions of its own, and the 16 partial tiles
// meet only at the end.  Lane (r, g) = (lane % 16, lane / 16) reads, per step
// t, the 16 bytes at 64 t + 16 g of weight row r of each tile: a load
// instruction covers 64 contiguous bytes of 16 rows.  Rows past the
// workgroup's share re-read its last row, in the same instruction, so they
// cost no extra traffic.
constexpr int kStrWaves = 16;
constexpr int kStrTiles = 4;                          // 64 rows at most per workgroup
constexpr int kStrGroups = 256;                       // one workgroup per CU

template <int NSTEP, int XH>
struct StreamLds {
  // dequantized activation slices (8 XH rows), rows padded so that the 8
  // rows of a read fall on distinct banks
  _Float16 x[kStrWaves][8 * XH][128 * NSTEP + 8];
  // weight scale slices, rows padded: the 16 rows of a read hit distinct banks
  uint8_t w[kStrWaves][16 * kStrTiles][8 * NSTEP + 4];
};

// The activations (XM):
//   kXCodes  NVFP4 codes, scales and tensor scale (`a`, `as`, `at`).
//   kXQuant  bf16 X [m, k] (`a`), quantized here to NVFP4 with the tensor
//            scale computed from the data, with the arithmetic of the
//            quantize kernels: every workgroup reduces max |X| over the whole
//            tensor (16 slices, one per wave) and quantizes its own slices;
//            workgroup 0 also writes the codes, scales and tensor scale out
//            (qcodes, qscales, qtscale).
//   kXRaw    bf16 X [m, k] (`a`) used as it is: W4A16 (pimento.cloud "FP8,
//            NVFP4 czy AWQ?", section "Dlaczego W8A8 i W4A16 to nie to
//            samo?": only the weights are 4-bit, the products stay 16-bit).
//            Each wave scales each row of its slice by the power of two 2^-E
//            that brings the slice row's max |x| into [1, 2) and rounds to
//            fp16: exact for every value above 2^-15 of that max (bf16 has 8
//            significant bits, fp16 11), the rest within 2^-25 of it; the
//            wave's partial sums are scaled back by 2^E (exact) before the
//            slices are added.
// `as` and `at` are unused but for kXCodes.
//
// kXQuant needs max |X| over the whole tensor before any weight can be used.
// While the weight stream is in flight, a load queued behind it waits for
// most of it, so the activation loads go first and only the first tile's
// weights with them; the rest goes out once every wave's part of max |X| is
// in.
//   kXRawH   fp16 X, the same way as kXRaw.
constexpr int kXCodes = 0, kXQuant = 1, kXRaw = 2, kXRawH = 3;

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// XH = 2: up to 16 activation rows, all 16 columns of the MFMA tile (XH = 1:
// 8 rows, the other 8 columns repeat them).
template <int NSTEP, int XM, int XH>
__global__ __launch_bounds__(64 * kStrWaves) void gemm_nv_stream(
    int m, int64_t n, int k, int rows_per_wg, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const float* __restrict__ at,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs,
    const float* __restrict__ bt, void* __restrict__ c, int c_dtype,
    uint8_t* __restrict__ qcodes, uint8_t* __restrict__ qscales, float* __restrict__ qtscale,
    float* __restrict__ part, int64_t pstride) {
  constexpr int NT = kStrTiles;
  __shared__ union {
    StreamLds<NSTEP, XH> s;
    v4f part[kStrWaves][NT][64];                      // the partial tiles, at the end
  } LU;
  __shared__ float red[kStrWaves];
  StreamLds<NSTEP, XH>& L = LU.s;

  constexpr bool QX = XM != kXCodes;                  // 16-bit X loaded here
  constexpr bool RAW = XM == kXRaw || XM == kXRawH;   // W4A16
  // the two 16-bit values of a dword of X, widened exactly
  auto xlo = [](uint32_t w) { return XM == kXRawH ? f16_lo(w) : bf16_lo(w); };
  auto xhi = [](uint32_t w) { return XM == kXRawH ? f16_hi(w) : bf16_hi(w); };
  constexpr bool GMAX = XM == kXQuant;                // max |X| over the tensor first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t nbase = (int64_t)blockIdx.x * rows_per_wg;
  int64_t nlast = nbase + rows_per_wg - 1;            // last row of this share
  if (nlast > n - 1) nlast = n - 1;
  // split k (part != nullptr; codes in or W4A16): workgroup row blockIdx.y
  // takes the 2048 NSTEP values from kc0 on, and its fp32 sums go to part
  const int kc0 = (int)blockIdx.y * (kStrWaves * 128 * NSTEP);
  // k not a whole number of chunks (codes in, W4A16; the one-launch
  // quantize takes whole chunks only): a slice that starts past k loads the
  // last slice again, in bounds, and adds nothing
  const bool kdead = !GMAX && kc0 + wave * (128 * NSTEP) >= k;
  const int ks0 = kdead ? k - 128 * NSTEP : kc0 + wave * (128 * NSTEP);   // first value of this wave's slice
  const int64_t kbytes = k / 2, kblocks = k / 16;

  // ---- activation slice: lane -> row lane / 8, the 16 NSTEP values (NSTEP
  // whole blocks) at ks0 + 16 NSTEP (lane % 8) --------------------------------------
  const int xrow = lane >> 3, xc = lane & 7;
  const bool live = xrow < m;
  const int64_t xsrc = live ? xrow : m - 1;
  const int xv0 = ks0 + 16 * NSTEP * xc;
  u32x4 xb[QX ? 2 * NSTEP : 1];                        // bf16 X, 8 values each
  uint32_t xq[XH][2 * NSTEP];                         // codes, 8 per dword (kXCodes)
  uint32_t xs[XH];                                    // NSTEP scale bytes (kXCodes)
  // bf16 X with 16 rows: row 8 + lane / 8 as well
  constexpr bool RAW2 = RAW && XH == 2;
  constexpr bool Q2 = XM == kXQuant && XH == 2;
  u32x4 xb2[(RAW2 || Q2) ? 2 * NSTEP : 1];
  const bool live2 = 8 + xrow < m;
  const int64_t xsrc2 = live2 ? 8 + xrow : m - 1;
  if (QX) {
#pragma unroll
    for (int i = 0; i < 2 * NSTEP; ++i)
      xb[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a) + xsrc * k + xv0 + 8 * i);
    if constexpr (RAW2 || Q2) {
#pragma unroll
      for (int i = 0; i < 2 * NSTEP; ++i)
        xb2[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a) + xsrc2 * k + xv0 + 8 * i);
    }
  } else {
    // row 8 hf + lane / 8 of each group of 8 rows
#pragma unroll
    for (int hf = 0; hf < XH; ++hf) {
      const int64_t xsh = 8 * hf + xrow < m ? 8 * hf + xrow : m - 1;
      const uint8_t* src = a + xsh * kbytes + xv0 / 2;
      if (NSTEP == 1) {
        const u32x2 h = *reinterpret_cast<const u32x2*>(src);
        xq[hf][0] = h.x; xq[hf][1] = h.y;
      } else {
        const u32x4 h = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int j = 0; j < 4; ++j) xq[hf][j] = h[j];
      }
      const uint8_t* ss = as + xsh * kblocks + xv0 / 16;
      xs[hf] = NSTEP == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(ss) : (uint32_t)*ss;
    }
  }

  // ---- weights: scale slices (lane p loads row p's 8 NSTEP bytes) and codes ----
  const int64_t swr = (nbase + lane <= nlast) ? nbase + lane : nlast;
  u32x4 sv;
  auto load_ws = [&]() {
    if (NSTEP == 2) {
      sv = *reinterpret_cast<const u32x4*>(bs + swr * kblocks + ks0 / 16);
    } else {
      const u32x2 h = *reinterpret_cast<const u32x2*>(bs + swr * kblocks + ks0 / 16);
      sv = (u32x4){h.x, h.y, 0u, 0u};
    }
  };
  u32x4 w[NT][NSTEP];
  auto load_w = [&](int t0, int t1) {
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) {
      if (tl < t0 || tl >= t1) continue;
      const int64_t wr = (nbase + 16 * tl + r <= nlast) ? nbase + 16 * tl + r : nlast;
#pragma unroll
      for (int t = 0; t < NSTEP; ++t)
        w[tl][t] = *reinterpret_cast<const u32x4*>(b + wr * kbytes + ks0 / 2 + 64 * t + 16 * g);
    }
  };
  if (GMAX) {
    load_w(0, 1);
  } else {
    load_ws();
    load_w(0, NT);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- activations into this wave's LDS region --------------------------------------
  _Float16* xdst = &L.x[wave][xrow][16 * NSTEP * xc];
  float xscale = 1.0f;                                // the activations' tensor scale
  float xscale2 = 1.0f;                               // W4A16, 16 rows: 2^E of row 8 + lane / 8
  if (QX) {
    // this wave's part of max |X|
    float am[NSTEP];
#pragma unroll
    for (int bl = 0; bl < NSTEP; ++bl) {
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          mx = fmaxf(mx, fmaxf(fabsf(xlo(xb[2 * bl + i][j])), fabsf(xhi(xb[2 * bl + i][j]))));
      am[bl] = live ? mx : 0.0f;
    }
    float wm = NSTEP == 2 ? fmaxf(am[0], am[NSTEP - 1]) : am[0];
    // the second group of 8 rows (one-launch quantize of 16 rows)
    float am2[NSTEP];
    if constexpr (Q2) {
#pragma unroll
      for (int bl = 0; bl < NSTEP; ++bl) {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            mx = fmaxf(mx, fmaxf(fabsf(xlo(xb2[2 * bl + i][j])), fabsf(xhi(xb2[2 * bl + i][j]))));
        am2[bl] = live2 ? mx : 0.0f;
        wm = fmaxf(wm, am2[bl]);
      }
    }
    float A = 0.0f;
    if (GMAX) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off));
      if (lane == 0) red[wave] = wm;
      // max |X| over the whole tensor once every wave's part is in `red`;
      // then the rest of the weights go out
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0), loads stay in flight
      __asm__ volatile("s_barrier" ::: "memory");
      load_ws();
      load_w(1, NT);
      __builtin_amdgcn_sched_barrier(0);
      A = red[0];
#pragma unroll
      for (int i = 1; i < kStrWaves; ++i) A = fmaxf(A, red[i]);
    } else {
      // max |x| of this slice row: the 8 lanes of row lane / 8
#pragma unroll
      for (int off = 4; off >= 1; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off));
      A = wm;
    }
    if (RAW) {
      // 2^-E with the slice row's max |x| in [2^E, 2^(E+1)); 1 for a zero row
      const int eb = (int)(as_u(A) >> 23);
      const int pe = A == 0.0f ? 127 : (254 - eb < 1 ? 1 : 254 - eb);
      const float p2 = as_f((uint32_t)pe << 23);
      xscale = as_f((uint32_t)(254 - pe) << 23);      // 2^E of row lane / 8, exact
#pragma unroll
      for (int i = 0; i < 2 * NSTEP; ++i) {
        v8h f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[2 * j] = (_Float16)(xlo(xb[i][j]) * p2);
          f[2 * j + 1] = (_Float16)(xhi(xb[i][j]) * p2);
        }
        if (!live) f = (v8h){0, 0, 0, 0, 0, 0, 0, 0};
        *reinterpret_cast<v8h*>(xdst + 8 * i) = f;
      }
      if constexpr (RAW2) {
        // the second group of 8 rows, scaled the same way (2^E in xscale2)
        float m2 = 0.0f;
#pragma unroll
        for (int i = 0; i < 2 * NSTEP; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            m2 = fmaxf(m2, fmaxf(fabsf(xlo(xb2[i][j])), fabsf(xhi(xb2[i][j]))));
        m2 = live2 ? m2 : 0.0f;
#pragma unroll
        for (int off = 4; off >= 1; off >>= 1) m2 = fmaxf(m2, __shfl_xor(m2, off));
        const int eb2 = (int)(as_u(m2) >> 23);
        const int pe2 = m2 == 0.0f ? 127 : (254 - eb2 < 1 ? 1 : 254 - eb2);
        const float q2 = as_f((uint32_t)pe2 << 23);
        xscale2 = as_f((uint32_t)(254 - pe2) << 23);
        _Float16* xd2 = &L.x[wave][8 + xrow][16 * NSTEP * xc];
#pragma unroll
        for (int i = 0; i < 2 * NSTEP; ++i) {
          v8h f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f[2 * j] = (_Float16)(xlo(xb2[i][j]) * q2);
            f[2 * j + 1] = (_Float16)(xhi(xb2[i][j]) * q2);
          }
          if (!live2) f = (v8h){0, 0, 0, 0, 0, 0, 0, 0};
          *reinterpret_cast<v8h*>(xd2 + 8 * i) = f;
        }
      }
    } else {
      float s_t = A / 2688.0f;                        // 6 * 448
      if (s_t == 0.0f) s_t = 1.0f;
      const float dd = 6.0f * s_t;
      xscale = s_t;
      const bool out = blockIdx.x == 0 && live;
#pragma unroll
      for (int bl = 0; bl < NSTEP; ++bl) {
        const uint32_t sbyte = e4m3_encode_pos(am[bl] / dd);
        const float S = e4m3_decode_pos(sbyte) * s_t;
        float rs = 1.0f / S;
        if (!(S != 0.0f && rs < __builtin_inff())) rs = 0.0f;   // zero block or overflowing reciprocal
        uint32_t wd[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 v = xb[2 * bl + h];
          uint32_t p = e2m1_pack2<0>(0u, bf16_lo(v[0]) * rs, bf16_hi(v[0]) * rs);
          p = e2m1_pack2<1>(p, bf16_lo(v[1]) * rs, bf16_hi(v[1]) * rs);
          p = e2m1_pack2<2>(p, bf16_lo(v[2]) * rs, bf16_hi(v[2]) * rs);
          p = e2m1_pack2<3>(p, bf16_lo(v[3]) * rs, bf16_hi(v[3]) * rs);
          wd[h] = p;
          v8h f = dequant8(p, (_Float16)e4m3_decode_pos(sbyte));
          if (!live) f = (v8h){0, 0, 0, 0, 0, 0, 0, 0};
          *reinterpret_cast<v8h*>(xdst + 16 * bl + 8 * h) = f;
        }
        if (XM == kXQuant && out) {
          *reinterpret_cast<u32x2*>(qcodes + xsrc * kbytes + (xv0 + 16 * bl) / 2) = (u32x2){wd[0], wd[1]};
          qscales[xsrc * kblocks + (xv0 + 16 * bl) / 16] = (uint8_t)sbyte;
        }
      }
      if constexpr (Q2) {
        // the second group of 8 rows, the same arithmetic
        _Float16* xd2 = &L.x[wave][8 + xrow][16 * NSTEP * xc];
        const bool out2 = blockIdx.x == 0 && live2;
#pragma unroll
        for (int bl = 0; bl < NSTEP; ++bl) {
          const uint32_t sbyte = e4m3_encode_pos(am2[bl] / dd);
          const float S = e4m3_decode_pos(sbyte) * s_t;
          float rs = 1.0f / S;
          if (!(S != 0.0f && rs < __builtin_inff())) rs = 0.0f;
          uint32_t wd[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 v = xb2[2 * bl + h];
            uint32_t p = e2m1_pack2<0>(0u, bf16_lo(v[0]) * rs, bf16_hi(v[0]) * rs);
            p = e2m1_pack2<1>(p, bf16_lo(v[1]) * rs, bf16_hi(v[1]) * rs);
            p = e2m1_pack2<2>(p, bf16_lo(v[2]) * rs, bf16_hi(v[2]) * rs);
            p = e2m1_pack2<3>(p, bf16_lo(v[3]) * rs, bf16_hi(v[3]) * rs);
            wd[h] = p;
            v8h f = dequant8(p, (_Float16)e4m3_decode_pos(sbyte));
            if (!live2) f = (v8h){0, 0, 0, 0, 0, 0, 0, 0};
            *reinterpret_cast<v8h*>(xd2 + 16 * bl + 8 * h) = f;
          }
          if (out2) {
            *reinterpret_cast<u32x2*>(qcodes + xsrc2 * kbytes + (xv0 + 16 * bl) / 2) = (u32x2){wd[0], wd[1]};
            qscales[xsrc2 * kblocks + (xv0 + 16 * bl) / 16] = (uint8_t)sbyte;
          }
        }
      }
      if (XM == kXQuant && blockIdx.x == 0 && tid == 0) *qtscale = s_t;
    }
  } else {
#pragma unroll
    for (int hf = 0; hf < XH; ++hf) {
      _Float16* xd = &L.x[wave][8 * hf + xrow][16 * NSTEP * xc];
      const bool lv = 8 * hf + xrow < m;
      // the E4M3 bytes to f16 (sign and NaN included)
      const v2h s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xs[hf], 1.0f, false);
#pragma unroll
      for (int bl = 0; bl < NSTEP; ++bl) {
        const _Float16 s = bl == 0 ? s01.x : s01.y;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          v8h f = dequant8(xq[hf][2 * bl + h], s);
          if (!lv) f = (v8h){0, 0, 0, 0, 0, 0, 0, 0};
          *reinterpret_cast<v8h*>(xd + 16 * bl + 8 * h) = f;
        }
      }
    }
  }
  {
    u32_alias* dd = reinterpret_cast<u32_alias*>(&L.w[wave][lane][0]);
    dd[0] = sv[0]; dd[1] = sv[1];
    if (NSTEP == 2) { dd[2] = sv[2]; dd[3] = sv[3]; }
  }
  // Only this wave reads these regions: LDS accesses of one wave complete in
  // order, so no barrier is needed.
  // rows >= m are zero; with XH = 1, r >= 8 repeats r - 8
  const _Float16* xf = &L.x[wave][XH == 2 ? r : (r & 7)][32 * g];

  v4f acc[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) acc[tl] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NSTEP; ++t) {
    v2h s[NT];
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) {
      const uint32_t p = *reinterpret_cast<const u16_alias*>(&L.w[wave][16 * tl + r][8 * t + 2 * g]);
      s[tl] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p, 1.0f, false);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {                     // 8 values per dword; blocks 2g, 2g+1
      const v8h fx = *reinterpret_cast<const v8h*>(xf + 128 * t + 8 * d);
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        const v8h fw = dequant8(w[tl][t][d], d < 2 ? s[tl].x : s[tl].y);
        acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw, fx, acc[tl], 0, 0, 0);
      }
    }
  }

  if (RAW) {
    // back to the scale of X: acc column lane % 16 is activation row
    // lane % 16, whose 2^E lane 8 (lane % 8) holds (rows >= 8 are zero)
    float e = __shfl(xscale, 8 * (lane & 7));
    if constexpr (RAW2) {
      const float e2 = __shfl(xscale2, 8 * (lane & 7));
      if ((lane & 15) >= 8) e = e2;
    }
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) acc[tl] *= e;
  }

  // ---- add the 16 slices, store ------------------------------------------------
  __syncthreads();                                    // LDS becomes the partial area
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) LU.part[wave][tl][lane] = kdead ? (v4f){0.f, 0.f, 0.f, 0.f} : acc[tl];
  __syncthreads();
  if (tid < 64 * NT) {                                // thread -> (tile, lane)
    const int tl = tid >> 6, l = tid & 63;
    v4f sum = LU.part[0][tl][l];
#pragma unroll
    for (int wv = 1; wv < kStrWaves; ++wv) sum += LU.part[wv][tl][l];
    const float scale = (XM == kXQuant ? xscale : RAW ? 1.0f : *at) * (*bt);
    // D layout: lane l holds weight rows 4 (l / 16) + e of the tile, activation row l % 16
    const int xr = l & 15, lr = 16 * tl + 4 * (l >> 4);   // first row within the share
    const int64_t ni = nbase + lr;
    if (xr < m && lr < rows_per_wg && ni <= nlast) {
      const int64_t o = (int64_t)xr * n + ni;
      if (part) {
        // codes in: unscaled (the reduction applies the tensor scales);
        // W4A16: times the weights' tensor scale
        float* pp = part + (int64_t)blockIdx.y * pstride + o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (lr + e < rows_per_wg && ni + e <= nlast) pp[e] = RAW ? sum[e] * scale : sum[e];
      } else if (c_dtype != kInF32 && lr + 3 < rows_per_wg && ni + 3 <= nlast && (o & 3) == 0) {
        const __bf16 h[4] = {(__bf16)(sum[0] * scale), (__bf16)(sum[1] * scale), (__bf16)(sum[2] * scale),
                             (__bf16)(sum[3] * scale)};
        *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(c) + o) = *reinterpret_cast<const u32x2*>(h);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (lr + e < rows_per_wg && ni + e <= nlast) store_out(c, c_dtype, o + e, sum[e] * scale);
      }
    }
  }
}

// W4A16 for any shape: thread -> one weight row j and up to 8 activation
// rows; the weights are widened exactly in fp32 (v * E4M3 scale, or v * 2^e)
// and the products summed in fp32.  The fallback of the streaming kernel.
template <int FMT, int DT>
__global__ __launch_bounds__(256) void gemm_w4a16_simple(
    int m, int64_t n, int k, const void* __restrict__ x, const uint8_t* __restrict__ b,
    const uint8_t* __restrict__ bs, const float* __restrict__ bt, void* __restrict__ c,
    int c_dtype) {
  constexpr int BS = FMT == kFmtNV ? 16 : 32;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int i0 = blockIdx.y * 8;
  if (j >= n) return;
  const int rows = m - i0 < 8 ? m - i0 : 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint8_t* wr = b + j * (int64_t)(k / 2);
  const uint8_t* sr = bs + j * (int64_t)(k / BS);
  for (int kb = 0; kb < k; kb += BS) {
    const uint32_t sb = sr[kb / BS];
    const float S = block_scale_value<FMT == kFmtNV>(sb);
    for (int t = 0; t < BS; t += 8) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(wr + (kb + t) / 2);
      const v2f p0 = e2m1_unpack2<0>(w), p1 = e2m1_unpack2<1>(w);
      const v2f p2 = e2m1_unpack2<2>(w), p3 = e2m1_unpack2<3>(w);
      const float wv[8] = {p0.x * S, p0.y * S, p1.x * S, p1.y * S, p2.x * S, p2.y * S, p3.x * S, p3.y * S};
      for (int i = 0; i < rows; ++i) {
        const int64_t xo = (int64_t)(i0 + i) * k + kb + t;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float xv;
          if (DT == kInF32) xv = reinterpret_cast<const float*>(x)[xo + e];
          else if (DT == kInBF16) xv = as_f((uint32_t)reinterpret_cast<const uint16_t*>(x)[xo + e] << 16);
          else xv = (float)reinterpret_cast<const _Float16*>(x)[xo + e];
          acc[i] = acc[i] + xv * wv[e];
        }
      }
    }
  }
  const float ts = FMT == kFmtNV ? *bt : 1.0f;
  for (int i = 0; i < rows; ++i) store_out(c, c_dtype, (int64_t)(i0 + i) * n + j, acc[i] * ts);
}

// The one-launch quantize's shapes with 8 activation rows: m <= 8, k = 2048
// or 4096, n <= 16384 (one round of workgroups).
bool stream_shape(int64_t m, int64_t n, int64_t k) {
  return m >= 1 && m <= 8 && (k == 2048 || k == 4096) && n >= 1 && n <= 16 * kStrTiles * kStrGroups;
}

// The stream kernel's k-step: NSTEP = 2 (chunks of 4096 values) when k is a
// multiple of 4096 or a multiple of 256 in (2048, 4096], else NSTEP = 1
// (chunks of 2048).
bool stream_nstep2(int64_t k) { return k % 4096 == 0 || (k > 2048 && k <= 4096 && k % 256 == 0); }

}  // namespace

// Chunks of k for the stream kernel (codes in or W4A16): k from 2048 on, a
// multiple of 128 (256 with NSTEP = 2); 0 for any other k.  A last chunk
// that k does not fill leaves the slices past k idle.
int64_t gemm_stream_chunks(int64_t k) {
  if (k < 2048 || k % 128 != 0) return 0;
  return stream_nstep2(k) ? (k + 4095) / 4096 : (k + 2047) / 2048;
}

namespace {

// An equal share of ceil(n / 256) weight rows per workgroup.
// nsplit > 1: k in nsplit chunks of 2048 NSTEP values (the last one
// possibly short), the chunks' fp32 sums in part.
template <int XM, int XH = 1>
hipError_t launch_stream(int m, int64_t n, int k, const uint8_t* a, const uint8_t* as, const float* at,
                         const uint8_t* b, const uint8_t* bs, const float* bt, void* c, int c_dtype,
                         uint8_t* qcodes, uint8_t* qscales, float* qtscale, hipStream_t stream,
                         int nsplit = 1, float* part = nullptr) {
  // Split k: as many rows per workgroup (at most 64) as fill whole rounds of
  // co-resident workgroups (two per CU with the 64 KiB of LDS of NSTEP = 1,
  // one with the 88 KiB of NSTEP = 2); short-lived workgroups of a few rows
  // would spend their time on the activation slice and the reduction, and a
  // round begun by a few workgroups costs a whole workgroup lifetime.
  const bool nstep2 = stream_nstep2(k);
  const int64_t slots = nstep2 || XH == 2 ? kStrGroups : 2 * kStrGroups;
  int rows = (int)((n + kStrGroups - 1) / kStrGroups);
  if (nsplit > 1 || n > 16 * kStrTiles * kStrGroups) {
    const int64_t rmax = 16 * kStrTiles;
    const int64_t rounds = (((n + rmax - 1) / rmax) * nsplit + slots - 1) / slots;
    const int64_t per_chunk = rounds * slots / nsplit;     // >= ceil(n / rmax)
    rows = (int)((n + per_chunk - 1) / per_chunk);
  }
  const dim3 grid((unsigned)((n + rows - 1) / rows), (unsigned)nsplit);
  const int64_t pstride = nsplit > 1 ? gemm_split_stride(m, n) : 0;
  if (nstep2)
    hipLaunchKernelGGL((gemm_nv_stream<2, XM, XH>), grid, dim3(64 * kStrWaves), 0, stream, m, n, k, rows, a, as,
                       at, b, bs, bt, c, c_dtype, qcodes, qscales, qtscale, part, pstride);
  else
    hipLaunchKernelGGL((gemm_nv_stream<1, XM, XH>), grid, dim3(64 * kStrWaves), 0, stream, m, n, k, rows, a, as,
                       at, b, bs, bt, c, c_dtype, qcodes, qscales, qtscale, part, pstride);
  return hipGetLastError();
}

// Chunks of the split-k stream kernel for NVFP4 codes with m <= 8 and more
// than one chunk of k (gemm_stream_chunks): whole chunks, as long as
// workgroups of at most 64 rows cover every chunk in one round of
// co-resident workgroups (two per CU for chunks of 2048, one for 4096); 0
// for any other shape.  Without
// the split, a long k and few rows (a down projection, say) leave few
// workgroups, each walking all of k; with more than one round, the unsplit
// kernels measured faster.
int stream_split(int fmt, int64_t m, int64_t n, int64_t k) {
  if (fmt != kFmtNV || m < 1 || m > 8 || n < 1) return 0;
  const int64_t s = gemm_stream_chunks(k);
  if (s < 2) return 0;
  // a k the older decode kernel cannot take (not a multiple of 1024): any
  // round count, as the generic kernel would be slower still.  A short last
  // chunk where that kernel can take k measured slower (8x5120x5120: 10.9
  // us split, 10.1 on the older kernel).
  if (k % kDecKC != 0) return s <= 64 ? (int)s : 0;
  if (k % 2048 != 0) return 0;
  const int64_t slots = stream_nstep2(k) ? kStrGroups : 2 * kStrGroups;
  return (n + 16 * kStrTiles - 1) / (16 * kStrTiles) * s <= slots ? (int)s : 0;
}

// Chunks of the split-k stream kernel for NVFP4 codes with 9..16 rows and
// 2 to 64 chunks of k, in whole rounds of workgroups for any n; 0 for any
// other shape.  With 16 activation rows per workgroup, the weights'
// dequantization is shared by twice the columns, so more than one round
// still pays here.
int stream_split16(int fmt, int64_t m, int64_t n, int64_t k) {
  if (fmt != kFmtNV || m <= 8 || m > 16 || n < 1) return 0;
  const int64_t s = gemm_stream_chunks(k);
  return s >= 2 && s <= 64 ? (int)s : 0;
}

}  // namespace

size_t gemm_skinny_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
  const int s = m > 8 ? stream_split16(fmt, m, n, k) : stream_split(fmt, m, n, k);
  return s > 1 ? (size_t)s * (size_t)gemm_split_stride(m, n) * sizeof(float) : 0;
}

hipError_t launch_gemm_skinny(int fmt, int64_t m, int64_t n, int64_t k,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_tscale, const uint8_t* b_codes,
                              const uint8_t* b_scales, const float* b_tscale,
                              void* c, int c_dtype, void* workspace, hipStream_t stream) {
  const bool aligned16 = ((reinterpret_cast<uintptr_t>(b_scales) | reinterpret_cast<uintptr_t>(b_codes) |
                           reinterpret_cast<uintptr_t>(a_codes)) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(a_scales) & 1) == 0;
  // one chunk of k (2048..4096 values), n within one round
  if (fmt == kFmtNV && m >= 1 && m <= 8 && gemm_stream_chunks(k) == 1 && n >= 1 &&
      n <= 16 * kStrTiles * kStrGroups && aligned16)
    return launch_stream<kXCodes>((int)m, n, (int)k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                                  b_tscale, c, c_dtype, nullptr, nullptr, nullptr, stream);
  // 9..16 rows: any n (past 16384 rows, whole rounds of up-to-64-row
  // workgroups); 8 rows past 16384 keep the older decode kernel below, as fast
  if (fmt == kFmtNV && m > 8 && m <= 16 && gemm_stream_chunks(k) == 1 && n >= 1 && aligned16)
    return launch_stream<kXCodes, 2>((int)m, n, (int)k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                                     b_tscale, c, c_dtype, nullptr, nullptr, nullptr, stream);
  const int nsplit = m > 8 ? stream_split16(fmt, m, n, k) : stream_split(fmt, m, n, k);
  if (nsplit > 1 && aligned16) {
    float* part = reinterpret_cast<float*>(workspace);
    const hipError_t e = m > 8 ? launch_stream<kXCodes, 2>((int)m, n, (int)k, a_codes, a_scales, a_tscale, b_codes,
                                                           b_scales, b_tscale, c, c_dtype, nullptr, nullptr,
                                                           nullptr, stream, nsplit, part)
                               : launch_stream<kXCodes>((int)m, n, (int)k, a_codes, a_scales, a_tscale, b_codes,
                                                        b_scales, b_tscale, c, c_dtype, nullptr, nullptr, nullptr,
                                                        stream, nsplit, part);
    if (e != hipSuccess) return e;
    return launch_split_reduce(part, nsplit, m, n, a_tscale, b_tscale, c, c_dtype, stream);
  }
  if (fmt == kFmtNV && m <= 8 && k % kDecKC == 0 && aligned16) {
    hipLaunchKernelGGL((gemm_nv_decode<kDecKC, 4>), dim3((unsigned)((n + kDecRows - 1) / kDecRows)),
                       dim3(256), 0, stream, (int)m, n, (int)k, a_codes, a_scales, a_tscale, b_codes,
                       b_scales, b_tscale, c, c_dtype);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((n + kRows - 1) / kRows));
  if (fmt == kFmtNV) {
    hipLaunchKernelGGL((gemm_nv_skinny<8>), grid, dim3(256), 0, stream, m, n, k, a_codes,
                       a_scales, a_tscale, b_codes, b_scales, b_tscale, c, c_dtype);
  } else {
    hipLaunchKernelGGL((gemm_mx_skinny<8>), grid, dim3(256), 0, stream, m, n, k, a_codes,
                       a_scales, b_codes, b_scales, c, c_dtype);
  }
  return hipGetLastError();
}

// Quantize bf16 activations (NVFP4, tensor scale from the data) and multiply,
// in one launch, for the decode shapes of the stream kernel; returns false
// (nothing launched) for any other shape.
bool launch_quantize_gemm_decode(int64_t m, int64_t n, int64_t k, const void* x,
                                 uint8_t* a_codes, uint8_t* a_scales, float* a_tscale,
                                 const uint8_t* b_codes, const uint8_t* b_scales,
                                 const float* b_tscale, void* c, int c_dtype, hipStream_t stream,
                                 hipError_t* err) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(b_codes) |
                         reinterpret_cast<uintptr_t>(b_scales) | reinterpret_cast<uintptr_t>(a_codes)) &
                        15) == 0;
  if (!(m >= 1 && m <= 16 && stream_shape(8, n, k) && aligned)) return false;
  if (m > 8)
    *err = launch_stream<kXQuant, 2>((int)m, n, (int)k, reinterpret_cast<const uint8_t*>(x), nullptr, nullptr,
                                     b_codes, b_scales, b_tscale, c, c_dtype, a_codes, a_scales, a_tscale, stream);
  else
    *err = launch_stream<kXQuant>((int)m, n, (int)k, reinterpret_cast<const uint8_t*>(x), nullptr, nullptr,
                                  b_codes, b_scales, b_tscale, c, c_dtype, a_codes, a_scales, a_tscale, stream);
  return true;
}

namespace {

// W4A16 chunks of k on the stream kernel for NVFP4 weights (at most 64 of
// gemm_stream_chunks), 0 for any other k.  Any n: past 16384 rows the
// workgroups take up to 64 rows in whole rounds.
int w4a16_chunks(int fmt, int64_t n, int64_t k) {
  if (fmt != kFmtNV || n < 1) return 0;
  const int64_t s = gemm_stream_chunks(k);
  return s <= 64 ? (int)s : 0;
}

}  // namespace

size_t gemm_w4a16_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
  const int s = w4a16_chunks(fmt, n, k);
  const int64_t mc = m < 16 ? m : 16;
  return s > 1 && mc > 0 ? (size_t)s * (size_t)gemm_split_stride(mc, n) * sizeof(float) : 0;
}

hipError_t launch_gemm_w4a16(int fmt, int64_t m, int64_t n, int64_t k, const void* x, int x_dtype,
                             const uint8_t* b_codes, const uint8_t* b_scales,
                             const float* b_tscale, void* c, int c_dtype, void* workspace,
                             hipStream_t stream) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(b_codes) |
                         reinterpret_cast<uintptr_t>(b_scales)) & 15) == 0;
  const int nsplit = x_dtype == kInBF16 || x_dtype == kInF16 ? w4a16_chunks(fmt, n, k) : 0;
  if (nsplit > 0 && aligned) {
    // streaming kernel, 16 activation rows per launch; a split k's chunk
    // sums (times the tensor scale) added by the reduction pass, which
    // reuses the workspace for the next 16 rows in stream order
    float* part = nsplit > 1 ? reinterpret_cast<float*>(workspace) : nullptr;
    const int64_t osz = c_dtype == kInF32 ? 4 : 2;
    for (int64_t i0 = 0; i0 < m; i0 += 16) {
      const int mc = (int)(m - i0 < 16 ? m - i0 : 16);
      const uint8_t* xa = reinterpret_cast<const uint8_t*>(x) + i0 * k * 2;
      void* ca = reinterpret_cast<char*>(c) + i0 * n * osz;
      hipError_t e;
      if (x_dtype == kInF16)
        e = mc > 8 ? launch_stream<kXRawH, 2>(mc, n, (int)k, xa, nullptr, nullptr, b_codes, b_scales, b_tscale, ca,
                                              c_dtype, nullptr, nullptr, nullptr, stream, nsplit, part)
                   : launch_stream<kXRawH>(mc, n, (int)k, xa, nullptr, nullptr, b_codes, b_scales, b_tscale, ca,
                                           c_dtype, nullptr, nullptr, nullptr, stream, nsplit, part);
      else
        e = mc > 8 ? launch_stream<kXRaw, 2>(mc, n, (int)k, xa, nullptr, nullptr, b_codes, b_scales, b_tscale, ca,
                                             c_dtype, nullptr, nullptr, nullptr, stream, nsplit, part)
                   : launch_stream<kXRaw>(mc, n, (int)k, xa, nullptr, nullptr, b_codes, b_scales, b_tscale, ca,
                                          c_dtype, nullptr, nullptr, nullptr, stream, nsplit, part);
      if (e == hipSuccess && nsplit > 1)
        e = launch_split_reduce(part, nsplit, mc, n, nullptr, nullptr, ca, c_dtype, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const dim3 grid((unsigned)((n + 255) / 256), (unsigned)((m + 7) / 8));
#define W4A16_SIMPLE(F, D)                                                                        \
  hipLaunchKernelGGL((gemm_w4a16_simple<F, D>), grid, dim3(256), 0, stream, (int)m, n, (int)k, x, \
                     b_codes, b_scales, b_tscale, c, c_dtype)
  if (fmt == kFmtNV) {
    if (x_dtype == kInF32) W4A16_SIMPLE(kFmtNV, kInF32);
    else if (x_dtype == kInBF16) W4A16_SIMPLE(kFmtNV, kInBF16);
    else W4A16_SIMPLE(kFmtNV, kInF16);
  } else {
    if (x_dtype == kInF32) W4A16_SIMPLE(kFmtMX, kInF32);
    else if (x_dtype == kInBF16) W4A16_SIMPLE(kFmtMX, kInBF16);
    else W4A16_SIMPLE(kFmtMX, kInF16);
  }
#undef W4A16_SIMPLE
  return hipGetLastError();
}

// MXFP4 W4A4 decode GEMM (m <= 16, k a multiple of 128 from 2048 on, any n): a weight
// stream on the block-scaled FP4 matrix instruction.  C[m, n] = sum_k
// deq(X)[m, k] deq(W)[n, k], with or without the activation quantize in the
// same launch.
//
// pimento.cloud "FP8, NVFP4 czy AWQ?", section "Dlaczego W8A8 i W4A16 to nie
// to samo?": token-by-token generation is bound by reading the weights, so W
// is streamed once.  The layout is that of the NVFP4 stream kernel: one
// workgroup of 16 waves per CU-share of ceil(n / 256) weight rows (at most 64,
// four 16-row tiles), the waves splitting k into slices of 128 NSTEP values
// and issuing all their loads at once, the 16 partial tiles added through LDS
// at the end.  Lane (r, g) = (lane % 16, lane / 16) holds, per step t, the 16
// bytes at 64 t + 16 g of weight row r of each tile: 32 values, exactly one
// MXFP4 block, which is one lane's share of a v_mfma_scale_f32_16x16x128
// operand with its E8M0 scale byte.  Nothing is dequantized: the matrix core
// applies both operands' block scales, so the products are exact and the sums
// are fp32.  The same lane holds the same 32 positions of activation row r
// (a zero operand for r >= m).  A k of more than one chunk (2048 values, or
// 4096) is split over rows of workgroups, each row's fp32 sums added by a
// second pass in order; in a short last chunk the slices past k add
// nothing.  Past 16384 weight rows the workgroups take up to 64 rows in
// whole rounds.
//
// The activations (XM):
//   kMxCodes  MXFP4 codes and scales.
//   kMxQuant  bf16 X quantized here.  MXFP4 has no tensor scale, so this
//             needs no tensor-wide maximum: each lane quantizes its own block
//             of X (amax, the smallest 2^k with amax <= 6 2^k, E2M1 codes of
//             x 2^-k) with the arithmetic of the quantize kernels and feeds
//             the codes to the matrix core directly; workgroup 0 also writes
//             them out.
//   kMxRaw    bf16 X as it is (W4A16: pimento.cloud, section "Dlaczego W8A8
//             i W4A16 to nie to samo?", only the weights are 4-bit): the
//             weights widened to bf16, v 2^e, which is exact (at most two
//             significant bits, bf16 has fp32's exponent range), and
//             v_mfma_f32_16x16x32_bf16 on the lane's 8 values per
//             instruction, the same 8 positions of the activation row.
#include <cstddef>

#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kMxCodes = 0, kMxQuant = 1, kMxRaw = 2;

constexpr int kMxWaves = 16;
constexpr int kMxTiles = 4;                           // 64 rows at most per workgroup
constexpr int kMxGroups = 256;                        // one workgroup per CU

// 4 NSTEP scale bytes of one row's slice (blocks ks0 / 32 ..), as dwords.
template <int NSTEP>
__device__ __forceinline__ void load_scale_slice(const uint8_t* p, uint32_t (&s)[NSTEP]) {
  if (NSTEP == 2) {
    const u32x2 h = *reinterpret_cast<const u32x2*>(p);
    s[0] = h.x;
    s[NSTEP - 1] = h.y;
  } else {
    s[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// 8 E2M1 values (one dword, low nibble first) times the E8M0 scale byte sb,
// as bf16.  Exact: v 2^(sb - 127) has at most two significant bits and lies
// in bf16's range but for sb = 254 with |v| >= 4.  The byte 0 (2^-127, an fp32
// subnormal) goes through fp32, 0xFF is NaN.
__device__ __forceinline__ v8bf mx_widen8_bf16(uint32_t w, uint32_t sb) {
  v8bf f;
  if (sb - 1u < 254u) {
    const float s = as_f(sb << 23);
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    f = (v8bf){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  } else {
    const float s = sb ? __builtin_nanf("") : as_f(0x00400000u);
    const v2f q0 = e2m1_unpack2<0>(w), q1 = e2m1_unpack2<1>(w);
    const v2f q2 = e2m1_unpack2<2>(w), q3 = e2m1_unpack2<3>(w);
    f = (v8bf){(__bf16)(q0.x * s), (__bf16)(q0.y * s), (__bf16)(q1.x * s), (__bf16)(q1.y * s),
               (__bf16)(q2.x * s), (__bf16)(q2.y * s), (__bf16)(q3.x * s), (__bf16)(q3.y * s)};
  }
  return f;
}

template <int NSTEP, int XM>
__global__ __launch_bounds__(64 * kMxWaves) void gemm_mx_stream(
    int m, int64_t n, int k, int rows_per_wg, const void* __restrict__ a, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs, void* __restrict__ c, int c_dtype,
    uint8_t* __restrict__ qcodes, uint8_t* __restrict__ qscales, float* __restrict__ part, int64_t pstride) {
  constexpr int NT = kMxTiles;
  constexpr bool QX = XM == kMxQuant;
  constexpr bool XB = XM != kMxCodes;                 // bf16 X loaded here
  __shared__ v4f tiles[kMxWaves][NT][64];          // the waves' partial tiles
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t nbase = (int64_t)blockIdx.x * rows_per_wg;
  int64_t nlast = nbase + rows_per_wg - 1;            // last row of this share
  if (nlast > n - 1) nlast = n - 1;
  // split k (part != nullptr): workgroup row blockIdx.y takes the 2048 NSTEP
  // values from kc0 on, and its fp32 sums go to part
  const int kc0 = (int)blockIdx.y * (kMxWaves * 128 * NSTEP);
  // k not a whole number of chunks: a slice that starts past k loads the
  // last slice again, in bounds, and adds (and writes) nothing
  const bool kdead = kc0 + wave * (128 * NSTEP) >= k;
  const int ks0 = kdead ? k - 128 * NSTEP : kc0 + wave * (128 * NSTEP);   // first value of this wave's slice
  const int64_t kbytes = k / 2, kblocks = k / 32;

  // ---- activations: row r, block ks0 / 32 + 4 t + g of step t ----------------
  const bool alive = r < m;
  const int64_t arow = alive ? r : m - 1;
  u32x4 xr[XB ? NSTEP : 1][XB ? 4 : 1];               // bf16 X, 8 values each
  u32x4 av[NSTEP];                                    // codes (kept as loaded for kMxCodes)
  uint32_t asl[NSTEP];                                // the row's 4 NSTEP scale bytes (kMxCodes)
  if (XB) {
#pragma unroll
    for (int t = 0; t < NSTEP; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xr[t][i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a) + arow * k + ks0 +
                                                   128 * t + 32 * g + 8 * i);
  } else {
#pragma unroll
    for (int t = 0; t < NSTEP; ++t)
      av[t] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a) + arow * kbytes + ks0 / 2 +
                                              64 * t + 16 * g);
    load_scale_slice<NSTEP>(as + arow * kblocks + ks0 / 32, asl);
  }

  // ---- weights: lane p loads row p's scale slice; codes per tile and step ------
  const int64_t swr = (nbase + lane <= nlast) ? nbase + lane : nlast;
  uint32_t wsl[NSTEP];
  load_scale_slice<NSTEP>(bs + swr * kblocks + ks0 / 32, wsl);
  u32x4 w[NT][NSTEP];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) {
    const int64_t wr = (nbase + 16 * tl + r <= nlast) ? nbase + 16 * tl + r : nlast;
#pragma unroll
    for (int t = 0; t < NSTEP; ++t)
      w[tl][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + wr * kbytes + ks0 / 2 + 64 * t + 16 * g));
  }

  // ---- activation operands and scale bytes -----------------------------------
  uint32_t asb[NSTEP];
  if (XM == kMxRaw) {
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) {
      asb[t] = 0u;
      av[t] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!alive) xr[t][i] = (u32x4){0u, 0u, 0u, 0u};
    }
  } else if (QX) {
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_lo(xr[t][i][j]);
          v[8 * i + 2 * j + 1] = bf16_hi(xr[t][i][j]);
        }
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; j += 2) amax = fmaxf(amax, fmaxf(fabsf(v[j]), fabsf(v[j + 1])));
      const int kx = mx_block_exponent(amax);
      const float rs = as_f((uint32_t)(127 - kx) << 23);   // 2^-k, a normal float for k in [-127, 126]
      uint32_t q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* p = v + 8 * i;
        uint32_t u = e2m1_pack2<0>(0u, p[0] * rs, p[1] * rs);
        u = e2m1_pack2<1>(u, p[2] * rs, p[3] * rs);
        u = e2m1_pack2<2>(u, p[4] * rs, p[5] * rs);
        q[i] = e2m1_pack2<3>(u, p[6] * rs, p[7] * rs);
      }
      asb[t] = (uint32_t)(kx + 127);
      av[t] = (u32x4){q[0], q[1], q[2], q[3]};
      if (blockIdx.x == 0 && alive && !kdead) {
        *reinterpret_cast<u32x4*>(qcodes + arow * kbytes + ks0 / 2 + 64 * t + 16 * g) = av[t];
        qscales[arow * kblocks + ks0 / 32 + 4 * t + g] = (uint8_t)asb[t];
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) asb[t] = (asl[t] >> (8 * g)) & 0xFFu;
  }
#pragma unroll
  for (int t = 0; t < NSTEP; ++t)
    if (!alive) av[t] = (u32x4){0u, 0u, 0u, 0u};

  // ---- products: one block-scaled MFMA per tile and step (W4A16: four bf16) ----
  v4f acc[NT];
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) acc[tl] = (v4f){0.f, 0.f, 0.f, 0.f};
  if (XM == kMxRaw) {
#pragma unroll
    for (int t = 0; t < NSTEP; ++t) {
#pragma unroll
      for (int tl = 0; tl < NT; ++tl) {
        const uint32_t sw = ((uint32_t)__shfl((int)wsl[t], 16 * tl + r) >> (8 * g)) & 0xFFu;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const v8bf fw = mx_widen8_bf16(w[tl][t][d], sw);
          acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw, __builtin_bit_cast(v8bf, xr[t][d]), acc[tl], 0, 0,
                                                            0);
        }
      }
    }
  } else
#pragma unroll
  for (int t = 0; t < NSTEP; ++t) {
    const v8i fa = {(int)av[t][0], (int)av[t][1], (int)av[t][2], (int)av[t][3], 0, 0, 0, 0};
#pragma unroll
    for (int tl = 0; tl < NT; ++tl) {
      // the weight row's scale byte, from the lane that loaded its slice
      const uint32_t sw = ((uint32_t)__shfl((int)wsl[t], 16 * tl + r) >> (8 * g)) & 0xFFu;
      const v8i fw = {(int)w[tl][t][0], (int)w[tl][t][1], (int)w[tl][t][2], (int)w[tl][t][3], 0, 0, 0, 0};
      acc[tl] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw, fa, acc[tl], 4, 4, 0, (int)sw, 0,
                                                                  (int)asb[t]);
    }
  }

  // ---- add the 16 slices, store ------------------------------------------------
#pragma unroll
  for (int tl = 0; tl < NT; ++tl) tiles[wave][tl][lane] = kdead ? (v4f){0.f, 0.f, 0.f, 0.f} : acc[tl];
  __syncthreads();
  if (tid < 64 * NT) {                                // thread -> (tile, lane)
    const int tl = tid >> 6, l = tid & 63;
    v4f sum = tiles[0][tl][l];
#pragma unroll
    for (int wv = 1; wv < kMxWaves; ++wv) sum += tiles[wv][tl][l];
    // D layout: lane l holds weight rows 4 (l / 16) + e of the tile, activation row l % 16
    const int xrw = l & 15, lr = 16 * tl + 4 * (l >> 4);
    const int64_t ni = nbase + lr;
    if (xrw < m && lr < rows_per_wg && ni <= nlast) {
      const int64_t o = (int64_t)xrw * n + ni;
      if (part) {
        float* pp = part + (int64_t)blockIdx.y * pstride + o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (lr + e < rows_per_wg && ni + e <= nlast) pp[e] = sum[e];
      } else if (c_dtype != kInF32 && lr + 3 < rows_per_wg && ni + 3 <= nlast && (o & 3) == 0) {
        const __bf16 h[4] = {(__bf16)sum[0], (__bf16)sum[1], (__bf16)sum[2], (__bf16)sum[3]};
        *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(c) + o) = *reinterpret_cast<const u32x2*>(h);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (lr + e < rows_per_wg && ni + e <= nlast) {
            if (c_dtype == kInF32) reinterpret_cast<float*>(c)[o + e] = sum[e];
            else reinterpret_cast<__bf16*>(c)[o + e] = (__bf16)sum[e];
          }
        }
      }
    }
  }
}

// Chunks of k for up to 16 activation rows (gemm_stream_chunks: chunks of
// 2048 values, of 4096 for a multiple of 4096 or a k up to 4096 that is a
// multiple of 256; the last one possibly short), at most 64; 0 for any
// other shape.  Any n.
int mx_chunks(int64_t m, int64_t n, int64_t k) {
  if (m < 1 || m > 16 || n < 1) return 0;
  const int64_t s = gemm_stream_chunks(k);
  return s <= 64 ? (int)s : 0;
}

// One launch for up to 16 activation rows; nsplit > 1: k in nsplit chunks,
// the chunks' fp32 sums in part, added by the reduction pass.
template <int XM>
hipError_t launch_mx_stream(int m, int64_t n, int k, const void* a, const uint8_t* as, const uint8_t* b,
                            const uint8_t* bs, void* c, int c_dtype, uint8_t* qcodes, uint8_t* qscales,
                            int nsplit, float* part, hipStream_t stream) {
  const bool nstep2 = k % 4096 == 0 || (k > 2048 && k <= 4096 && k % 256 == 0);   // chunks of 4096
  // one workgroup per CU-share of rows; with a split or past 16384 rows, as
  // many rows (at most 64) as fill whole rounds of co-resident workgroups
  // (two per CU with NSTEP = 1, one with NSTEP = 2)
  int rows = (int)((n + kMxGroups - 1) / kMxGroups);
  if (nsplit > 1 || n > 16 * kMxTiles * kMxGroups) {
    const int64_t slots = nstep2 ? kMxGroups : 2 * kMxGroups, rmax = 16 * kMxTiles;
    const int64_t rounds = (((n + rmax - 1) / rmax) * nsplit + slots - 1) / slots;
    const int64_t per_chunk = rounds * slots / nsplit;
    rows = (int)((n + per_chunk - 1) / per_chunk);
  }
  const dim3 grid((unsigned)((n + rows - 1) / rows), (unsigned)nsplit);
  const int64_t pstride = nsplit > 1 ? gemm_split_stride(m, n) : 0;
  if (nstep2)
    hipLaunchKernelGGL((gemm_mx_stream<2, XM>), grid, dim3(64 * kMxWaves), 0, stream, m, n, k, rows, a, as, b,
                       bs, c, c_dtype, qcodes, qscales, part, pstride);
  else
    hipLaunchKernelGGL((gemm_mx_stream<1, XM>), grid, dim3(64 * kMxWaves), 0, stream, m, n, k, rows, a, as, b,
                       bs, c, c_dtype, qcodes, qscales, part, pstride);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && nsplit > 1) e = launch_split_reduce(part, nsplit, m, n, nullptr, nullptr, c, c_dtype, stream);
  return e;
}

bool aligned_to(const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) == 0; }

}  // namespace

size_t gemm_mx_stream_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const int64_t mc = m < 16 ? m : 16;
  const int s = mx_chunks(mc, n, k);
  return s > 1 ? (size_t)s * (size_t)gemm_split_stride(mc, n) * sizeof(float) : 0;
}

bool launch_gemm_mx_decode(int64_t m, int64_t n, int64_t k, const uint8_t* a_codes,
                           const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                           void* c, int c_dtype, void* workspace, hipStream_t stream, hipError_t* err) {
  const int s = mx_chunks(m, n, k);
  if (!(s > 0 && aligned_to(a_codes, 16) && aligned_to(b_codes, 16) && aligned_to(a_scales, 8) &&
        aligned_to(b_scales, 8)))
    return false;
  *err = launch_mx_stream<kMxCodes>((int)m, n, (int)k, a_codes, a_scales, b_codes, b_scales, c, c_dtype, nullptr,
                                    nullptr, s, reinterpret_cast<float*>(workspace), stream);
  return true;
}

bool launch_quantize_gemm_mx_decode(int64_t m, int64_t n, int64_t k, const void* x, uint8_t* a_codes,
                                    uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                                    void* c, int c_dtype, void* workspace, hipStream_t stream, hipError_t* err) {
  const int s = mx_chunks(m, n, k);
  if (!(s > 0 && aligned_to(x, 16) && aligned_to(a_codes, 16) && aligned_to(b_codes, 16) &&
        aligned_to(b_scales, 8)))
    return false;
  *err = launch_mx_stream<kMxQuant>((int)m, n, (int)k, x, nullptr, b_codes, b_scales, c, c_dtype, a_codes,
                                    a_scales, s, reinterpret_cast<float*>(workspace), stream);
  return true;
}

bool launch_gemm_w4a16_mx(int64_t m, int64_t n, int64_t k, const void* x, const uint8_t* b_codes,
                          const uint8_t* b_scales, void* c, int c_dtype, void* workspace, hipStream_t stream,
                          hipError_t* err) {
  const int s = mx_chunks(1, n, k);
  if (!(s > 0 && aligned_to(x, 16) && aligned_to(b_codes, 16) && aligned_to(b_scales, 8))) return false;
  // 16 activation rows per launch; a split k's partial sums reuse the
  // workspace for the next 16 rows in stream order
  const int64_t osz = c_dtype == kInF32 ? 4 : 2;
  *err = hipSuccess;
  for (int64_t i0 = 0; i0 < m && *err == hipSuccess; i0 += 16) {
    const int mc = (int)(m - i0 < 16 ? m - i0 : 16);
    const uint16_t* xa = reinterpret_cast<const uint16_t*>(x) + i0 * k;
    void* ca = reinterpret_cast<char*>(c) + i0 * n * osz;
    *err = launch_mx_stream<kMxRaw>(mc, n, (int)k, xa, nullptr, b_codes, b_scales, ca, c_dtype, nullptr, nullptr, s,
                                    reinterpret_cast<float*>(workspace), stream);
  }
  return true;
}

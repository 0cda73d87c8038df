// W4A4 GEMM for many activation rows (prefill / large m) on gfx950.
//
// C[m, n] = sum_k deq(A)[m, k] deq(B)[n, k], A = activations [m, k], B =
// weights [n, k], both quantized along k (pimento.cloud "FP8, NVFP4 czy
// AWQ?", section "Dlaczego W8A8 i W4A16 to nie to samo?": W4A4 runs the
// products on low-precision matrix units).
//
// Tiling: one 256-thread workgroup computes a 256 x 256 tile of C; its four
// waves own 128 x 128 quadrants.  k advances in stages of 256 values; the
// packed codes (128 bytes per row per stage) and the scale bytes of A and B
// for a stage sit in LDS, double buffered, written from registers that were
// loaded one stage ahead with coalesced 16-byte loads.  In LDS the 16-byte
// chunk c of a row r is stored at c ^ (r & 7), which spreads the 32-row MFMA
// fragment reads over all banks.
//
// MXFP4 (E8M0 scale per 32 values): v_mfma_scale_f32_32x32x64_f8f6f4 with
// both operands E2M1.  Lane (row r, half h) of an MFMA holds 32 values; in
// step s (0..3) of a stage it holds block 4h + s, so the four scale bytes it
// needs in a stage form one dword and the instruction's op_sel picks byte s.
// NVFP4 (E4M3 scale per 16 values): each 8-value fragment is decoded to
// fp16 and multiplied by its block scale in fp16 (exact: at most 6
// significant bits, range [2^-10, 2688]); v_mfma_f32_32x32x16_f16
// accumulates in fp32 and the epilogue applies the two FP32 tensor scales.
// Lane half h owns values [128h, 128h + 128) of a stage, 8 per step.
//
// Workgroup -> tile mapping is XCD-aware: consecutive workgroup ids land on
// different XCDs (each with its own L2), so the ids are regrouped to give
// every XCD a contiguous run of tiles, ordered m-fastest, so that the tiles
// sharing a weight slab run on the same L2.
#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 256;
constexpr int ROWB = BK / 2;          // code bytes per row per stage
constexpr int NXCD = 8;

template <int FMT>
struct LargeStage {
  static constexpr int SPR = (FMT == kFmtNV) ? BK / 16 : BK / 32;   // scale bytes per row
  uint8_t a[BM * ROWB];
  uint8_t b[BN * ROWB];
  uint8_t as[BM * SPR];
  uint8_t bs[BN * SPR];
};

__device__ __forceinline__ int swz8(int row, int chunk) { return chunk ^ (row & 7); }

// Scaled fp4 MFMA whose scale byte (op_sel) is step ks of the lane's dword;
// ks is an unrolled loop index, so the switch folds to one instruction.
__device__ __forceinline__ v16f mfma_mx(int ks, v8i a, v8i b, v16f c, int sa, int sb) {
  switch (ks) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 1, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 2, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 3, sa, 3, sb);
  }
}

__device__ __forceinline__ v8h dequant8(uint32_t w, _Float16 s) {
  const v2h sv = {s, s};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sv;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sv;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sv;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sv;
  return (v8h){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

template <int FMT>
__global__ __launch_bounds__(256, 1) void gemm_large(
    int64_t m, int64_t n, int64_t k, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const float* __restrict__ at,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs,
    const float* __restrict__ bt, void* __restrict__ c, int c_dtype,
    int tiles_m, int tiles_n) {
  using Stage = LargeStage<FMT>;
  constexpr int SPR = Stage::SPR;
  __shared__ __attribute__((aligned(16))) Stage st[2];

  // ---- tile from workgroup id (XCD-aware) --------------------------------
  const int ntiles = tiles_m * tiles_n;
  const int wg = blockIdx.x;
  int tile = wg;
  if (ntiles % NXCD == 0) tile = (wg % NXCD) * (ntiles / NXCD) + wg / NXCD;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t kbytes = k / 2, srow = (FMT == kFmtNV) ? k / 16 : k / 32;
  const int nstages = (int)(k / BK);

  // ---- global -> register staging for one stage --------------------------
  // codes: 2048 16-byte chunks per operand, 8 per thread; chunk q = tid + 256 i
  // is row q / 8, column chunk q % 8 (a wave covers 8 full 128-byte rows).
  u32x4 ra[8], rb[8];
  uint32_t rsa[SPR / 4], rsb[SPR / 4];      // this thread's row of scale bytes
  // Buffer resources: one scalar descriptor per operand and a 32-bit row
  // offset per load (the operands are below 2 GiB); the stage offset goes in
  // the scalar soffset.
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, (int)(m * kbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)b, (short)0, (int)(n * kbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_as = __builtin_amdgcn_make_buffer_rsrc((void*)as, (short)0, (int)(m * srow), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_bs = __builtin_amdgcn_make_buffer_rsrc((void*)bs, (short)0, (int)(n * srow), 0x00020000);
  const int64_t arow_s = (m0 + tid < m) ? m0 + tid : m - 1;   // scale row (one per thread)
  const int64_t brow_s = (n0 + tid < n) ? n0 + tid : n - 1;
  const int sa_off = (int)(arow_s * srow), sb_off = (int)(brow_s * srow);
  auto load_stage = [&](int sidx) {
    const int kb = sidx * ROWB;                                // byte offset in a row
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i, row = q >> 3, cc = q & 7;
      const int64_t ar = (m0 + row < m) ? m0 + row : m - 1;
      const int64_t br = (n0 + row < n) ? n0 + row : n - 1;
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rs_a, (int)(ar * kbytes) + cc * 16, kb, 0);
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rs_b, (int)(br * kbytes) + cc * 16, kb, 2);
    }
    const int sbo = sidx * SPR;
    if (SPR == 16) {
      const u32x4 va = __builtin_amdgcn_raw_buffer_load_b128(rs_as, sa_off, sbo, 0);
      const u32x4 vb = __builtin_amdgcn_raw_buffer_load_b128(rs_bs, sb_off, sbo, 0);
#pragma unroll
      for (int j = 0; j < SPR / 4; ++j) { rsa[j] = va[j]; rsb[j] = vb[j]; }
    } else {
      const u32x2 va = __builtin_amdgcn_raw_buffer_load_b64(rs_as, sa_off, sbo, 0);
      const u32x2 vb = __builtin_amdgcn_raw_buffer_load_b64(rs_bs, sb_off, sbo, 0);
#pragma unroll
      for (int j = 0; j < SPR / 4; ++j) { rsa[j] = va[j]; rsb[j] = vb[j]; }
    }
  };
  auto store_stage = [&](Stage& S) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i, row = q >> 3, cc = q & 7;
      *reinterpret_cast<u32x4*>(&S.a[row * ROWB + swz8(row, cc) * 16]) = ra[i];
      *reinterpret_cast<u32x4*>(&S.b[row * ROWB + swz8(row, cc) * 16]) = rb[i];
    }
#pragma unroll
    for (int j = 0; j < SPR / 4; ++j) {
      reinterpret_cast<uint32_t*>(&S.as[tid * SPR])[j] = rsa[j];
      reinterpret_cast<uint32_t*>(&S.bs[tid * SPR])[j] = rsb[j];
    }
  };

  // ---- accumulators: 4 x 4 tiles of 32 x 32 per wave ---------------------
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5;
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  load_stage(0);
  store_stage(st[0]);
  if (nstages > 1) load_stage(1);
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    Stage& S = st[s & 1];
    if (FMT == kFmtMX) {
      int sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa[i] = *reinterpret_cast<const int*>(&S.as[(wm * 128 + 32 * i + r) * SPR + 4 * h]);
        sb[i] = *reinterpret_cast<const int*>(&S.bs[(wn * 128 + 32 * i + r) * SPR + 4 * h]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 fb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rb_ = wn * 128 + 32 * j + r;
          fb[j] = *reinterpret_cast<const u32x4*>(&S.b[rb_ * ROWB + swz8(rb_, 4 * h + ks) * 16]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ra_ = wm * 128 + 32 * i + r;
          const u32x4 va = *reinterpret_cast<const u32x4*>(&S.a[ra_ * ROWB + swz8(ra_, 4 * h + ks) * 16]);
          const v8i fa = {(int)va[0], (int)va[1], (int)va[2], (int)va[3], 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v8i fbj = {(int)fb[j][0], (int)fb[j][1], (int)fb[j][2], (int)fb[j][3], 0, 0, 0, 0};
            acc[i][j] = mfma_mx(ks, fa, fbj, acc[i][j], sa[i], sb[j]);
          }
        }
      }
    } else {
      // scales: blocks 8h .. 8h+7 of this stage for each of the 4 row tiles
      u32x2 sa2[4], sb2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa2[i] = *reinterpret_cast<const u32x2*>(&S.as[(wm * 128 + 32 * i + r) * SPR + 8 * h]);
        sb2[i] = *reinterpret_cast<const u32x2*>(&S.bs[(wn * 128 + 32 * i + r) * SPR + 8 * h]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {              // 16-byte code chunk 4h + q: 4 steps
        u32x4 ca[4], cb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ra_ = wm * 128 + 32 * i + r, rb_ = wn * 128 + 32 * i + r;
          ca[i] = *reinterpret_cast<const u32x4*>(&S.a[ra_ * ROWB + swz8(ra_, 4 * h + q) * 16]);
          cb[i] = *reinterpret_cast<const u32x4*>(&S.b[rb_ * ROWB + swz8(rb_, 4 * h + q) * 16]);
        }
        // blocks 2q and 2q+1 of this lane's 8: bytes 2q, 2q+1 of the scale pair
        v2h sca[4], scb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t wa = sa2[i][q >> 1], wb = sb2[i][q >> 1];
          sca[i] = (q & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa, 1.0f, true)
                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa, 1.0f, false);
          scb[i] = (q & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb, 1.0f, true)
                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb, 1.0f, false);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {            // 8 values per dword = half a block
          v8h fa[4], fb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            fa[i] = dequant8(ca[i][d], d < 2 ? sca[i].x : sca[i].y);
            fb[i] = dequant8(cb[i][d], d < 2 ? scb[i].x : scb[i].y);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (s + 1 < nstages) {
      store_stage(st[(s + 1) & 1]);
      if (s + 2 < nstages) load_stage(s + 2);
    }
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------
  // 32x32 D layout: lane holds column lane % 32, register e holds row
  // 8 * (e / 4) + 4 * (lane / 32) + e % 4.
  const float ts = (FMT == kFmtNV) ? (*at) * (*bt) : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + r;
      if (col >= n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row < m) {
          const float v = acc[i][j][e] * ts;
          if (c_dtype == kInF32) reinterpret_cast<float*>(c)[row * n + col] = v;
          else reinterpret_cast<__bf16*>(c)[row * n + col] = (__bf16)v;
        }
      }
    }
}

}  // namespace

bool gemm_large_supported(int fmt, int64_t m, int64_t n, int64_t k) {
  (void)fmt;
  const int64_t lim = int64_t(1) << 31;     // 32-bit buffer offsets
  return m >= 128 && n >= 128 && k % BK == 0 && m * (k / 2) < lim && n * (k / 2) < lim;
}

hipError_t launch_gemm_large(int fmt, int64_t m, int64_t n, int64_t k,
                             const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tscale, const uint8_t* b_codes,
                             const uint8_t* b_scales, const float* b_tscale,
                             void* c, int c_dtype, hipStream_t stream) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  if (fmt == kFmtMX) {
    hipLaunchKernelGGL((gemm_large<kFmtMX>), grid, dim3(256), 0, stream, m, n, k, a_codes,
                       a_scales, a_tscale, b_codes, b_scales, b_tscale, c, c_dtype, tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL((gemm_large<kFmtNV>), grid, dim3(256), 0, stream, m, n, k, a_codes,
                       a_scales, a_tscale, b_codes, b_scales, b_tscale, c, c_dtype, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

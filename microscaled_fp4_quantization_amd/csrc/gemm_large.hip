// W4A4 GEMM for many activation rows (prefill / large m) on gfx950.
//
// C[m, n] = sum_k deq(A)[m, k] deq(B)[n, k], A = activations [m, k], B =
// weights [n, k], both quantized along k (pimento.cloud "FP8, NVFP4 czy
// AWQ?", section "Dlaczego W8A8 i W4A16 to nie to samo?": W4A4 runs the
// products on low-precision matrix units).
//
// Tiling: a workgroup computes a 256 x 256 tile of C with WMW x WNW waves.
// k advances in stages of 128 values (64 code bytes per row).  Stages live
// in a 4-deep LDS ring filled by direct global->LDS buffer loads, so three
// stages are in flight while one is multiplied and no registers are spent on
// staging.  A direct load writes lane i's 16 bytes at base + 16 i, so the LDS
// layout is chosen through the global addresses: in a row r, 16-byte chunk c
// is stored at position c ^ ((r >> 2) & 3), which keeps the 32-row MFMA
// fragment reads at the minimum number of bank cycles.
//
// Scales travel in groups of 16 bytes per row (4 stages of MXFP4, 2 of
// NVFP4), one 16-byte load per lane, into a 3-slot LDS ring of their own:
// fetching a stage's 4 or 8 scale bytes per row on its own would cost one
// memory request per row for a few bytes, and the request rate, not the
// byte rate, bounds the operand stream.  Group g + 2 is fetched once the
// stages of group g - 1 are consumed.
//
// MXFP4 (E8M0 scale per 32 values): v_mfma_scale_f32_32x32x64_f8f6f4, both
// operands E2M1.  In k-step ks (0, 1) of a stage, lane (row r, half h)
// holds block 2h + ks; its two scale bytes are shifted into the low half of
// the scale register so the instruction's op_sel is the constant ks.
// NVFP4 (E4M3 scale per 16 values): fragments are decoded to fp16 and
// multiplied by their block scale in fp16 (exact: at most 6 significant
// bits, range [2^-10, 2688]); v_mfma_f32_32x32x16_f16 accumulates in fp32;
// the two FP32 tensor scales are applied in the epilogue.  Lane half h owns
// values [64h, 64h + 64) of a stage (blocks 4h .. 4h+3), 8 per k-step.
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int ROWB = BK / 2;          // code bytes per row per stage
constexpr int NSTAGE = 4;             // LDS ring depth
constexpr int NXCD = 8;
// waves per workgroup along m and n
constexpr int kMXWM = 2, kMXWN = 4;
constexpr int kNVWM = 2, kNVWN = 4;

constexpr int NSGRP = 3;              // scale-group ring depth

struct LargeStage {
  uint8_t a[BM * ROWB];
  uint8_t b[BN * ROWB];
};

// One scale group: 4 words (16 bytes) per row, rows contiguous, A then B.
struct ScaleGroup {
  uint32_t w[2][BM * 4];
};

// All of a workgroup's LDS in one object: the loop's explicit vmcnt waits and
// barriers order the direct loads against the reads, and with a single
// object the compiler adds no waits of its own (with several, it drains
// every load in flight before the first read of the object a load targets).
struct LargeSmem {
  LargeStage st[NSTAGE];
  ScaleGroup sg[NSGRP];
};

// stages per scale group: 16 bytes per row hold 4 MXFP4 stages (one E8M0
// byte per 32 values) or 2 NVFP4 stages (one E4M3 byte per 16 values)
template <int FMT>
constexpr int stages_per_group() { return FMT == kFmtNV ? 2 : 4; }

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// Scaled fp4 MFMA whose scale byte (op_sel) is the k-step ks; ks is an
// unrolled loop index, so the branch folds to one instruction.
__device__ __forceinline__ v16f mfma_mx(int ks, v8i a, v8i b, v16f c, int sa, int sb) {
  if (ks == 0) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 1, sa, 1, sb);
}

__device__ __forceinline__ v8h dequant8(uint32_t w, _Float16 s) {
  const v2h sv = {s, s};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sv;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sv;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sv;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sv;
  return (v8h){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Direct buffer -> LDS load of SIZE bytes per lane (lane i writes lds + SIZE i).
// Kept out of the host compilation pass: there the builtin makes clang drop
// the kernel template's host stub.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, void* lds, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, soff, 0, 0);
#endif
}
__device__ __forceinline__ void load_lds16_nt(__amdgpu_buffer_rsrc_t rs, void* lds, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, soff, 0, 2);
#endif
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // vmcnt N (N < 64); expcnt and lgkmcnt at their maximum (no wait)
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int FMT, int WMW, int WNW>
__global__ __launch_bounds__(64 * WMW * WNW, 1) void gemm_large(
    int m, int n, int k, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const float* __restrict__ at,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs,
    const float* __restrict__ bt, void* __restrict__ c, int c_dtype,
    int tiles_m, int tiles_n) {
  using Stage = LargeStage;
  constexpr int G = stages_per_group<FMT>();
  constexpr int NW = WMW * WNW;                // waves
  constexpr int NL = BM * ROWB / 1024 / NW;    // 1 KiB code blocks per operand per wave
  constexpr int NSG = 8 / NW;                  // 1 KiB scale-group blocks (A and B) per wave
  constexpr int TM = BM / WMW, TN = BN / WNW;  // wave tile
  constexpr int TI = TM / 32, TJ = TN / 32;    // 32x32 MFMA tiles per wave
  static_assert(BM == BN && NL * NW * 1024 == BM * ROWB && NSG * NW == 8 && 4 * NL + 2 * NSG < 64, "tile shape");
  __shared__ __attribute__((aligned(16))) LargeSmem smem;
  Stage* st = smem.st;
  ScaleGroup* sgr = smem.sg;

  // ---- tile from workgroup id (XCD-aware) --------------------------------
  const int ntiles = tiles_m * tiles_n;
  const int wg = blockIdx.x;
  int tile = wg;
  if (ntiles % NXCD == 0) tile = (wg % NXCD) * (ntiles / NXCD) + wg / NXCD;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int kbytes = k / 2, srow = (FMT == kFmtNV) ? k / 16 : k / 32;
  const int nstages = k / BK;
  const int ngroups = (nstages + G - 1) / G;

  // ---- direct global -> LDS loads of one stage ----------------------------
  // Code block q (1 KiB = 16 rows x 64 bytes) of an operand: lane p fills
  // position p, i.e. row 16 q + p / 4, stored chunk p % 4, which holds the
  // logical chunk (p % 4) ^ ((row >> 2) & 3).  All offsets are 32-bit: the
  // operands are below 2 GiB.  Rows past m or n re-read the last row.
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, m * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)b, (short)0, n * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_as = __builtin_amdgcn_make_buffer_rsrc((void*)as, (short)0, m * srow, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_bs = __builtin_amdgcn_make_buffer_rsrc((void*)bs, (short)0, n * srow, 0x00020000);
  int voff_a[NL], voff_b[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int q = i * NW + wave;
    const int row = 16 * q + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    const int ar = (m0 + row < m) ? m0 + row : m - 1;
    const int br = (n0 + row < n) ? n0 + row : n - 1;
    voff_a[i] = ar * kbytes + chunk * 16;
    voff_b[i] = br * kbytes + chunk * 16;
  }
  // Scale-group block j of this wave: g = j * NW + wave selects the operand
  // (g / 4) and rows 64 (g % 4) .. + 63; lane p loads row 64 (g % 4) + p.
  int voff_s[NSG];
#pragma unroll
  for (int j = 0; j < NSG; ++j) {
    const int g = j * NW + wave;
    const bool isb = g >= 4;
    const int row = 64 * (g % 4) + lane;
    const int lim = isb ? n : m, base = isb ? n0 : m0;
    const int rr = (base + row < lim) ? base + row : lim - 1;
    voff_s[j] = rr * srow;
  }
  // Stage sidx into ring slot `slot`.
  auto issue_stage = [&](int slot, int sidx) {
    Stage& S = st[slot];
    const int kb = sidx * ROWB;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = i * NW + wave;
      load_lds16(rs_a, &S.a[q * 1024], voff_a[i], kb);
      load_lds16_nt(rs_b, &S.b[q * 1024], voff_b[i], kb);
    }
  };
  // Scale group gidx into scale slot `slot` (16-byte aligned: the row pitch
  // is a multiple of 16 bytes and nstages a multiple of G).
  auto issue_group = [&](int slot, int gidx) {
#pragma unroll
    for (int j = 0; j < NSG; ++j) {
      const int g = j * NW + wave;
      const bool isb = g >= 4;
      load_lds16(isb ? rs_bs : rs_as, &sgr[slot].w[isb][256 * (g % 4)], voff_s[j], 16 * gidx);
    }
  };

  // ---- accumulators: TI x TJ tiles of 32 x 32 per wave -------------------
  const int wm = wave / WNW, wn = wave % WNW;
  const int r = lane & 31, h = lane >> 5;
  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Prologue, in the order the steady state would have issued it: iteration
  // i issues code stage i + 3 and, when i % G == 0, scale group i / G + 2, so
  // the virtual iterations -2G, -G, -3, -2, -1 give groups 0 and 1 and
  // stages 0, 1, 2 (indexes clamped; a repeated stage or group is never
  // read).
  issue_group(0, 0);
  if (G == 2) {
    issue_stage(0, 0);
    issue_stage(1, nstages > 1 ? 1 : 0);
    issue_group(1, ngroups > 1 ? 1 : 0);
    issue_stage(2, nstages > 2 ? 2 : nstages - 1);
  } else {
    issue_group(1, ngroups > 1 ? 1 : 0);
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p) issue_stage(p, p < nstages ? p : nstages - 1);
  }

  // Every iteration waits for the oldest stage and issues exactly one more
  // (near the end a repeat of the last stage into the free slot), so the loop
  // body has no data-dependent branch and the accumulators stay in place.
  for (int s = 0; s < nstages; ++s) {
    // This thread's loads of stage s (and of its scale group, issued earlier)
    // have landed.  Issued after them: stages s + 1 and s + 2 and the groups
    // issued in iterations s - 3 .. s - 1, one for each multiple of G there.
    if (G == 4) {
      if ((s & 3) == 0) wait_vm<4 * NL>();
      else wait_vm<4 * NL + NSG>();
    } else {
      if ((s & 1) == 0) wait_vm<4 * NL + NSG>();
      else wait_vm<4 * NL + 2 * NSG>();
    }
    // Every wave's part of stage s has landed and stage s-1 is consumed.  A
    // bare s_barrier: __syncthreads() would also drain the loads of the later
    // stages still in flight.  The memory clobber keeps the compiler from
    // moving LDS reads across it.
    __asm__ volatile("s_barrier" ::: "memory");
    const int nxt = s + NSTAGE - 1;
    issue_stage(nxt % NSTAGE, nxt < nstages ? nxt : nstages - 1);
    const int grp = s / G;
    if (s % G == 0) {
      // group grp - 1 is consumed: its slot takes group grp + 2
      const int gn = grp + 2;
      issue_group(gn % NSGRP, gn < ngroups ? gn : ngroups - 1);
    }
    const Stage& S = st[s % NSTAGE];
    const ScaleGroup& SG = sgr[grp % NSGRP];
    const int sw = (s % G) * (4 / G);            // first scale word of stage s

    if (FMT == kFmtMX) {
      int sa[TI], sb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) sa[i] = (int)(SG.w[0][4 * (wm * TM + 32 * i + r) + sw] >> (16 * h));
#pragma unroll
      for (int j = 0; j < TJ; ++j) sb[j] = (int)(SG.w[1][4 * (wn * TN + 32 * j + r) + sw] >> (16 * h));
      // all fragments of the stage first: one LDS wait instead of one per tile
      u32x4 fa[2][TI], fb[2][TJ];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int rb = wn * TN + 32 * j + r;
          fb[ks][j] = *reinterpret_cast<const u32x4*>(&S.b[rb * ROWB + swz(rb, 2 * h + ks) * 16]);
        }
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int ra = wm * TM + 32 * i + r;
          fa[ks][i] = *reinterpret_cast<const u32x4*>(&S.a[ra * ROWB + swz(ra, 2 * h + ks) * 16]);
        }
      }
      // Keep the reads ahead of the MFMAs as one block: interleaving them in
      // small groups leaves the matrix pipe idle on every LDS wait, while a
      // read block overlaps the MFMA block of the other wave on the SIMD.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const v8i a8 = {(int)fa[ks][i][0], (int)fa[ks][i][1], (int)fa[ks][i][2], (int)fa[ks][i][3], 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v8i b8 = {(int)fb[ks][j][0], (int)fb[ks][j][1], (int)fb[ks][j][2], (int)fb[ks][j][3], 0, 0, 0, 0};
            acc[i][j] = mfma_mx(ks, a8, b8, acc[i][j], sa[i], sb[j]);
          }
        }
    } else {
      // this lane's 4 block scales (word h of its row), decoded in pairs
      v2h sa01[TI], sa23[TI], sb01[TJ], sb23[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const uint32_t w = SG.w[0][4 * (wm * TM + 32 * i + r) + sw + h];
        sa01[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
        sa23[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const uint32_t w = SG.w[1][4 * (wn * TN + 32 * j + r) + sw + h];
        sb01[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
        sb23[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {              // code chunk 2h + q: blocks 4h + 2q, +1
        u32x4 ca[TI], cb[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int ra = wm * TM + 32 * i + r;
          ca[i] = *reinterpret_cast<const u32x4*>(&S.a[ra * ROWB + swz(ra, 2 * h + q) * 16]);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int rb = wn * TN + 32 * j + r;
          cb[j] = *reinterpret_cast<const u32x4*>(&S.b[rb * ROWB + swz(rb, 2 * h + q) * 16]);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {            // 8 values per dword
          v8h fa[TI], fb[TJ];
#pragma unroll
          for (int i = 0; i < TI; ++i) {
            const v2h sp = q ? sa23[i] : sa01[i];
            fa[i] = dequant8(ca[i][d], d < 2 ? sp.x : sp.y);
          }
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v2h sp = q ? sb23[j] : sb01[j];
            fb[j] = dequant8(cb[j][d], d < 2 ? sp.x : sp.y);
          }
#pragma unroll
          for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  wait_vm<0>();                 // no load may land in LDS after the workgroup ends

  // ---- epilogue -----------------------------------------------------------
  // 32x32 D layout: lane holds column lane % 32, register e holds row
  // 8 * (e / 4) + 4 * (lane / 32) + e % 4.
  const float ts = (FMT == kFmtNV) ? (*at) * (*bt) : 1.0f;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = n0 + wn * TN + 32 * j + r;
      if (col >= n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * TM + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row < m) {
          const float v = acc[i][j][e] * ts;
          const int64_t idx = (int64_t)row * n + col;
          if (c_dtype == kInF32) reinterpret_cast<float*>(c)[idx] = v;
          else reinterpret_cast<__bf16*>(c)[idx] = (__bf16)v;
        }
      }
    }
}

}  // namespace

bool gemm_large_supported(int fmt, int64_t m, int64_t n, int64_t k) {
  const int64_t lim = int64_t(1) << 31;     // 32-bit buffer offsets
  // 16-byte scale rows: k a multiple of 512 (MXFP4) or 256 (NVFP4)
  const int64_t kq = (fmt == kFmtNV) ? 256 : 512;
  return m >= 128 && n >= 128 && k % kq == 0 && m * (k / 2) < lim && n * (k / 2) < lim;
}

hipError_t launch_gemm_large(int fmt, int64_t m, int64_t n, int64_t k,
                             const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tscale, const uint8_t* b_codes,
                             const uint8_t* b_scales, const float* b_tscale,
                             void* c, int c_dtype, hipStream_t stream) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  if (fmt == kFmtMX) {
    hipLaunchKernelGGL((gemm_large<kFmtMX, kMXWM, kMXWN>), grid, dim3(64 * kMXWM * kMXWN), 0, stream,
                       (int)m, (int)n, (int)k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                       b_tscale, c, c_dtype, tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL((gemm_large<kFmtNV, kNVWM, kNVWN>), grid, dim3(64 * kNVWM * kNVWN), 0, stream,
                       (int)m, (int)n, (int)k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                       b_tscale, c, c_dtype, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

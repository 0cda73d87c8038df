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
#include <type_traits>

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
constexpr int kMXWM = 2, kMXWN = 2;
constexpr int kNVWM = 2, kNVWN = 2;

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

__device__ __forceinline__ void wait_lgkm0() {
  // lgkmcnt 0; vmcnt and expcnt at their maximum (no wait)
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // vmcnt N (N < 64); expcnt and lgkmcnt at their maximum (no wait)
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Fragments of one stage for one wave: code chunks x = 0, 1 of its A rows
// and B columns (MXFP4: k-step x; NVFP4: chunk 2h + x), and the lane's scale
// word per row (MXFP4: the stage's word, bytes 2h and 2h + 1 are this lane's;
// NVFP4: word h of the stage).  Nothing here consumes the loaded values, so
// the reads stay in flight while the previous stage is multiplied.
template <int TI, int TJ>
struct Frags {
  u32x4 a[2][TI];
  u32x4 b[2][TJ];
  uint32_t sa[TI];
  uint32_t sb[TJ];
};

// Writes a workgroup's 256 x 256 tile of C = ts * acc.  The MFMAs take B as
// the first operand, so in each 32x32 block a lane holds output row
// r = lane % 32 and, in registers 4g .. 4g + 3, the four consecutive columns
// 8g + 4h .. + 3.  The tile goes through LDS (ep: the workgroup's operand
// ring, free once every wave is past its last fragment read) in row-major
// order and leaves as 16-byte row chunks: direct stores of the fragments
// would scatter 2- or 4-byte pieces over 32 rows.
//
// The tile starts at row m0 and column n0; only rows >= m_lo and columns >=
// n_lo are this workgroup's (a last tile that was moved back so that all of
// its rows exist leaves the overlap to its neighbour).
template <int WMW, int WNW, int TI, int TJ>
__device__ __forceinline__ void store_tile(const v16f (&acc)[TI][TJ], uint8_t* ep, float ts,
                                           void* __restrict__ c, int c_dtype, int m, int n,
                                           int m0, int n0, int m_lo, int n_lo) {
  constexpr int NW = WMW * WNW, TM = BM / WMW, TN = BN / WNW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int r = lane & 31, h = lane >> 5;
  wait_lgkm0();
  __asm__ volatile("s_barrier" ::: "memory");
  const bool f32 = (c_dtype == kInF32);
  // bf16: the whole 256 x 256 tile, rows of 528 bytes (512 + 16: 16-byte
  // aligned, writes of the 32 rows of a block spread over the banks);
  // f32: one 128-row band (the rows of the waves with wm = band) at a time,
  // rows of 1040 bytes.
  const int pitch = f32 ? 1040 : 528;
  const int nband = f32 ? 2 : 1;
  const int band_rows = BM / nband;
  const bool vec_ok = f32 ? (n % 4 == 0) : (n % 8 == 0);
  for (int band = 0; band < nband; ++band) {
    if (!f32 || wm == band) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int row = (f32 ? 0 : wm * TM) + 32 * i + r;   // row within the band
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = wn * TN + 32 * j + 8 * g + 4 * h;
            const float v0 = acc[i][j][4 * g] * ts, v1 = acc[i][j][4 * g + 1] * ts;
            const float v2 = acc[i][j][4 * g + 2] * ts, v3 = acc[i][j][4 * g + 3] * ts;
            if (f32) {
              *reinterpret_cast<float4*>(ep + row * pitch + col * 4) = make_float4(v0, v1, v2, v3);
            } else {
              const __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1, b2 = (__bf16)v2, b3 = (__bf16)v3;
              uint2 u;
              u.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
              u.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
              *reinterpret_cast<uint2*>(ep + row * pitch + col * 2) = u;
            }
          }
        }
    }
    __syncthreads();
    // 16-byte chunks: 32 (bf16) or 64 (f32) per row
    const int cpr = f32 ? 64 : 32, epc = f32 ? 4 : 8;
    const int row0 = m0 + band * band_rows;
    for (int idx = tid; idx < band_rows * cpr; idx += 64 * NW) {
      const int lr = idx / cpr, ch = idx % cpr;
      const int grow = row0 + lr, gcol = n0 + ch * epc;
      if (grow < m_lo || grow >= m || gcol + epc <= n_lo || gcol >= n) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(ep + lr * pitch + ch * 16);
      const int64_t off = (int64_t)grow * n + gcol;
      if (vec_ok && gcol >= n_lo && gcol + epc <= n) {
        if (f32) *reinterpret_cast<uint4*>(reinterpret_cast<float*>(c) + off) = v;
        else *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(c) + off) = v;
      } else if (f32) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gcol + e >= n_lo && gcol + e < n) reinterpret_cast<uint32_t*>(c)[off + e] = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
          if (gcol + e >= n_lo && gcol + e < n) reinterpret_cast<uint16_t*>(c)[off + e] = (uint16_t)(w >> (16 * (e & 1)));
        }
      }
    }
    if (band + 1 < nband) __syncthreads();
  }
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
  static_assert(BM == BN && NL * NW * 1024 == BM * ROWB && NSG * NW == 8 && 6 * NL + 2 * NSG < 64, "tile shape");
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
  const int ngroups = nstages / G;

  // ---- direct global -> LDS loads -----------------------------------------
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
  // Code stage t (clamped to the last; a repeat is never read) into slot t % NSTAGE.
  auto issue_stage = [&](int t) {
    Stage& S = st[t % NSTAGE];
    const int kb = (t < nstages ? t : nstages - 1) * ROWB;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = i * NW + wave;
      load_lds16(rs_a, &S.a[q * 1024], voff_a[i], kb);
      load_lds16(rs_b, &S.b[q * 1024], voff_b[i], kb);
    }
  };
  // Scale group g (clamped to the last) into scale slot g % NSGRP; 16-byte
  // aligned: the row pitch is a multiple of 16 bytes and nstages of G.
  auto issue_group = [&](int g) {
    ScaleGroup& SG = sgr[g % NSGRP];
    const int gb = 16 * (g < ngroups ? g : ngroups - 1);
#pragma unroll
    for (int j = 0; j < NSG; ++j) {
      const int gw = j * NW + wave;
      const bool isb = gw >= 4;
      load_lds16(isb ? rs_bs : rs_as, &SG.w[isb][256 * (gw % 4)], voff_s[j], gb);
    }
  };

  // ---- per-wave fragments ------------------------------------------------
  const int wm = wave / WNW, wn = wave % WNW;
  const int r = lane & 31, h = lane >> 5;
  auto read_frags = [&](int t, Frags<TI, TJ>& F) {
    const Stage& S = st[t % NSTAGE];
    const ScaleGroup& SG = sgr[(t / G) % NSGRP];
    const int sw = (t % G) * (4 / G);            // first scale word of stage t
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int ra = wm * TM + 32 * i + r;
        F.a[x][i] = *reinterpret_cast<const u32x4*>(&S.a[ra * ROWB + swz(ra, 2 * h + x) * 16]);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int rb = wn * TN + 32 * j + r;
        F.b[x][j] = *reinterpret_cast<const u32x4*>(&S.b[rb * ROWB + swz(rb, 2 * h + x) * 16]);
      }
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const uint32_t* w = &SG.w[0][4 * (wm * TM + 32 * i + r) + sw];
      F.sa[i] = (FMT == kFmtMX) ? w[0] : w[h];
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const uint32_t* w = &SG.w[1][4 * (wn * TN + 32 * j + r) + sw];
      F.sb[j] = (FMT == kFmtMX) ? w[0] : w[h];
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto compute = [&](const Frags<TI, TJ>& F) {
    if (FMT == kFmtMX) {
      // this lane's two scale bytes into the low half: op_sel is then ks
      int sa[TI], sb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) sa[i] = (int)(F.sa[i] >> (16 * h));
#pragma unroll
      for (int j = 0; j < TJ; ++j) sb[j] = (int)(F.sb[j] >> (16 * h));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const v8i a8 = {(int)F.a[ks][i][0], (int)F.a[ks][i][1], (int)F.a[ks][i][2], (int)F.a[ks][i][3], 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v8i b8 = {(int)F.b[ks][j][0], (int)F.b[ks][j][1], (int)F.b[ks][j][2], (int)F.b[ks][j][3], 0, 0, 0, 0};
            acc[i][j] = mfma_mx(ks, b8, a8, acc[i][j], sb[j], sa[i]);
          }
        }
    } else {
      // this lane's 4 block scales (word h of its row), decoded in pairs
      v2h sa01[TI], sa23[TI], sb01[TJ], sb23[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        sa01[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(F.sa[i], 1.0f, false);
        sa23[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(F.sa[i], 1.0f, true);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        sb01[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(F.sb[j], 1.0f, false);
        sb23[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(F.sb[j], 1.0f, true);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {              // code chunk 2h + q: blocks 4h + 2q, +1
#pragma unroll
        for (int d = 0; d < 4; ++d) {            // 8 values per dword
          v8h fa[TI], fb[TJ];
#pragma unroll
          for (int i = 0; i < TI; ++i) {
            const v2h sp = q ? sa23[i] : sa01[i];
            fa[i] = dequant8(F.a[q][i][d], d < 2 ? sp.x : sp.y);
          }
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const v2h sp = q ? sb23[j] : sb01[j];
            fb[j] = dequant8(F.b[q][j][d], d < 2 ? sp.x : sp.y);
          }
#pragma unroll
          for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // ---- software pipeline ----------------------------------------------------
  // Iteration s: wait for stage s + 1 (this wave's loads, then everyone's at
  // the barrier, which also closes every wave's LDS reads of stage s), load
  // stage s + 4 into the slot stage s vacated, at the end of a scale group
  // load group (s + 1) / G + 2 into the slot of the group just finished,
  // read the fragments of stage s + 1, and multiply stage s from registers
  // while those reads are in flight.
  //
  // In-order completion of this wave's loads gives the wait counts.  The
  // issue order is that of the steady state from virtual iterations on:
  // iteration i loads stage i + 4 and, when (i + 1) % G == 0, group
  // (i + 1) / G + 2.  Issued after stage s + 1: stages s + 2, s + 3 and the
  // groups of iterations s - 3 .. s - 1.  A group is issued 2G + 1 > 4
  // iterations before its first stage is read, ahead of that stage's codes.
  if (G == 4) {
    issue_group(0);                              // virtual iteration -9
    issue_group(1);                              // -5
#pragma unroll
    for (int t = 0; t < 4; ++t) issue_stage(t);  // -4 .. -1
    issue_group(2);                              // -1
    wait_vm<6 * NL + NSG>();                     // stage 0, group 0
  } else {
    issue_group(0);                              // -5
    issue_stage(0);                              // -4
    issue_stage(1);                              // -3
    issue_group(1);                              // -3
    issue_stage(2);                              // -2
    issue_stage(3);                              // -1
    issue_group(2);                              // -1
    wait_vm<6 * NL + 2 * NSG>();                 // stage 0, group 0
  }
  __asm__ volatile("s_barrier" ::: "memory");
  Frags<TI, TJ> F0, F1;
  read_frags(0, F0);

  // Step J (0 .. G-1) of a trip of G stages: a compile-time position, so the
  // wait counts and the group load need no branch and the loop body stays
  // one block the compiler cannot reshuffle across the barriers.
  auto step = [&](auto J, int s, const Frags<TI, TJ>& Fc, Frags<TI, TJ>& Fn) {
    constexpr int j = decltype(J)::value;
    if constexpr (G == 4) {
      if constexpr (j == 3) wait_vm<4 * NL>();
      else wait_vm<4 * NL + NSG>();
    } else {
      if constexpr (j == 0) wait_vm<4 * NL + 2 * NSG>();
      else wait_vm<4 * NL + NSG>();
    }
    // LDS reads of stage s done in this wave (a builtin wait, which the
    // compiler's own wait insertion takes into account), then in every wave;
    // the memory clobber keeps the compiler from moving LDS accesses across.
    wait_lgkm0();
    __asm__ volatile("s_barrier" ::: "memory");
    issue_stage(s + NSTAGE);
    if constexpr (j == G - 1) issue_group((s + 1) / G + 2);
    // at s = nstages - 1 this reads the repeated last stage: valid, unused
    read_frags(s + 1, Fn);
    compute(Fc);
    // Spread the loads and LDS reads over the multiplies: a direct load can
    // stall issue while the memory pipeline drains, and in one block it
    // would idle the matrix core that long.
    if constexpr (FMT == kFmtMX) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);   // MFMA
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // nstages is a multiple of G (k is a multiple of 512 or 256)
  for (int s = 0; s < nstages; s += G) {
    step(std::integral_constant<int, 0>{}, s, F0, F1);
    step(std::integral_constant<int, 1>{}, s + 1, F1, F0);
    if constexpr (G == 4) {
      step(std::integral_constant<int, 2>{}, s + 2, F0, F1);
      step(std::integral_constant<int, 3>{}, s + 3, F1, F0);
    }
  }

  wait_vm<0>();                 // no load may land in LDS after the workgroup ends

  // ---- epilogue -----------------------------------------------------------
  const float ts = (FMT == kFmtNV) ? (*at) * (*bt) : 1.0f;
  store_tile<WMW, WNW>(acc, reinterpret_cast<uint8_t*>(&smem), ts, c, c_dtype, m, n, m0, n0, m0, n0);
}

// ---- MXFP4: 256-value stages ----------------------------------------------
// A stage holds 256 k-values of every row: 128 code bytes, so one direct
// load of 64 lanes covers 8 whole rows in full 128-byte lines.  (With
// 64-byte rows every load touches twice the lines for the same bytes, and the
// number of lines, not bytes, bounds the rate at which a CU's loads are
// served.)  Two stage slots (128 KiB) hold the ring; the fragments of half a
// stage (128 values) are read into registers while the previous half is
// multiplied, so a slot is free once the second half of its stage is in
// registers.  Scales come in groups of 32 bytes per row (4 stages) into a
// 2-slot ring of their own (32 KiB): with 16-byte groups the scale loads
// touch half as many lines as the codes and slow the stream by a third.
constexpr int MXBK = 256;                 // k values per stage
constexpr int MXROWB = MXBK / 2;          // code bytes per row per stage
constexpr int MXG = 4;                    // stages per scale group
constexpr int MXSGB = MXG * MXBK / 32;    // scale bytes per row per group

struct MxStage {
  uint8_t a[BM * MXROWB];
  uint8_t b[BN * MXROWB];
};
struct MxScaleGroup {
  uint8_t a[BM * MXSGB];
  uint8_t b[BN * MXSGB];
};
struct MxSmem {                           // 160 KiB: the whole LDS of a CU
  MxStage st[2];
  MxScaleGroup sg[2];
};

// Stored position of 16-byte code chunk c (0..7) of row r: the 16 rows a
// 16-lane read phase touches land on 16 different 16-byte bank groups.
__device__ __forceinline__ int swz_mx(int r, int c) { return c ^ ((r >> 1) & 7); }
// Stored position of 16-byte half hh of the 32-byte scale row r.
__device__ __forceinline__ int swz_mxs(int r, int hh) { return hh ^ ((r >> 3) & 1); }

template <int WMW, int WNW>
__global__ __launch_bounds__(64 * WMW * WNW, 1) void gemm_large_mx(
    int m, int n, int k, const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs, void* __restrict__ c,
    int c_dtype, int tiles_m, int tiles_n) {
  constexpr int NW = WMW * WNW;
  constexpr int NL = BM * MXROWB / 1024 / NW;        // code loads per operand per wave per stage
  constexpr int NSG = 2 * BM * MXSGB / 1024 / NW;    // scale loads per wave per group
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int TI = TM / 32, TJ = TN / 32;
  static_assert(BM == BN && NL * NW * 1024 == BM * MXROWB && NSG * NW * 1024 == 2 * BM * MXSGB, "tile shape");
  static_assert(2 * NL + NSG < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) MxSmem smem;

  const int ntiles = tiles_m * tiles_n;
  const int wg = blockIdx.x;
  int tile = wg;
  if (ntiles % NXCD == 0) tile = (wg % NXCD) * (ntiles / NXCD) + wg / NXCD;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  // A last tile that would run past m or n is moved back to end at the last
  // row or column (m, n >= 256): every row it loads exists, and the rows and
  // columns it shares with its neighbour are left to the neighbour.
  const int m_lo = tm * BM, n_lo = tn * BN;
  const int m0 = m_lo + BM <= m ? m_lo : m - BM;
  const int n0 = n_lo + BN <= n ? n_lo : n - BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kbytes = k / 2, srow = k / 32;
  const int nst = k / MXBK;                          // even: k is a multiple of 512
  const int ngr = (nst + MXG - 1) / MXG;

  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, m * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)b, (short)0, n * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_as = __builtin_amdgcn_make_buffer_rsrc((void*)as, (short)0, m * srow, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_bs = __builtin_amdgcn_make_buffer_rsrc((void*)bs, (short)0, n * srow, 0x00020000);
  // Code load i of the wave fills 1 KiB block q = i NW + wave of an operand's
  // slot: rows 8q .. 8q + 7; lane p writes row 8q + p / 8 at stored position
  // p % 8, i.e. fetches chunk (p % 8) ^ ((row >> 1) & 7), which does not
  // depend on i.  The lane's offset is that of load 0; rows 32 i further on,
  // the tile's first row and the stage go into the uniform offset.
  const int crow = 8 * wave + (lane >> 3);
  const int voff_c = crow * kbytes + swz_mx(crow, lane & 7) * 16;
  // Scale load j of the wave fills 1 KiB block g = j NW + wave of a group
  // slot: operand g / 8, rows 32 (g % 8) .. + 31, i.e. rows 32 wave + 128
  // (j % 2) of operand j / 2; lane p writes row 32 (g % 8) + p / 2 at stored
  // half p % 2, i.e. fetches half (p % 2) ^ ((row >> 3) & 1).
  static_assert(NW == 4 && NSG == 4, "scale-load mapping");
  const int srw = 32 * wave + (lane >> 1);
  const int voff_s = srw * srow;
  const int hoff_s = 16 * swz_mxs(srw, lane & 1);
  // stage t (clamped to the last; a repeat is never read) into slot t % 2
  auto issue_stage = [&](int t) {
    MxStage& S = smem.st[t & 1];
    const int kb = (t < nst ? t : nst - 1) * MXROWB;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = i * NW + wave;
      load_lds16(rs_a, &S.a[q * 1024], voff_c, (m0 + 32 * i) * kbytes + kb);
      load_lds16(rs_b, &S.b[q * 1024], voff_c, (n0 + 32 * i) * kbytes + kb);
    }
  };
  // scale group g (clamped to the last) into group slot g % 2.  A last group
  // of two stages has only its first half inside the row: the second half
  // then repeats the first and is never read.
  auto issue_group = [&](int g) {
    MxScaleGroup& SG = smem.sg[g & 1];
    const int gc = g < ngr ? g : ngr - 1;
    const int gb = MXSGB * gc;
    const bool whole = gb + MXSGB <= srow;
    const int vo = voff_s + (whole ? hoff_s : 0);
#pragma unroll
    for (int j = 0; j < NSG; ++j) {
      const int gw = j * NW + wave;
      const bool isb = j >= 2;
      load_lds16(isb ? rs_bs : rs_as, (isb ? SG.b : SG.a) + 1024 * (gw % 8), vo,
                 ((isb ? n0 : m0) + 128 * (j & 1)) * srow + gb);
    }
  };

  const int wm = wave / WNW, wn = wave % WNW;
  const int r = lane & 31, h = lane >> 5;
  // Half-stage u = 2 t + x: values [128 x, 128 x + 128) of stage t, k-steps
  // ks = 0, 1 of 64 values.  Lane (r, h) takes chunk 4 x + 2 ks + h of its
  // rows (block 4 x + 2 ks + h of the stage) and the scale word x of the
  // stage's 8 scale bytes, whose bytes 2 ks + h it uses.
  auto read_frags = [&](int u, Frags<TI, TJ>& F) {
    const int t = u >> 1, x = u & 1;
    const MxStage& S = smem.st[t & 1];
    const MxScaleGroup& SG = smem.sg[(t / MXG) & 1];
    const int sl = t % MXG;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int ra = wm * TM + 32 * i + r;
        F.a[ks][i] = *reinterpret_cast<const u32x4*>(&S.a[ra * MXROWB + swz_mx(ra, 4 * x + 2 * ks + h) * 16]);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int rb = wn * TN + 32 * j + r;
        F.b[ks][j] = *reinterpret_cast<const u32x4*>(&S.b[rb * MXROWB + swz_mx(rb, 4 * x + 2 * ks + h) * 16]);
      }
    }
    const int wb = 8 * (sl & 1) + 4 * x;             // byte of the word within its 16-byte half
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int ra = wm * TM + 32 * i + r;
      F.sa[i] = *reinterpret_cast<const uint32_t*>(&SG.a[ra * MXSGB + swz_mxs(ra, sl >> 1) * 16 + wb]);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int rb = wn * TN + 32 * j + r;
      F.sb[j] = *reinterpret_cast<const uint32_t*>(&SG.b[rb * MXSGB + swz_mxs(rb, sl >> 1) * 16 + wb]);
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // MFMAs [lo, hi) of a half-stage, in the order (k-step, i, j).  The lane's
  // scale bytes 2 ks + h are moved to bytes 2 ks, so op_sel is 2 ks.
  auto compute = [&](const Frags<TI, TJ>& F, auto LO, auto HI) {
    constexpr int lo = decltype(LO)::value, hi = decltype(HI)::value;
#pragma unroll
    for (int q = lo; q < hi; ++q) {
      const int ks = q / (TI * TJ), i = q / TJ % TI, j = q % TJ;
      const int sa = (int)(F.sa[i] >> (8 * h)), sb = (int)(F.sb[j] >> (8 * h));
      const v8i a8 = {(int)F.a[ks][i][0], (int)F.a[ks][i][1], (int)F.a[ks][i][2], (int)F.a[ks][i][3], 0, 0, 0, 0};
      const v8i b8 = {(int)F.b[ks][j][0], (int)F.b[ks][j][1], (int)F.b[ks][j][2], (int)F.b[ks][j][3], 0, 0, 0, 0};
      if (ks == 0)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 0, sb, 0, sa);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 2, sb, 2, sa);
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using CE = std::integral_constant<int, 8>;                 // MFMAs ahead of a barrier
  using CN = std::integral_constant<int, 2 * TI * TJ>;       // MFMAs per half-stage

  // ---- software pipeline ----------------------------------------------------
  // Half-step u multiplies half-stage u from registers while the fragments
  // of half-stage u + 1 are read.  Each half-step starts with a few MFMAs so
  // that the matrix core stays busy across its wait and barrier.
  //   even u = 2 t: read the fragments of (t, 1), the last of stage t; once
  //     every wave has them (barrier), load stage t + 2 into slot t % 2, and
  //     with t % 4 == 3 the scale group of stages t + 5 .. t + 8 into the
  //     slot of the group just read.
  //   odd u = 2 t + 1: wait for stage t + 1 (own loads by count: issued after
  //     it are stage t + 2 and maybe a group; everyone's at the barrier), then
  //     read the fragments of (t + 1, 0).
  // A stage is loaded about three half-steps before it is first read: the
  // single stage in flight needs that long to land.
  // Issue order: group 0, stages 0, 1, group 1, then per even half-step the
  // stage and (every fourth) the group.
  issue_group(0);
  issue_stage(0);
  issue_stage(1);
  issue_group(1);
  wait_vm<2 * NL + NSG>();                   // stage 0 and group 0
  __asm__ volatile("s_barrier" ::: "memory");
  Frags<TI, TJ> F0, F1;
  read_frags(0, F0);

  auto step = [&](auto J, int u, const Frags<TI, TJ>& Fc, Frags<TI, TJ>& Fn) {
    constexpr int j = decltype(J)::value;      // u % 8
    const int t = u >> 1;
    if constexpr ((j & 1) == 0) {
      read_frags(u + 1, Fn);
      compute(Fc, C0{}, CE{});
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * TI + 2 * TJ + TI + TJ, 0);   // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, CE::value, 0);                   // MFMA
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkm0();
      __asm__ volatile("s_barrier" ::: "memory");
      issue_stage(t + 2);
      if constexpr (j == 6) issue_group((t + 2) / MXG + 1);
      compute(Fc, CE{}, CN{});
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);                        // global loads
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);                        // MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
      compute(Fc, C0{}, CE{});
      __builtin_amdgcn_sched_barrier(0);
      // stage t + 1; issued after it: stage t + 2 and, at j == 7, a group
      if constexpr (j == 7) wait_vm<2 * NL + NSG>();
      else wait_vm<2 * NL>();
      __asm__ volatile("s_barrier" ::: "memory");
      read_frags(u + 1, Fn);                   // past the end: a repeated stage, unused
      compute(Fc, CE{}, CN{});
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                        // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);                        // MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int nfull = nst / MXG * MXG;
  for (int t = 0; t < nfull; t += MXG) {
    const int u = 2 * t;
    step(std::integral_constant<int, 0>{}, u, F0, F1);
    step(std::integral_constant<int, 1>{}, u + 1, F1, F0);
    step(std::integral_constant<int, 2>{}, u + 2, F0, F1);
    step(std::integral_constant<int, 3>{}, u + 3, F1, F0);
    step(std::integral_constant<int, 4>{}, u + 4, F0, F1);
    step(std::integral_constant<int, 5>{}, u + 5, F1, F0);
    step(std::integral_constant<int, 6>{}, u + 6, F0, F1);
    step(std::integral_constant<int, 7>{}, u + 7, F1, F0);
  }
  if (nfull < nst) {                           // two stages left (k = 512 mod 1024)
    const int u = 2 * nfull;
    step(std::integral_constant<int, 0>{}, u, F0, F1);
    step(std::integral_constant<int, 1>{}, u + 1, F1, F0);
    step(std::integral_constant<int, 2>{}, u + 2, F0, F1);
    step(std::integral_constant<int, 3>{}, u + 3, F1, F0);
  }

  wait_vm<0>();                 // no load may land in LDS after the workgroup ends
  store_tile<WMW, WNW>(acc, reinterpret_cast<uint8_t*>(&smem), 1.0f, c, c_dtype, m, n, m0, n0, m_lo, n_lo);
}

}  // namespace

bool gemm_large_supported(int fmt, int64_t m, int64_t n, int64_t k) {
  const int64_t lim = int64_t(1) << 31;     // 32-bit buffer offsets
  // 16-byte scale rows: k a multiple of 512 (MXFP4) or 256 (NVFP4)
  const int64_t kq = (fmt == kFmtNV) ? 256 : 512;
  // MXFP4 tiles are moved back to lie inside the operands: m, n >= 256
  const int64_t mn = (fmt == kFmtNV) ? 128 : 256;
  return m >= mn && n >= mn && k % kq == 0 && m * (k / 2) < lim && n * (k / 2) < lim;
}

hipError_t launch_gemm_large(int fmt, int64_t m, int64_t n, int64_t k,
                             const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tscale, const uint8_t* b_codes,
                             const uint8_t* b_scales, const float* b_tscale,
                             void* c, int c_dtype, hipStream_t stream) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  if (fmt == kFmtMX) {
    hipLaunchKernelGGL((gemm_large_mx<kMXWM, kMXWN>), grid, dim3(64 * kMXWM * kMXWN), 0, stream,
                       (int)m, (int)n, (int)k, a_codes, a_scales, b_codes, b_scales, c, c_dtype,
                       tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL((gemm_large<kFmtNV, kNVWM, kNVWN>), grid, dim3(64 * kNVWM * kNVWN), 0, stream,
                       (int)m, (int)n, (int)k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                       b_tscale, c, c_dtype, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

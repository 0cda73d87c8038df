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
  // The MFMAs take B as the first operand, so in each 32x32 block a lane holds
  // output row r = lane % 32 and, in registers 4g .. 4g + 3, the four
  // consecutive columns 8g + 4h .. + 3.  The tile goes through LDS (the ring
  // is free now) in row-major order and leaves as 16-byte row chunks: direct
  // stores of the fragments would scatter 2- or 4-byte pieces over 32 rows.
  wait_lgkm0();
  __asm__ volatile("s_barrier" ::: "memory");
  const float ts = (FMT == kFmtNV) ? (*at) * (*bt) : 1.0f;
  uint8_t* ep = reinterpret_cast<uint8_t*>(&smem);
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
      if (grow >= m || gcol >= n) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(ep + lr * pitch + ch * 16);
      const int64_t off = (int64_t)grow * n + gcol;
      if (vec_ok && gcol + epc <= n) {
        if (f32) *reinterpret_cast<uint4*>(reinterpret_cast<float*>(c) + off) = v;
        else *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(c) + off) = v;
      } else if (f32) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gcol + e < n) reinterpret_cast<uint32_t*>(c)[off + e] = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
          if (gcol + e < n) reinterpret_cast<uint16_t*>(c)[off + e] = (uint16_t)(w >> (16 * (e & 1)));
        }
      }
    }
    if (band + 1 < nband) __syncthreads();
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

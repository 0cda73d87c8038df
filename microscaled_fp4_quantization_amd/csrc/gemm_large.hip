// W4A4 GEMM for many activation rows (prefill / large m) on gfx950.
//
// C[m, n] = sum_k deq(A)[m, k] deq(B)[n, k], A = activations [m, k], B =
// weights [n, k], both quantized along k (pimento.cloud "FP8, NVFP4 czy
// AWQ?", section "Dlaczego W8A8 i W4A16 to nie to samo?": W4A4 runs the
// products on low-precision matrix units).
//
// Two kernels, each one workgroup of 4 waves (one per SIMD) per CU and a
// 256-row tile of C; k advances in stages staged through LDS by direct
// global->LDS buffer loads, so loads in flight spend no registers.  A direct
// load writes lane i's 16 bytes at base + 16 i, so the LDS layout is chosen
// through the global addresses (16-byte chunks permuted within a row so that
// fragment reads spread over the LDS banks).
//
// NVFP4 (gemm_nv4w): stages of 128 k-values (64 code bytes per row) in a
// 4-deep ring; scales in groups of 16 bytes per row (2 stages) in a 3-slot
// ring of their own (fetching a stage's 8 scale bytes per row on its own
// would cost one memory request per row for a few bytes, and the request
// rate, not the byte rate, bounds the operand stream).  The fragments are
// decoded to fp16 and multiplied by their block scale in fp16 (exact: at
// most 6 significant bits, range [2^-10, 2688]); v_mfma_f32_16x16x32_f16
// accumulates in fp32; the two FP32 tensor scales are applied in the
// epilogue.  Tile 256 x 224 or 256 x 256.
//
// MXFP4 (gemm_large_mx, E8M0 scale per 32 values):
// v_mfma_scale_f32_32x32x64_f8f6f4, both operands E2M1, stages of 256
// k-values.  Tile 256 x 256.
//
// Workgroup -> tile mapping is XCD-aware: consecutive workgroup ids land on
// different XCDs (each with its own L2), so the ids are regrouped to give
// every XCD a contiguous run of tiles, ordered m-fastest, so that the tiles
// sharing a weight slab run on the same L2.
#include <type_traits>

#include <utility>

#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int ROWB = BK / 2;          // code bytes per row per stage
constexpr int NSTAGE = 4;             // LDS ring depth
constexpr int NXCD = 8;
// waves per workgroup along m and n
constexpr int kMXWM = 2, kMXWN = 2;
// Elements between two split-k slices of fp32 partial sums in the GEMM
// workspace: m n rounded up to a multiple of 4 (16-byte aligned slices).
__host__ __device__ __forceinline__ int64_t split_stride(int64_t m, int64_t n) { return (m * n + 3) / 4 * 4; }

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

// Writes a workgroup's 256 x BNT tile of C = ts * acc.  The MFMAs take B as
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
template <int WMW, int WNW, int TI, int TJ, int BNT = BN>
__device__ __forceinline__ void store_tile(const v16f (&acc)[TI][TJ], uint8_t* ep, float ts,
                                           void* __restrict__ c, int c_dtype, int m, int n,
                                           int m0, int n0, int m_lo, int n_lo) {
  constexpr int NW = WMW * WNW, TM = BM / WMW, TN = BNT / WNW;
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
    // 16-byte chunks: BNT / 8 (bf16) or BNT / 4 (f32) per row
    const int cpr = f32 ? BNT / 4 : BNT / 8, epc = f32 ? 4 : 8;
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

// ---- NVFP4 helpers ---------------------------------------------------------
// 16-byte chunk c of a 64-byte code row r is stored at position
// c ^ ((r >> 2) & 3): the LDS has 64 banks of 4 bytes (16 groups of 16
// bytes), a 64-byte row spans 4 groups, and the 16 rows a 16-lane phase of a
// 16-byte fragment read touches then fall on 16 different groups.
__device__ __forceinline__ int swz16(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

template <int WMW, int WNW, int TI, int TJ, int BNT = BN>
__device__ __forceinline__ void store_tile16(const v4f (&acc)[TI][TJ], uint8_t* ep, float ts,
                                             void* __restrict__ c, int c_dtype, int m, int n,
                                             int m0, int n0) {
  // lane (r, g) of block (i, j) holds C row 16 i + r, columns 16 j + 4 g .. + 3
  constexpr int NW = WMW * WNW, TM = BM / WMW, TN = BNT / WNW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int r = lane & 15, g = lane >> 4;
  wait_lgkm0();
  __asm__ volatile("s_barrier" ::: "memory");
  const bool f32 = (c_dtype == kInF32);
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
          const int row = (f32 ? 0 : wm * TM) + 16 * i + r;
          const int col = wn * TN + 16 * j + 4 * g;
          const float v0 = acc[i][j][0] * ts, v1 = acc[i][j][1] * ts;
          const float v2 = acc[i][j][2] * ts, v3 = acc[i][j][3] * ts;
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
    __syncthreads();
    const int cpr = f32 ? BNT / 4 : BNT / 8, epc = f32 ? 4 : 8;
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

// Where the NVFP4 kernel's conversions go in a k-step.  Row i of the TI x TJ
// MFMAs (q = TJ i .. TJ i + TJ - 1) is followed, spread evenly after its
// MFMAs, by its pieces: kind 0 = A row idx of this k-step (row i + 1: its
// register is free once row i - 1 is issued and must be ready for row
// i + 1), 1 = B fragment idx of the next k-step, 2 = A row 0 of the next
// k-step (last row), 3 / 4 = the next stage's B / A scale pair idx (last
// k-step of a stage).  u = piece (values 2u, 2u + 1) of a conversion.  In a
// stage's last k-step the next stage's words are read first, so its B
// conversions start at row 3, after its scale pairs (rows 1 and 2).
struct ConvPiece {
  int kind, idx, u;
};
template <int TI, int TJ>
struct ConvRows {
  ConvPiece p[TI][32];
  int n[TI];
};
template <int TI, int TJ>
constexpr ConvRows<TI, TJ> conv_rows(bool last) {
  ConvRows<TI, TJ> r{};
  for (int i = 0; i < TI; ++i) r.n[i] = 0;
  for (int i = 0; i + 1 < TI; ++i)
    for (int u = 0; u < 4; ++u) r.p[i][r.n[i]++] = ConvPiece{0, i + 1, u};
  if (last) {
    for (int j = 0; j < TJ; ++j) r.p[1][r.n[1]++] = ConvPiece{3, j, 0};
    for (int i = 0; i < TI; ++i) r.p[2][r.n[2]++] = ConvPiece{4, i, 0};
  }
  const int b0 = last ? 3 : 0, nb = TI - b0;
  for (int k = 0; k < 4 * TJ; ++k) {
    const int row = b0 + k * nb / (4 * TJ);
    r.p[row][r.n[row]++] = ConvPiece{1, k / 4, k % 4};
  }
  for (int u = 0; u < 4; ++u) r.p[TI - 1][r.n[TI - 1]++] = ConvPiece{2, 0, u};
  return r;
}
// f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N - 1>{}),
// expanded at compile time whatever the loop unroller decides.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int TI, int TJ>
constexpr bool conv_rows_ok() {
  for (int l = 0; l < 2; ++l) {
    const ConvRows<TI, TJ> r = conv_rows<TI, TJ>(l == 1);
    for (int i = 0; i < TI; ++i) {
      if (r.n[i] > 32 || r.n[i] < 1) return false;
      // an A row's pieces come before the row's other pieces, so they land
      // among its MFMAs; the rest is checked by construction
      for (int k = 0; k < r.n[i]; ++k)
        if (r.p[i][k].kind == 0 && r.p[i][k].idx != i + 1) return false;
    }
  }
  return true;
}

// ---- NVFP4: 16x16x32 f16 MFMAs, one wave per SIMD --------------------------
// Measured alternatives on 2048 x 28672 x 8192: eight waves of 128 x 64 run
// the multiply-and-convert work alone at 1.9 PFLOP/s but read the fragments
// from LDS 1.5x as often per MFMA as four waves of 128 x 128 (each wave reads
// its own rows), and with two waves per SIMD there are no registers left to
// read the next stage's fragments ahead: 0.86-0.92 ms.  Four waves, one per
// SIMD, keep 224 or 256 accumulators per lane in AGPRs and read stage s + 1's
// fragments into registers while stage s is multiplied.
//
// The tile is 256 x BNT with BNT = 256 or 224 (wave tile 128 x BNT / 2 =
// 8 x BNT / 32 blocks of 16 x 16): 224 divides the 14336- and 28672-wide
// weights into 1024 tiles for m = 4096 and 2048, i.e. exactly four rounds of
// the 256 CUs, where 256-wide tiles give 896 and leave half the CUs idle for
// the last round.  B rows are staged 256 at a time regardless (the extra
// rows are clamped re-reads, never multiplied).
//
// Fragment layout and k-slots as gemm_nv16: lane group g = lane / 16 reads
// the 16-byte chunk g of its row (k in [32 g, 32 g + 32) of the stage) and in
// k-step s uses its dword s (NVFP4 block 2 g + s / 2).
template <int TI, int TJ>
struct Frags16 {
  u32x4 a[TI];
  u32x4 b[TJ];
  uint32_t sa[TI];     // the two scale bytes of chunk g (low half)
  uint32_t sb[TJ];
};

template <int BNT>
__global__ __launch_bounds__(256, 1) void gemm_nv4w(
    int m, int n, int k, const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
    const float* __restrict__ at, const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs,
    const float* __restrict__ bt, void* __restrict__ c, int c_dtype, int tiles_m, int tiles_n,
    int ksplit, float* __restrict__ part) {
  using Stage = LargeStage;
  constexpr int WMW = 2, WNW = 2, NW = 4;
  constexpr int G = 2;                         // NVFP4 stages per 16-byte scale group
  constexpr int NL = BM * ROWB / 1024 / NW;    // 1 KiB code blocks per operand per wave (4)
  constexpr int NSG = 8 / NW;                  // 1 KiB scale-group blocks per wave (2)
  constexpr int TM = BM / WMW, TN = BNT / WNW;
  constexpr int TI = TM / 16, TJ = TN / 16;
  static_assert(BNT % 32 == 0 && BNT <= BN && 6 * NL + 2 * NSG < 64, "tile shape");
  __shared__ __attribute__((aligned(16))) LargeSmem smem;
  Stage* st = smem.st;
  ScaleGroup* sgr = smem.sg;

  const int ntiles = tiles_m * tiles_n;
  const int wg = blockIdx.x;
  int tile = wg;
  if (ntiles % NXCD == 0) tile = (wg % NXCD) * (ntiles / NXCD) + wg / NXCD;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BNT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kbytes = k / 2, srow = k / 16;
  // split k: workgroup row blockIdx.y takes values [ksplit y, ksplit (y + 1))
  const int kofs = (int)blockIdx.y * ksplit;
  const int nstages = ksplit / BK;
  const int ngroups = nstages / G;

  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)a, (short)0, m * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)b, (short)0, n * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_as = __builtin_amdgcn_make_buffer_rsrc((void*)as, (short)0, m * srow, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_bs = __builtin_amdgcn_make_buffer_rsrc((void*)bs, (short)0, n * srow, 0x00020000);
  // Code block q = i NW + wave (16 rows x 64 bytes): lane p fills position
  // p, i.e. row 16 q + p / 4 at stored chunk p % 4, holding logical chunk
  // (p % 4) ^ ((row >> 2) & 3), which does not depend on i.  The lane's
  // offset is that of block i = 0; the 64 i rows further on, the tile's first
  // row and the stage go into the uniform offset.  Rows past m or n read
  // past the buffer's end (the buffer load returns zeros) or into the next
  // rows: they only reach outputs that are not stored.
  const int crow = 16 * wave + (lane >> 2);
  const int voff_c = crow * kbytes + swz16(crow, lane & 3) * 16;
  // scale-group block j of this wave: g = j NW + wave selects the operand
  // (g / 4) and rows 64 (g % 4) .. + 63; lane p loads row 64 (g % 4) + p
  const int voff_s = lane * srow;
  auto issue_stage = [&](int t) {
    Stage& S = st[t % NSTAGE];
    const int kb = (t < nstages ? t : nstages - 1) * ROWB + kofs / 2;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = i * NW + wave;
      load_lds16(rs_a, &S.a[q * 1024], voff_c, (m0 + 64 * i) * kbytes + kb);
      load_lds16(rs_b, &S.b[q * 1024], voff_c, (n0 + 64 * i) * kbytes + kb);
    }
  };
  // load q of issue_stage(t) (A block q / 2 for even q, B for odd) and
  // load j of issue_group(g)
  auto issue_load = [&](int t, int q) {
    Stage& S = st[t % NSTAGE];
    const int kb = (t < nstages ? t : nstages - 1) * ROWB + kofs / 2;
    const int i = q >> 1, blk = i * NW + wave;
    if ((q & 1) == 0) load_lds16(rs_a, &S.a[blk * 1024], voff_c, (m0 + 64 * i) * kbytes + kb);
    else load_lds16(rs_b, &S.b[blk * 1024], voff_c, (n0 + 64 * i) * kbytes + kb);
  };
  auto issue_group_load = [&](int g, int j) {
    ScaleGroup& SG = sgr[g % NSGRP];
    const int gb = 16 * (g < ngroups ? g : ngroups - 1) + kofs / 16;
    const int gw = j * NW + wave;
    const bool isb = gw >= 4;
    load_lds16(isb ? rs_bs : rs_as, &SG.w[isb][256 * (gw % 4)], voff_s,
               ((isb ? n0 : m0) + 64 * (gw % 4)) * srow + gb);
  };
  auto issue_group = [&](int g) {
    ScaleGroup& SG = sgr[g % NSGRP];
    const int gb = 16 * (g < ngroups ? g : ngroups - 1) + kofs / 16;
#pragma unroll
    for (int j = 0; j < NSG; ++j) {
      const int gw = j * NW + wave;
      const bool isb = gw >= 4;
      load_lds16(isb ? rs_bs : rs_as, &SG.w[isb][256 * (gw % 4)], voff_s,
                 ((isb ? n0 : m0) + 64 * (gw % 4)) * srow + gb);
    }
  };

  const int wm = wave / WNW, wn = wave % WNW;
  const int r = lane & 15, g4 = lane >> 4;
  // per-lane byte offsets in the shared object of the first A / B fragment
  // row and of their scale words; fragment i / j lies 1 KiB (codes) or 256
  // bytes (scales) further on
  const uint8_t* sm = reinterpret_cast<const uint8_t*>(&smem);
  const int ra0 = wm * TM + r, rb0 = wn * TN + r;
  const int a_lane = (int)offsetof(Stage, a) + ra0 * ROWB + swz16(ra0, g4) * 16;
  const int b_lane = (int)offsetof(Stage, b) + rb0 * ROWB + swz16(rb0, g4) * 16;
  const int sa_lane = (int)offsetof(LargeSmem, sg) + (int)offsetof(ScaleGroup, w) + 16 * ra0 + 4 * (g4 >> 1);
  const int sb_lane = (int)offsetof(LargeSmem, sg) + (int)offsetof(ScaleGroup, w) + BM * 16 + 16 * rb0 + 4 * (g4 >> 1);
  auto read_frags = [&](int t, Frags16<TI, TJ>& F) {
    int ao = (t % NSTAGE) * (int)sizeof(Stage) + a_lane;
    int bo = (t % NSTAGE) * (int)sizeof(Stage) + b_lane;
    const int sgo = ((t / G) % NSGRP) * (int)sizeof(ScaleGroup) + (t % G) * 8;
    int sao = sgo + sa_lane, sbo = sgo + sb_lane;
    __asm__ volatile("" : "+v"(ao), "+v"(bo), "+v"(sao), "+v"(sbo));
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      F.a[i] = *reinterpret_cast<const u32x4*>(sm + ao + 1024 * i);
      F.sa[i] = *reinterpret_cast<const uint32_t*>(sm + sao + 256 * i);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      F.b[j] = *reinterpret_cast<const u32x4*>(sm + bo + 1024 * j);
      F.sb[j] = *reinterpret_cast<const uint32_t*>(sm + sbo + 256 * j);
    }
  };

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int sh = 16 * (g4 & 1);

  // ---- the conversions, spread between the MFMAs ---------------------------
  // A k-step issues its TI x TJ MFMAs (q = 0 .. NQ - 1: row q / TJ, column
  // q % TJ) from converted operands: hb[s & 1][j] for the B fragments and
  // ha[i & 1] for A row i.  The conversions the later MFMAs need run between
  // them, about two VALU instructions after each MFMA: the next row's A
  // fragment during each row, the next k-step's B fragments and first A
  // fragment during the whole k-step.  A wave keeps the matrix core busy
  // with that many independent VALU instructions between MFMAs, while
  // converted in clusters the conversions and the MFMAs ran one after the
  // other.  A scheduling fence after every MFMA keeps this order (the rows'
  // pieces: conv_rows).  In k-step 3 the next stage's fragment words are
  // read from LDS as their registers free up (its B and scale words first,
  // A row i once row i's last word is converted), and its scale pairs are
  // converted.

  // piece t (values 2t, 2t + 1) of the conversion of word w under half hi of
  // the scale pair sp, into the v8h x
  auto conv_piece = [&](v8h& x, uint32_t w, v2h sp, int hi, int t) {
    const _Float16 sv = hi ? sp.y : sp.x;
    const v2h s2 = {sv, sv};
    v2h pc;
    switch (t) {
      case 0: pc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2; break;
      case 1: pc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2; break;
      case 2: pc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2; break;
      default: pc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2; break;
    }
    x[2 * t] = pc.x;
    x[2 * t + 1] = pc.y;
  };
  auto scale_pair = [&](uint32_t word) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word >> sh, 1.0f, false); };

  static_assert(conv_rows_ok<TI, TJ>(), "conversion plan");
  constexpr int NQ = TI * TJ;
  v8h hb[2][TJ], ha[2];
  v2h sap[TI], sbp[TJ], sapn[TI], sbpn[TJ];

  // Software pipeline: iteration s waits for stage s + 1 (this wave's loads
  // by count, everyone's at the barrier, which also ends every wave's LDS
  // reads of stage s), then multiplies stage s from registers in four
  // k-steps.  Between the first MFMAs of k-step 0 it loads stage s + 4 into
  // the slot stage s vacated and, at the end of a scale group, group
  // (s + 1) / 2 + 2 into the slot of the group just finished; in k-step 3
  // each fragment's registers take its stage s + 1 words once its last word
  // is converted (one set of fragment registers instead of two, with fewer
  // AGPR <-> VGPR moves).  Issued after stage s + 1 in the steady state:
  // stages s + 2, s + 3 and the groups of iterations s - 3 .. s - 1.
  issue_group(0);                              // -5
  issue_stage(0);                              // -4
  issue_stage(1);                              // -3
  issue_group(1);                              // -3
  issue_stage(2);                              // -2
  issue_stage(3);                              // -1
  issue_group(2);                              // -1
  wait_vm<6 * NL + 2 * NSG>();                 // stage 0, group 0
  __asm__ volatile("s_barrier" ::: "memory");
  Frags16<TI, TJ> F;
  read_frags(0, F);
  // the first k-step's operands
#pragma unroll
  for (int i = 0; i < TI; ++i) sap[i] = scale_pair(F.sa[i]);
#pragma unroll
  for (int j = 0; j < TJ; ++j) sbp[j] = scale_pair(F.sb[j]);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) conv_piece(hb[0][j], F.b[j][0], sbp[j], 0, t);
    conv_piece(ha[0], F.a[0][0], sap[0], 0, t);
  }

  // k-step S of stage s (the fragments in F); in k-step 3 the words of stage
  // s + 1 replace them
  auto kstep = [&](auto SS, int s) {
    constexpr int S = decltype(SS)::value;
    constexpr bool LAST = S == 3;
    constexpr int HI = S < 2 ? 0 : 1;                      // scale half of this k-step
    constexpr int HN = LAST ? 0 : (S + 1 < 2 ? 0 : 1);     // of the next one
    const int tn = s + 1;
    int ao = (tn % NSTAGE) * (int)sizeof(Stage) + a_lane;
    int bo = (tn % NSTAGE) * (int)sizeof(Stage) + b_lane;
    const int sgo = ((tn / G) % NSGRP) * (int)sizeof(ScaleGroup) + (tn % G) * 8;
    int sao = sgo + sa_lane, sbo = sgo + sb_lane;
    if constexpr (LAST) {
      __asm__ volatile("" : "+v"(ao), "+v"(bo), "+v"(sao), "+v"(sbo));
      // stage s + 1's B words, scale words and A row 0 (row 0's last word of
      // this stage was converted in k-step 2)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        F.b[j] = *reinterpret_cast<const u32x4*>(sm + bo + 1024 * j);
        F.sb[j] = *reinterpret_cast<const uint32_t*>(sm + sbo + 256 * j);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) F.sa[i] = *reinterpret_cast<const uint32_t*>(sm + sao + 256 * i);
      F.a[0] = *reinterpret_cast<const u32x4*>(sm + ao);
    }
    constexpr ConvRows<TI, TJ> R = conv_rows<TI, TJ>(LAST);
    // MFMA q and the conversion pieces placed after it; q is a constant once
    // the slots are expanded: by the loop unroller for 8 x 7 blocks, by
    // static_for for 8 x 8 (the unroller leaves those rolled, and the
    // fragment registers then spill)
    auto slot = [&](int q) {
      const int i = q / TJ, j = q % TJ;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hb[S & 1][j], ha[i & 1], acc[i][j], 0, 0, 0);
      if constexpr (S == 0) {
        // this stage's loads: stage s + 4, then after odd stages a scale group
        if (q < 2 * NL) issue_load(s + NSTAGE, q);
        if (q >= 2 * NL && q < 2 * NL + NSG && (s & 1) == 1) issue_group_load((s + 1) / G + 2, q - 2 * NL);
      }
#pragma unroll
      for (int k = 0; k < R.n[i]; ++k) {
        if (TJ * i + k * TJ / R.n[i] != q) continue;
        const int kind = R.p[i][k].kind, idx = R.p[i][k].idx, u = R.p[i][k].u;
        if (kind == 0) {
          conv_piece(ha[idx & 1], F.a[idx][S], sap[idx], HI, u);
          if (LAST && u == 3) F.a[idx] = *reinterpret_cast<const u32x4*>(sm + ao + 1024 * idx);
        } else if (kind == 1) {
          if (LAST) conv_piece(hb[(S + 1) & 1][idx], F.b[idx][0], sbpn[idx], HN, u);
          else conv_piece(hb[(S + 1) & 1][idx], F.b[idx][(S + 1) & 3], sbp[idx], HN, u);
        } else if (kind == 2) {
          if (LAST) conv_piece(ha[0], F.a[0][0], sapn[0], HN, u);
          else conv_piece(ha[0], F.a[0][(S + 1) & 3], sap[0], HN, u);
        } else if (kind == 3) {
          sbpn[idx] = scale_pair(F.sb[idx]);
        } else {
          sapn[idx] = scale_pair(F.sa[idx]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (TJ == 7) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) slot(q);
    } else {
      static_for<NQ>([&](auto Q) { slot(decltype(Q)::value); });
    }
    if constexpr (LAST) {
#pragma unroll
      for (int i = 0; i < TI; ++i) sap[i] = sapn[i];
#pragma unroll
      for (int j = 0; j < TJ; ++j) sbp[j] = sbpn[j];
    }
  };

  for (int s = 0; s < nstages; ++s) {
    // stage s + 1 (this wave's loads by count, everyone's at the barrier,
    // which also ends every wave's LDS reads of stage s - 1's slot)
    if ((s & 1) == 0) wait_vm<4 * NL + 2 * NSG>();
    else wait_vm<4 * NL + NSG>();
    wait_lgkm0();
    __asm__ volatile("s_barrier" ::: "memory");
    kstep(std::integral_constant<int, 0>{}, s);
    kstep(std::integral_constant<int, 1>{}, s);
    kstep(std::integral_constant<int, 2>{}, s);
    kstep(std::integral_constant<int, 3>{}, s);    // at s = nstages - 1: the repeated last stage, unused
  }
  static_assert(G == 2, "scale-group parity");

  wait_vm<0>();                 // no load may land in LDS after the workgroup ends
  // split k: this slice's unscaled fp32 sums into the workspace
  void* dst = part ? static_cast<void*>(part + (int64_t)blockIdx.y * split_stride(m, n)) : c;
  const float ts = part ? 1.0f : (*at) * (*bt);
  store_tile16<WMW, WNW, TI, TJ, BNT>(acc, reinterpret_cast<uint8_t*>(&smem), ts, dst,
                                      part ? kInF32 : c_dtype, m, n, m0, n0);
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

// One 256 x BNT tile (BNT = 256, or 128 for the half-width tiles that finish
// a grid whose last round of full tiles would leave CUs idle): tile `tile`
// of the tiles_m-row grid of such tiles over the columns n_begin .. n - 1.
template <int WMW, int WNW, int BNT>
__device__ __forceinline__ void mx_tile(
    MxSmem& smem, int tile, int m, int n, int k, const uint8_t* __restrict__ a,
    const uint8_t* __restrict__ as, const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs,
    void* __restrict__ c, int c_dtype, int tiles_m, int n_begin, int ksplit, float* __restrict__ part) {
  constexpr int NW = WMW * WNW;
  constexpr int NL = BM * MXROWB / 1024 / NW;        // A code loads per wave per stage
  constexpr int NLB = BNT * MXROWB / 1024 / NW;      // B code loads per wave per stage
  // scale loads per wave per group: two of A's 128-row halves, one or two of B's
  constexpr int NSG = 2 + BNT / 128;
  constexpr int NLD = NL + NLB;                      // code loads per wave per stage
  constexpr int TM = BM / WMW, TN = BNT / WNW;
  constexpr int TI = TM / 32, TJ = TN / 32;
  static_assert(BNT <= BN && BNT % 128 == 0 && NL * NW * 1024 == BM * MXROWB && NLB * NW * 1024 == BNT * MXROWB &&
                2 * BM * MXSGB == 4 * NW * 1024, "tile shape");
  static_assert(NLD + NSG < 64, "vmcnt range");

  const int tm = tile % tiles_m, tn = tile / tiles_m;
  // A last tile that would run past m or n is moved back to end at the last
  // row or column (n - n_begin >= BNT): every row it loads exists, and the
  // rows and columns it shares with its neighbour are left to the neighbour.
  // With m < 256 the one row of tiles stays at row 0: its rows past m load
  // nothing from the buffer (out of range) and are not stored.
  const int m_lo = tm * BM, n_lo = n_begin + tn * BNT;
  const int m0 = (m_lo + BM <= m || m < BM) ? m_lo : m - BM;
  const int n0 = n_lo + BNT <= n ? n_lo : n - BNT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kbytes = k / 2, srow = k / 32;
  // split k: workgroup row blockIdx.y takes values [ksplit y, ksplit (y + 1))
  const int kofs = (int)blockIdx.y * ksplit;
  const int nst = ksplit / MXBK;                     // even: ksplit is a multiple of 512
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
  static_assert(NW == 4, "scale-load mapping");
  const int srw = 32 * wave + (lane >> 1);
  const int voff_s = srw * srow;
  const int hoff_s = 16 * swz_mxs(srw, lane & 1);
  // stage t (clamped to the last; a repeat is never read) into slot t % 2
  auto issue_stage = [&](int t) {
    MxStage& S = smem.st[t & 1];
    const int kb = (t < nst ? t : nst - 1) * MXROWB + kofs / 2;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = i * NW + wave;
      load_lds16(rs_a, &S.a[q * 1024], voff_c, (m0 + 32 * i) * kbytes + kb);
      if (i < NLB) load_lds16(rs_b, &S.b[q * 1024], voff_c, (n0 + 32 * i) * kbytes + kb);
    }
  };
  // scale group g (clamped to the last) into group slot g % 2.  A last group
  // of two stages has only its first half inside the row: the second half
  // then repeats the first and is never read.  Load j < 2 covers A's rows
  // 128 j .. + 127, load j >= 2 B's rows 128 (j - 2) .. + 127.
  auto issue_group = [&](int g) {
    MxScaleGroup& SG = smem.sg[g & 1];
    const int gc = g < ngr ? g : ngr - 1;
    const int gb = MXSGB * gc;
    const bool whole = gb + MXSGB <= ksplit / 32;
    const int vo = voff_s + (whole ? hoff_s : 0);
#pragma unroll
    for (int j = 0; j < NSG; ++j) {
      const int gw = j * NW + wave;
      const bool isb = j >= 2;
      load_lds16(isb ? rs_bs : rs_as, (isb ? SG.b : SG.a) + 1024 * (gw % 8), vo,
                 ((isb ? n0 : m0) + 128 * (j & 1)) * srow + gb + kofs / 32);
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
  using CE = std::integral_constant<int, BNT == BN ? 8 : 4>; // MFMAs ahead of a barrier
  using CN = std::integral_constant<int, 2 * TI * TJ>;       // MFMAs per half-stage
  // the MFMAs after the barrier, in NIG groups of MPG between groups of
  // direct loads (even half-steps) or fragment reads (odd half-steps)
  constexpr int NIG = BNT == BN ? 8 : 6;
  constexpr int MPG = (CN::value - CE::value) / NIG;
  static_assert(MPG * NIG == CN::value - CE::value, "interleave");

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
  wait_vm<NLD + NSG>();                      // stage 0 and group 0
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
      for (int g = 0; g < NIG; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);                        // global loads
        __builtin_amdgcn_sched_group_barrier(0x008, MPG, 0);                      // MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
      compute(Fc, C0{}, CE{});
      __builtin_amdgcn_sched_barrier(0);
      // stage t + 1; issued after it: stage t + 2 and, at j == 7, a group
      if constexpr (j == 7) wait_vm<NLD + NSG>();
      else wait_vm<NLD>();
      __asm__ volatile("s_barrier" ::: "memory");
      read_frags(u + 1, Fn);                   // past the end: a repeated stage, unused
      compute(Fc, CE{}, CN{});
#pragma unroll
      for (int g = 0; g < NIG; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                        // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, MPG, 0);                      // MFMA
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
  // split k: this slice's fp32 sums into the workspace
  void* dst = part ? static_cast<void*>(part + (int64_t)blockIdx.y * split_stride(m, n)) : c;
  store_tile<WMW, WNW, TI, TJ, BNT>(acc, reinterpret_cast<uint8_t*>(&smem), 1.0f, dst,
                                    part ? kInF32 : c_dtype, m, n, m0, n0, m_lo, n_lo);
}

// Tile order within a class of cnt tiles: each XCD (workgroup w runs on XCD
// w % 8) takes a contiguous run of tiles, m fastest, so that the tiles in
// flight on an XCD share weight rows in its L2.
__device__ __forceinline__ int xcd_tile(int local, int cnt) {
  return cnt % NXCD == 0 ? (local % NXCD) * (cnt / NXCD) + local / NXCD : local;
}

// Workgroups [0, full) take the 256 x 256 tiles of columns 0 .. n_half - 1
// (n_half = n when there are no half-width tiles), the rest the 256 x 128
// tiles of columns n_half .. n - 1.  When both classes are there, full is a
// multiple of 8, so both keep the XCD order.
template <int WMW, int WNW>
__global__ __launch_bounds__(64 * WMW * WNW, 1) void gemm_large_mx(
    int m, int n, int k, const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ b, const uint8_t* __restrict__ bs, void* __restrict__ c,
    int c_dtype, int tiles_m, int full, int half, int n_half, int ksplit, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) MxSmem smem;
  const int wg = blockIdx.x;
  if (wg < full)
    mx_tile<WMW, WNW, BN>(smem, xcd_tile(wg, full), m, n, k, a, as, b, bs, c, c_dtype, tiles_m, 0,
                          ksplit, part);
  else
    mx_tile<WMW, WNW, BN / 2>(smem, xcd_tile(wg - full, half), m, n, k, a, as, b, bs, c, c_dtype,
                              tiles_m, n_half, ksplit, part);
}

// Split k: C = ts (sum over slices of the fp32 partial sums), the slices
// added in order.  Thread -> 4 consecutive elements.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int nsplit,
                                                           int64_t mn, int64_t stride,
                                                           const float* __restrict__ at,
                                                           const float* __restrict__ bt,
                                                           void* __restrict__ c, int c_dtype) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  float4 s = *reinterpret_cast<const float4*>(part + i);
  for (int z = 1; z < nsplit; ++z) {
    const float4 v = *reinterpret_cast<const float4*>(part + z * stride + i);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  const float ts = at ? (*at) * (*bt) : 1.0f;
  const float o[4] = {s.x * ts, s.y * ts, s.z * ts, s.w * ts};
  if (i + 4 <= mn && c_dtype != kInF32) {
    const __bf16 h[4] = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
    *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(c) + i) = *reinterpret_cast<const uint2*>(h);
  } else if (i + 4 <= mn) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + i) = make_float4(o[0], o[1], o[2], o[3]);
  } else {
    for (int e = 0; i + e < mn; ++e) {
      if (c_dtype == kInF32) reinterpret_cast<float*>(c)[i + e] = o[e];
      else reinterpret_cast<__bf16*>(c)[i + e] = (__bf16)o[e];
    }
  }
}

}  // namespace

int64_t gemm_split_stride(int64_t m, int64_t n) { return split_stride(m, n); }

hipError_t launch_split_reduce(const float* part, int nsplit, int64_t m, int64_t n, const float* at,
                               const float* bt, void* c, int c_dtype, hipStream_t stream) {
  const int64_t mn = m * n;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((mn + 1023) / 1024)), dim3(256), 0, stream, part,
                     nsplit, mn, split_stride(m, n), at, bt, c, c_dtype);
  return hipGetLastError();
}

bool gemm_large_supported(int fmt, int64_t m, int64_t n, int64_t k) {
  const int64_t lim = int64_t(1) << 31;     // 32-bit buffer offsets
  // 16-byte scale rows: k a multiple of 512 (MXFP4) or 256 (NVFP4)
  const int64_t kq = (fmt == kFmtNV) ? 256 : 512;
  // MXFP4 tiles are moved back to lie inside the operands: n >= 256 (a small
  // m keeps one row of tiles at row 0: from 33 rows, where the 16-row decode
  // groups stop)
  const int64_t mmin = (fmt == kFmtNV) ? 128 : 33, nmin = (fmt == kFmtNV) ? 128 : 256;
  return m >= mmin && n >= nmin && k % kq == 0 && m * (k / 2) < lim && n * (k / 2) < lim;
}

namespace {

constexpr int64_t kCUs = 256;

// NVFP4 tile width: 224 or 256 columns, whichever needs fewer tile-column
// rounds of the 256 CUs (time ~ rounds x width).
int nv_tile_width(int64_t m, int64_t n) {
  const int64_t tiles_m = (m + BM - 1) / BM;
  auto cost = [&](int64_t bn) { return (tiles_m * ((n + bn - 1) / bn) + kCUs - 1) / kCUs * bn; };
  return cost(224) < cost(256) ? 224 : 256;
}

// Slices of k per tile: while the tiles (times the slices) fill at most half
// the CUs, split k in two again (at most 4 slices, each a whole number of the
// kernel's k-unit: 256 values NVFP4, 512 MXFP4) if that saves at least twice
// what it costs.  Saved: half of a slice's time, for a tile alone on its CU
// ~24 ns (NVFP4) or ~6.8 ns (MXFP4) per k-value as measured; cost: the fp32
// partial sums written and read back, 8 bytes per output and slice, at
// ~5 TB/s.  (MXFP4's 2048 x 3584 x 8192 in two slices: 28 us saved against
// 23 us of traffic, slower in practice; NVFP4's: 98 us against 23.)
int large_split(int fmt, int64_t m, int64_t n, int64_t k) {
  // MXFP4 with one row of tiles: half-width tiles instead (measured faster:
  // 128x14336x4096 22.6 us unsplit against 36 us in two slices)
  if (fmt == kFmtMX && m < BM) return 1;
  const int64_t bn = fmt == kFmtNV ? nv_tile_width(m, n) : BN;
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + bn - 1) / bn);
  const int64_t unit = fmt == kFmtNV ? 256 : 512;
  const double ns_per_k = fmt == kFmtNV ? 24.0 : 6.8;
  int s = 1;
  while (s < 4 && 2 * s * tiles <= kCUs && k % (2 * s * unit) == 0) {
    const double saved_ns = ns_per_k * (double)k / (2.0 * s);
    const double cost_ns = 8.0 * (2 * s - (s > 1 ? s : 0)) * (double)(m * n) / 5000.0;  // B / (B/ns)
    if (saved_ns < 2.0 * cost_ns) break;
    s *= 2;
  }
  return s;
}

// MXFP4 tile classes.  A 256 x 128 tile takes ~0.6 of a 256 x 256 tile's
// time, so half-width tiles pay where full ones would leave CUs idle:
// - the 256 x 256 tiles fill some whole rounds of the CUs and then at most
//   half of one more: the tile columns that fit in the whole rounds stay 256
//   wide and the rest of the columns go to 256 x 128 tiles (2048 x 28672 x
//   8192: 896 tiles, 3.5 rounds, become 768 + 256 half-width tiles);
// - the 256 x 256 tiles fill at most half the CUs: every tile is half-width
//   (2048 x 3584 x 8192: 112 tiles become 224).
// The time model counts rounds (a round of half-width tiles as 0.6) and keeps
// the full tiles unless it saves a tenth of a round.  full and half are the
// counts, n_half the first column of the half-width tiles.
void mx_tile_classes(int64_t m, int64_t n, int* full, int* half, int64_t* n_half) {
  const int64_t tiles_m = (m + BM - 1) / BM, ntiles = tiles_m * ((n + BN - 1) / BN);
  auto rounds = [](int64_t t) { return (double)((t + kCUs - 1) / kCUs); };
  *full = (int)ntiles;
  *half = 0;
  *n_half = n;
  double best = rounds(ntiles) - 0.1;
  const int64_t all_half = tiles_m * ((n + BN / 2 - 1) / (BN / 2));
  if (0.6 * rounds(all_half) < best) {
    best = 0.6 * rounds(all_half);
    *full = 0;
    *half = (int)all_half;
    *n_half = 0;
  }
  const int64_t rem = ntiles % kCUs;
  if (ntiles <= kCUs || rem == 0 || rem > kCUs / 2) return;
  int64_t cols = (ntiles - rem) / tiles_m;           // full-width tile columns
  while (cols > 0 && (tiles_m * cols) % NXCD != 0) --cols;
  const int64_t nh = cols * BN;
  if (cols == 0 || n - nh < BN / 2) return;
  const int64_t h = tiles_m * ((n - nh + BN / 2 - 1) / (BN / 2));
  const double split = rounds(tiles_m * cols) + 0.6 * rounds(h);
  if (split < best) {
    *full = (int)(tiles_m * cols);
    *half = (int)h;
    *n_half = nh;
  }
}

}  // namespace

size_t gemm_large_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
  const int s = large_split(fmt, m, n, k);
  return s > 1 ? (size_t)s * (size_t)split_stride(m, n) * sizeof(float) : 0;
}

hipError_t launch_gemm_large(int fmt, int64_t m, int64_t n, int64_t k,
                             const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_tscale, const uint8_t* b_codes,
                             const uint8_t* b_scales, const float* b_tscale,
                             void* c, int c_dtype, void* workspace, hipStream_t stream) {
  const int nsplit = large_split(fmt, m, n, k);
  const int ksplit = (int)(k / nsplit);
  float* part = nsplit > 1 ? reinterpret_cast<float*>(workspace) : nullptr;
  const int tiles_m = (int)((m + BM - 1) / BM);
  if (fmt == kFmtMX) {
    int full = (int)(tiles_m * ((n + BN - 1) / BN)), half = 0;
    int64_t n_half = n;
    if (nsplit == 1) mx_tile_classes(m, n, &full, &half, &n_half);
    hipLaunchKernelGGL((gemm_large_mx<kMXWM, kMXWN>), dim3((unsigned)(full + half), (unsigned)nsplit),
                       dim3(64 * kMXWM * kMXWN), 0, stream, (int)m, (int)n, (int)k, a_codes, a_scales,
                       b_codes, b_scales, c, c_dtype, tiles_m, full, half, (int)n_half, ksplit, part);
  } else if (nv_tile_width(m, n) == 224) {
    const int tn = (int)((n + 223) / 224);
    hipLaunchKernelGGL((gemm_nv4w<224>), dim3((unsigned)(tiles_m * tn), (unsigned)nsplit), dim3(256), 0,
                       stream, (int)m, (int)n, (int)k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                       b_tscale, c, c_dtype, tiles_m, tn, ksplit, part);
  } else {
    const int tn = (int)((n + 255) / 256);
    hipLaunchKernelGGL((gemm_nv4w<256>), dim3((unsigned)(tiles_m * tn), (unsigned)nsplit), dim3(256), 0,
                       stream, (int)m, (int)n, (int)k, a_codes, a_scales, a_tscale, b_codes, b_scales,
                       b_tscale, c, c_dtype, tiles_m, tn, ksplit, part);
  }
  if (nsplit > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t mn = m * n;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((mn + 1023) / 1024)), dim3(256), 0, stream,
                       part, nsplit, mn, split_stride(m, n), fmt == kFmtNV ? a_tscale : nullptr,
                       fmt == kFmtNV ? b_tscale : nullptr, c, c_dtype);
  }
  return hipGetLastError();
}

// MR-GPTQ weight quantization to NVFP4 / MXFP4 for gfx950.
//
// hyper.ai, paper 2509.23202 (MR-GPTQ), Abstract: GPTQ adapted to FP4 with
// blockwise Hadamard transforms (rotation fused into the weights, computed
// online for the activations).  pimento.cloud "FP8, NVFP4 czy AWQ?",
// section "Czym roznia sie FP8, NVFP4, MXFP4 i AWQ?": GPTQ quantizes the
// weights layer by layer with error correction.
//
// Pipeline (fp64 linear algebra; the quantization decisions in fp32 exactly
// as the quantizer takes them):
//   1. Wr, Xr: W and the calibration X rotated by the blockwise Hadamard
//      transform (fp32, as the fused quantizer), widened to fp64.
//   2. H = 2 / N Xr^T Xr (gemm_f64).
//   3. Dead features (H_jj = 0): H_jj = 1 and their weights zeroed; then
//      H_jj += damp * mean(diag H).  The damped H is stored flipped,
//      H'[i][j] = H[k-1-i][k-1-j].
//   4. X = L'^-1 for L' = cholesky(H'), recursively (cholinv: 128 x 128
//      leaves in one workgroup each, everything above them large GEMMs).
//      The upper Cholesky factor U of H^-1 is then U[i][j] = X[k-1-i][k-1-j]:
//      with J the reversal, H^-1 = J (J H J)^-1 J = (J L'^-1 J)^T (J L'^-1 J).
//   5. NVFP4 tensor scale max |Wr| / 2688.
//   6. The columns in blocks of 128: gptq_block_kernel walks a block's
//      columns for 64 rows per wave (weights in registers and LDS, U's block
//      in LDS): block scale from the current weights at each quantization
//      block start, code, err = (w - q) / U_jj, the block's later columns
//      take -err U_jj'; then the rest of the block's group of 512 columns
//      takes -E_block U[block, rest] in one gemm_f64, and after the group's
//      last block the columns right of the group take -E_group U[group,
//      right] in one more (GPTQ's deferred error correction, in two levels).
#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

constexpr int kBC = 128;         // GPTQ column block
constexpr int kOuter = 512;      // group of column blocks whose corrections of the
                                 // columns right of the group go out as one product
constexpr int kRows = 64;        // rows per GPTQ workgroup

// ---- C = beta C + alpha A B, general strides ------------------------------------
// A(i, t) = a[i * sa0 + t * sa1] (M x K), B(t, j) = b[t * sb0 + j * sb1]
// (K x N), C[i * ldc + j] (M x N).  beta == 0 never reads C.  A T x T tile
// (T = 32 or 64) per workgroup of 4 waves, each wave a T/2 x T/2 quarter as
// (T/32) x (T/32) v_mfma_f64_16x16x4_f64 tiles (lane l: A row l % 16 / B
// column l % 16 at k-slot l / 16; C column l % 16).  The tiles go through
// LDS in chunks of 2048 / T k; the next chunk's global loads are in flight
// while the current chunk is multiplied.  (Unlike the fp32 16 x 16 MFMAs,
// the fp64 one leaves item e of lane l at row 4 e + l / 16.)
// Triangular operands narrow each tile's k-range (the skipped products are
// zeros); kLowerTiles computes only the tiles that meet the lower triangle.
enum : int {
  kTriBTransLower = 1,   // B(t, j) = 0 for t > j: k ends at the tile's last column
  kTriBLower = 2,        // B(t, j) = 0 for t < j: k starts at the tile's first column
  kTriALower = 4,        // A(i, t) = 0 for t > i: k ends at the tile's last row
  kLowerTiles = 8,       // C: tiles strictly above the diagonal are left alone
};

struct GemmArgs {
  const double* a;
  const double* b;
  double* c;
  int64_t sa0, sa1, sb0, sb1, ldc;
  int m, n, k;
  double alpha, beta;
  int tri;
};

typedef double v4d __attribute__((ext_vector_type(4)));

template <int T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemm_f64_kernel(
    GemmArgs G) {
  constexpr int KC = 2048 / T;           // k-chunk: 8 elements of A and of B per thread
  constexpr int NT = T / 32;             // MFMA tiles per wave along each side
  __shared__ double As[KC][T + 1];
  __shared__ double Bs[KC][T + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // a triangular operand makes the tiles' k-ranges unequal: the longest go
  // out first (tile columns or rows in order of their k-range, slowest index)
  int bx = blockIdx.x, by = blockIdx.y;
  const int lin = by * gridDim.x + bx;
  if (G.tri & kTriBTransLower) {
    bx = gridDim.x - 1 - lin / gridDim.y;
    by = lin % gridDim.y;
  } else if (G.tri & kTriBLower) {
    bx = lin / gridDim.y;
    by = lin % gridDim.y;
  } else if (G.tri & kTriALower) {
    by = gridDim.y - 1 - lin / gridDim.x;
    bx = lin % gridDim.x;
  }
  const int i0 = by * T, j0 = bx * T;
  const int wr = (T / 2) * (wave >> 1), wc = (T / 2) * (wave & 1);
  if ((G.tri & kLowerTiles) && j0 > i0) return;
  int kb = 0, ke = G.k;
  if (G.tri & kTriBTransLower) ke = min(ke, j0 + T);
  if (G.tri & kTriBLower) kb = j0;
  if (G.tri & kTriALower) ke = min(ke, i0 + T);
  // loaders: T * KC elements of each tile, fastest along the unit-stride side.
  // Element e of a thread sits at a fixed offset (along the tile's row or k
  // side) from the thread's first one, so one base pointer per operand and a
  // uniform step per element give every address.
  const bool a_i_fast = (G.sa0 < 0 ? -G.sa0 : G.sa0) <= (G.sa1 < 0 ? -G.sa1 : G.sa1);
  const bool b_j_fast = (G.sb1 < 0 ? -G.sb1 : G.sb1) <= (G.sb0 < 0 ? -G.sb0 : G.sb0);
  const int a_i = a_i_fast ? tid % T : tid / KC, a_t = a_i_fast ? tid / T : tid % KC;
  const int a_di = a_i_fast ? 0 : 256 / KC, a_dt = a_i_fast ? 256 / T : 0;
  const int b_j = b_j_fast ? tid % T : tid / KC, b_t = b_j_fast ? tid / T : tid % KC;
  const int b_dj = b_j_fast ? 0 : 256 / KC, b_dt = b_j_fast ? 256 / T : 0;
  const double* a_base = G.a + (int64_t)(i0 + a_i) * G.sa0 + (int64_t)a_t * G.sa1;
  const double* b_base = G.b + (int64_t)b_t * G.sb0 + (int64_t)(j0 + b_j) * G.sb1;
  const int64_t a_step = a_di * G.sa0 + a_dt * G.sa1, b_step = b_dt * G.sb0 + b_dj * G.sb1;
  double ra[8], rb[8];
  const bool inner = i0 + T <= G.m && j0 + T <= G.n;   // no row or column bound
  auto fetch = [&](int t0) {
    const double* pa = a_base + (int64_t)t0 * G.sa1;
    const double* pb = b_base + (int64_t)t0 * G.sb0;
    if (inner && t0 + KC <= G.k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ra[e] = pa[e * a_step];
        rb[e] = pb[e * b_step];
      }
      return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool oka = i0 + a_i + a_di * e < G.m && t0 + a_t + a_dt * e < G.k;
      ra[e] = oka ? pa[e * a_step] : 0.0;
      const bool okb = j0 + b_j + b_dj * e < G.n && t0 + b_t + b_dt * e < G.k;
      rb[e] = okb ? pb[e * b_step] : 0.0;
    }
  };
  v4d acc[NT][NT];
#pragma unroll
  for (int x = 0; x < NT; ++x)
#pragma unroll
    for (int y = 0; y < NT; ++y) acc[x][y] = (v4d){0.0, 0.0, 0.0, 0.0};
  if (kb < ke) fetch(kb);
  for (int t0 = kb; t0 < ke; t0 += KC) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      As[a_t + a_dt * e][a_i + a_di * e] = ra[e];
      Bs[b_t + b_dt * e][b_j + b_dj * e] = rb[e];
    }
    __syncthreads();
    if (t0 + KC < ke) fetch(t0 + KC);
#pragma unroll
    for (int ks = 0; ks < KC; ks += 4) {
      const int kk = ks + (lane >> 4), r = lane & 15;
      double av[NT], bv[NT];
#pragma unroll
      for (int x = 0; x < NT; ++x) av[x] = As[kk][wr + 16 * x + r];
#pragma unroll
      for (int y = 0; y < NT; ++y) bv[y] = Bs[kk][wc + 16 * y + r];
#pragma unroll
      for (int x = 0; x < NT; ++x)
#pragma unroll
        for (int y = 0; y < NT; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
    __syncthreads();
  }
  // all of C's old values are read before the first store (a store ahead of
  // a load of the same array would make every element a round trip)
  if (G.beta != 0.0) {
#pragma unroll
    for (int x = 0; x < NT; ++x)
#pragma unroll
      for (int y = 0; y < NT; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = i0 + wr + 16 * x + 4 * e + (lane >> 4);
          const int gj = j0 + wc + 16 * y + (lane & 15);
          const double old = (gi < G.m && gj < G.n) ? G.c[gi * G.ldc + gj] : 0.0;
          acc[x][y][e] = G.beta * old + G.alpha * acc[x][y][e];
        }
  } else {
#pragma unroll
    for (int x = 0; x < NT; ++x)
#pragma unroll
      for (int y = 0; y < NT; ++y) acc[x][y] *= G.alpha;
  }
#pragma unroll
  for (int x = 0; x < NT; ++x)
#pragma unroll
    for (int y = 0; y < NT; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = i0 + wr + 16 * x + 4 * e + (lane >> 4);
        const int gj = j0 + wc + 16 * y + (lane & 15);
        if (gi < G.m && gj < G.n) G.c[gi * G.ldc + gj] = acc[x][y][e];
      }
}

// A 32 x 32 tile (64-k chunks) where 64 x 64 tiles would leave most of the
// chip idle: the small products at the bottom of the factorization's
// recursion, bound by the latency of their k-loop.
hipError_t gemm_f64(const GemmArgs& G, hipStream_t stream) {
  if (G.m <= 0 || G.n <= 0) return hipSuccess;
  const int64_t t64 = (int64_t)((G.m + 63) / 64) * ((G.n + 63) / 64);
  if (t64 < 64) {
    const dim3 grid((unsigned)((G.n + 31) / 32), (unsigned)((G.m + 31) / 32));
    hipLaunchKernelGGL(gemm_f64_kernel<32>, grid, dim3(256), 0, stream, G);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((G.n + 63) / 64), (unsigned)((G.m + 63) / 64));
  hipLaunchKernelGGL(gemm_f64_kernel<64>, grid, dim3(256), 0, stream, G);
  return hipGetLastError();
}

// ---- dead features, damping, flip -------------------------------------------------
// One workgroup: dead[j] = (H_jj == 0); scal[0] = damp * mean of the diagonal
// with the dead entries counted as 1.
__global__ __launch_bounds__(1024) void gptq_damp_kernel(const double* __restrict__ H, int k,
                                                         double damp, int* __restrict__ dead,
                                                         double* __restrict__ scal) {
  __shared__ double part[1024];
  double s = 0.0;
  for (int j = threadIdx.x; j < k; j += 1024) {
    const double d = H[(int64_t)j * k + j];
    dead[j] = d == 0.0;
    s += d == 0.0 ? 1.0 : d;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) scal[0] = damp * (part[0] / k);
}

// Hf[i][j] = H[k-1-i][k-1-j], diagonal dead -> 1, plus the damping.
__global__ __launch_bounds__(256) void gptq_flip_kernel(const double* __restrict__ H, int k,
                                                        const int* __restrict__ dead,
                                                        const double* __restrict__ scal,
                                                        double* __restrict__ Hf) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)k * k) return;
  const int i = (int)(idx / k), j = (int)(idx - (int64_t)i * k);
  const int si = k - 1 - i, sj = k - 1 - j;
  double v = si >= sj ? H[(int64_t)si * k + sj] : H[(int64_t)sj * k + si];   // lower part of H
  if (i == j) v = (dead[si] ? 1.0 : v) + scal[0];
  Hf[idx] = v;
}

// Zero the dead feature columns of the rotated weights [n, k].
__global__ __launch_bounds__(256) void gptq_zero_dead_kernel(double* __restrict__ W, int64_t n,
                                                             int k, const int* __restrict__ dead) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * k) return;
  if (dead[idx % k]) W[idx] = 0.0;
}

__global__ __launch_bounds__(256) void fill_f64_kernel(double* __restrict__ p, int64_t count) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < count) p[idx] = 0.0;
}

// max |W| (as fp32, a monotone rounding) -> NVFP4 tensor scale fp32(A) / 2688,
// in two passes: one partial maximum per workgroup, then one workgroup.
constexpr int kMaxParts = 1024;

__global__ __launch_bounds__(256) void gptq_amax_kernel(const double* __restrict__ W, int64_t count,
                                                        float* __restrict__ parts) {
  __shared__ float red[256];
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256)
    m = fmaxf(m, fabsf((float)W[i]));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) parts[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kMaxParts) void gptq_tscale_kernel(const float* __restrict__ parts,
                                                                int nparts, float* __restrict__ ts) {
  __shared__ float red[kMaxParts];
  red[threadIdx.x] = (int)threadIdx.x < nparts ? parts[threadIdx.x] : 0.0f;
  __syncthreads();
  for (int w = kMaxParts / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float s_t = red[0] / 2688.0f;             // 6 * 448
    ts[0] = s_t == 0.0f ? 1.0f : s_t;
  }
}

// ---- Cholesky factor and its inverse, recursively -----------------------------------
// cholinv(A) for the symmetric positive definite block A (lower part read):
// with A = [[A11, .], [A21, A22]],
//   L11, X11 = cholinv(A11)           (X11 = L11^-1)
//   L21 = A21 X11^T                   (= A21 L11^-T)
//   L22, X22 = cholinv(A22 - L21 L21^T)
//   X21 = -X22 L21 X11
// so every step above the 128 x 128 leaves is one large GEMM.  Only X = L^-1
// is kept: L21 lives in the X21 slot until X21 replaces it, the product
// L21 X11 in the (consumed) A21 slot.
constexpr int kLeaf = 128;

// Leaf: the 128 x 128 diagonal block at (p, p) of A, in one workgroup.  X =
// L^-1 comes out of one right-looking sweep that never forms L: thread
// (i, jj) keeps a[t] = A'[i][jj + 8t] (the trailing matrix) and
// x[t] = B'[i][jj + 8t] (B' = I minus the rows already eliminated) in
// registers.  With d_c = A'[c][c], step c takes, for every row r > c,
//   A'[r][j] -= A'[r][c] A'[j][c] / d_c   (c < j <= r)
//   B'[r]    -= A'[r][c] B'[c] / d_c
// and X's row r is B'[r] / sqrt(d_r) once step r - 1 is done (L's column c
// is A'[., c] / sqrt(d_c), so these are the usual updates with both factors
// unscaled).  The values step c reads (A'[., c] below the diagonal, B'[c]
// left of it: one LDS vector, as B'[c] is zero right of c) are published by
// their owners at the end of step c - 1, so each step has one barrier.  The
// whole 128 x 128 block of X is written, zeros above the diagonal included.
__global__ __launch_bounds__(1024) void cholinv_leaf_kernel(const double* __restrict__ A,
                                                            double* __restrict__ X, int k, int p) {
  __shared__ double v[2][kLeaf];
  __shared__ double inv_d[kLeaf];        // 1 / d_c
  __shared__ double inv_s[kLeaf];        // 1 / sqrt(d_c)
  const int tid = threadIdx.x, i = tid >> 3, jj = tid & 7;
  double a[kLeaf / 8], x[kLeaf / 8];
#pragma unroll
  for (int t = 0; t < kLeaf / 8; ++t) {
    const int col = jj + 8 * t;
    a[t] = col <= i ? A[(int64_t)(p + i) * k + p + col] : 0.0;
    x[t] = col == i ? 1.0 : 0.0;
  }
  // step 0's inputs: A'[., 0] and B'[0] = e_0
  if (jj == 0) v[0][i] = i == 0 ? 1.0 : a[0];
  if (i == 0 && jj == 0) {
    inv_d[0] = 1.0 / a[0];
    inv_s[0] = 1.0 / sqrt(a[0]);
  }
  __syncthreads();
#pragma unroll
  for (int tc = 0; tc < kLeaf / 8; ++tc) {
#pragma unroll 1
    for (int cj = 0; cj < 8; ++cj) {
      const int c = 8 * tc + cj, b = c & 1;
      if (i > c) {
        const double li = v[b][i] * inv_d[c];
        // a[t] right of the row's diagonal (and left of c) is never read
        // again, so those entries take the update unguarded
#pragma unroll
        for (int t = 0; t < kLeaf / 8; ++t) {
          const double u = v[b][jj + 8 * t];
          if (t > tc) {
            a[t] = fma(-li, u, a[t]);
          } else if (t < tc) {
            x[t] = fma(-li, u, x[t]);
          } else {
            a[t] = fma(-li, u, a[t]);
            x[t] = jj > cj ? x[t] : fma(-li, u, x[t]);
          }
        }
        // publish step c + 1's inputs: A'[., c+1] (owner jj == (c+1) & 7)
        // and B'[c + 1] (row c + 1)
        const int n1 = c + 1;
        const double an = cj < 7 ? a[tc] : a[tc + 1 < kLeaf / 8 ? tc + 1 : tc];
        if (jj == (n1 & 7)) {
          if (i > n1) v[b ^ 1][i] = an;
          if (i == n1) {
            // v_rcp_f64 / v_rsq_f64 refined by two Newton steps each
            double r = __builtin_amdgcn_rcp(an);
            r = fma(r, fma(-an, r, 1.0), r);
            r = fma(r, fma(-an, r, 1.0), r);
            double q = __builtin_amdgcn_rsq(an);
            q = q * fma(-0.5 * an * q, q, 1.5);
            q = q * fma(-0.5 * an * q, q, 1.5);
            inv_d[n1] = r;
            inv_s[n1] = q;
          }
        }
        if (i == n1) {
#pragma unroll
          for (int t = 0; t <= tc + 1 && t < kLeaf / 8; ++t)
            if (jj + 8 * t <= n1) v[b ^ 1][jj + 8 * t] = x[t];
        }
      }
      __syncthreads();
    }
  }
  const double sc = inv_s[i];
#pragma unroll
  for (int t = 0; t < kLeaf / 8; ++t) X[(int64_t)(p + i) * k + p + jj + 8 * t] = x[t] * sc;
}

// ---- the GPTQ column block ---------------------------------------------------------
// One wave per 64 rows, one row per lane.  The block's 128 columns are walked
// in four sub-blocks of 32: the sub-block's weights sit in registers, its
// columns are quantized in order and each err is corrected into the
// sub-block's later columns at once; then the sub-block's 32 errs correct
// the later sub-blocks' weights (kept in LDS), 32 columns at a time, in the
// errs' order.  U's block (uniform over the rows) is staged in LDS as 32 x 32
// tiles by rows and read with the same address in every lane.
constexpr int kSub = 32;

// U's tiles: ut[s] = the diagonal tile s (ut[s][i][c] = U[32s+i][32s+c], 0 for
// c < i), ut[4 + off_tile(s, s2)] = the tile (s, s2), s < s2, by rows.
constexpr int kTiles = 10;

struct BlockLds {
  double ut[kTiles][kSub][kSub];
  double ws[kBC][kRows];                   // the block's current weights, [column][row]
};

__device__ __forceinline__ int off_tile(int s, int s2) { return 3 * s - (s * (s - 1)) / 2 + (s2 - s - 1); }

// (s, s2) of tile slot t
__device__ __forceinline__ int tile_row(int t) { return t < 4 ? t : (t < 7 ? 0 : (t < 9 ? 1 : 2)); }
__device__ __forceinline__ int tile_col(int t) {
  return t < 4 ? t : (t < 7 ? t - 3 : (t < 9 ? t - 5 : 3));
}

template <int FMT>
__global__ __launch_bounds__(kRows) __attribute__((amdgpu_waves_per_eu(1, 1))) void gptq_block_kernel(const double* __restrict__ W, int64_t n,
                                                           int k, int c0,
                                                           const double* __restrict__ Xi,
                                                           const float* __restrict__ tscale,
                                                           double* __restrict__ E,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  constexpr bool NV = FMT == kFmtNV;
  constexpr int B = NV ? 16 : 32;
  __shared__ BlockLds L;
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * kRows + lane;
  const bool live = row < n;
  const int64_t rr = live ? row : n - 1;
  // U[c0 + a][c0 + b] = Xi[(k-1-c0-a) k + (k-1-c0-b)]
  const double* ub = Xi + (int64_t)(k - 1 - c0) * k + (k - 1 - c0);
  // staged in batches, all of a batch's loads in flight before its stores
  constexpr int kStage = 32;               // elements per lane per batch
  for (int base = 0; base < kTiles * kSub * kSub; base += kRows * kStage) {
    double val[kStage];
#pragma unroll
    for (int q = 0; q < kStage; ++q) {
      const int e = base + kRows * q + lane;
      const int t = e >> 10, i = (e >> 5) & (kSub - 1), c = e & (kSub - 1);
      const int a = kSub * tile_row(t) + i, b = kSub * tile_col(t) + c;
      val[q] = (e < kTiles * kSub * kSub && (t >= 4 || c >= i)) ? ub[-(int64_t)a * k - b] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < kStage; ++q) {
      const int e = base + kRows * q + lane;
      if (e < kTiles * kSub * kSub) (&L.ut[0][0][0])[e] = val[q];
    }
  }
  const double2* wrow = reinterpret_cast<const double2*>(W + rr * k + c0);
  for (int base = 0; base < kBC / 2; base += kStage / 2) {
    double2 val[kStage / 2];
#pragma unroll
    for (int q = 0; q < kStage / 2; ++q) val[q] = wrow[base + q];
#pragma unroll
    for (int q = 0; q < kStage / 2; ++q) {
      L.ws[2 * (base + q)][lane] = val[q].x;
      L.ws[2 * (base + q) + 1][lane] = val[q].y;
    }
  }
  __syncthreads();
  const float s_t = NV ? *tscale : 1.0f;
  const float d6 = 6.0f * s_t;
#pragma unroll 1
  for (int s = 0; s < kBC / kSub; ++s) {
    double w[kSub];
#pragma unroll
    for (int c = 0; c < kSub; ++c) w[c] = L.ws[kSub * s + c][lane];
    double e[kSub];
    uint32_t cw[4] = {0u, 0u, 0u, 0u};
    float r = 0.0f;
    double deq = 0.0;
    bool usable = false;
    // U's rows for the walk, one row ahead (row i+1 is read while column i
    // is worked on)
    const double2* ud2 = reinterpret_cast<const double2*>(&L.ut[s][0][0]);
    double2 uc[kSub / 2];
#pragma unroll
    for (int h = 0; h < kSub / 2; ++h) uc[h] = ud2[h];
#pragma unroll
    for (int i = 0; i < kSub; ++i) {
      const int col = c0 + kSub * s + i;
      double2 un[kSub / 2];
      if (i + 1 < kSub) {
#pragma unroll
        for (int h = (i + 1) / 2; h < kSub / 2; ++h) un[h] = ud2[(i + 1) * (kSub / 2) + h];
      }
      if ((i & (B - 1)) == 0) {
        // the block scale from the block's current weights, the quantizer's rule
        float a = 0.0f;
#pragma unroll
        for (int q = 0; q < B; ++q) a = fmaxf(a, fabsf((float)w[i + q]));
        uint32_t sbyte;
        if (NV) {
          sbyte = e4m3_encode_pos(a / d6);
          const float S = e4m3_decode_pos(sbyte) * s_t;
          r = 1.0f / S;
          usable = S != 0.0f && r < __builtin_inff();
          if (!usable) r = 0.0f;
          deq = (double)e4m3_decode_pos(sbyte) * (double)s_t;
        } else {
          usable = a > 0.0f;
          const int kx = usable ? mx_block_exponent(a) : -127;
          sbyte = (uint32_t)(kx + 127);
          r = usable ? as_f((uint32_t)(127 - kx) << 23) : 0.0f;
          deq = (double)block_scale_value<false>(sbyte);
        }
        if (live) scales[row * (k / B) + col / B] = (uint8_t)sbyte;
      }
      const float wf = (float)w[i];
      const uint32_t pk = e2m1_pack2<0>(0u, wf * r, 0.0f) & 0xFu;
      const uint32_t code = usable ? pk : (as_u(wf) >> 31) << 3;   // sign only
      const double q = usable ? (double)e2m1_unpack2<0>(pk).x * deq : 0.0;
      cw[i >> 3] |= code << (4 * (i & 7));
      const double err = (w[i] - q) / ((i & 1) ? uc[i / 2].y : uc[i / 2].x);
      e[i] = err;
#pragma unroll
      for (int c = i + 1; c < kSub; ++c) {
        w[c] = fma(-err, (c & 1) ? uc[c / 2].y : uc[c / 2].x, w[c]);
        // apply the update here: left to the compiler, the products sink
        // towards the next block-scale maximum and their operands pile up
        // in registers
        __asm__ volatile("" : "+v"(w[c]));
      }
#pragma unroll
      for (int h = (i + 1) / 2; h < kSub / 2; ++h) uc[h] = un[h];
    }
    if (live) {
      *reinterpret_cast<uint4*>(codes + row * (k / 2) + (c0 + kSub * s) / 2) =
          make_uint4(cw[0], cw[1], cw[2], cw[3]);
      double* er = E + row * kOuter + kSub * s;
#pragma unroll
      for (int i = 0; i < kSub; i += 2)
        *reinterpret_cast<double2*>(er + i) = make_double2(e[i], e[i + 1]);
    }
    for (int s2 = s + 1; s2 < kBC / kSub; ++s2) {
      const int t = off_tile(s, s2);
      double v[kSub];
#pragma unroll
      for (int c = 0; c < kSub; ++c) v[c] = L.ws[kSub * s2 + c][lane];
      const double2* uo2 = reinterpret_cast<const double2*>(&L.ut[4 + t][0][0]);
      double2 uc2[kSub / 2];
#pragma unroll
      for (int h = 0; h < kSub / 2; ++h) uc2[h] = uo2[h];
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        double2 un2[kSub / 2];
        if (i + 1 < kSub) {
#pragma unroll
          for (int h = 0; h < kSub / 2; ++h) un2[h] = uo2[(i + 1) * (kSub / 2) + h];
        }
#pragma unroll
        for (int h = 0; h < kSub / 2; ++h) {
          v[2 * h] = fma(-e[i], uc2[h].x, v[2 * h]);
          v[2 * h + 1] = fma(-e[i], uc2[h].y, v[2 * h + 1]);
        }
#pragma unroll
        for (int h = 0; h < kSub / 2; ++h) uc2[h] = un2[h];
      }
#pragma unroll
      for (int c = 0; c < kSub; ++c) L.ws[kSub * s2 + c][lane] = v[c];
    }
  }
}

}  // namespace

size_t gptq_workspace_bytes(int64_t n, int64_t k, int64_t n_calib) {
  // Wr [n, k], Xr [N, k], two k x k matrices, E [n, 512], the partial
  // maxima, scalars and the dead flags
  const int64_t doubles = n * k + n_calib * k + 2 * k * k + n * kOuter + kMaxParts / 2 + 4;
  return (size_t)doubles * sizeof(double) + (size_t)k * sizeof(int) + 256;
}

namespace {

// L^-1 of the Cholesky factor of the n x n block at (p, p) of A into the same
// block of X (A's block is consumed); n a multiple of 128.
hipError_t cholinv(double* A, double* X, int k, int p, int n, hipStream_t stream) {
  if (n == kLeaf) {
    hipLaunchKernelGGL(cholinv_leaf_kernel, dim3(1), dim3(1024), 0, stream, A, X, k, p);
    return hipGetLastError();
  }
  const int h = kLeaf * ((n / kLeaf + 1) / 2), r = n - h;
  const int64_t K = k;
  double* A21 = A + (p + h) * K + p;
  double* A22 = A + (p + h) * K + p + h;
  double* X11 = X + p * K + p;
  double* X21 = X + (p + h) * K + p;
  double* X22 = X + (p + h) * K + p + h;
  hipError_t e = cholinv(A, X, k, p, h, stream);
  if (e != hipSuccess) return e;
  // L21 = A21 X11^T into the X21 slot
  const GemmArgs g1 = {A21, X11, X21, K, 1, 1, K, K, r, h, h, 1.0, 0.0, kTriBTransLower};
  if ((e = gemm_f64(g1, stream)) != hipSuccess) return e;
  // A22 -= L21 L21^T (its lower part)
  const GemmArgs g2 = {X21, X21, A22, K, 1, 1, K, K, r, r, h, -1.0, 1.0, kLowerTiles};
  if ((e = gemm_f64(g2, stream)) != hipSuccess) return e;
  if ((e = cholinv(A, X, k, p + h, r, stream)) != hipSuccess) return e;
  // L21 X11 into the A21 slot, then X21 = -X22 (L21 X11)
  const GemmArgs g3 = {X21, X11, A21, K, 1, K, 1, K, r, h, h, 1.0, 0.0, kTriBLower};
  if ((e = gemm_f64(g3, stream)) != hipSuccess) return e;
  const GemmArgs g4 = {X22, A21, X21, K, 1, K, 1, K, r, h, r, -1.0, 0.0, kTriALower};
  return gemm_f64(g4, stream);
}

}  // namespace

hipError_t launch_gptq(int fmt, const void* w, int w_dtype, int64_t n, int64_t k, const void* x,
                       int x_dtype, int64_t n_calib, double damp, bool rotate, uint8_t* codes,
                       uint8_t* scales, float* tscale, void* workspace, hipStream_t stream) {
  const int bsz = fmt == kFmtNV ? 16 : 32;
  double* Wr = reinterpret_cast<double*>(workspace);
  double* Xr = Wr + n * k;
  double* H = Xr + n_calib * k;          // H, then the inverse of the factor
  double* Lf = H + k * k;                // flipped damped H (consumed by the factorization)
  double* E = Lf + k * k;
  float* parts = reinterpret_cast<float*>(E + n * kOuter);
  double* scal = E + n * kOuter + kMaxParts / 2;
  int* dead = reinterpret_cast<int*>(scal + 4);
  const int ki = (int)k;
  hipError_t e;
#define FP4_TRY(call) \
  if ((e = (call)) != hipSuccess) return e
  FP4_TRY(launch_rotate_f64(w, w_dtype, n * k, rotate ? bsz : 0, Wr, stream));
  FP4_TRY(launch_rotate_f64(x, x_dtype, n_calib * k, rotate ? bsz : 0, Xr, stream));
  // H = 2 / N Xr^T Xr (lower tiles): A(i, t) = Xr[t][i], B(t, j) = Xr[t][j]
  {
    GemmArgs G = {Xr, Xr, H, 1, k, k, 1, k, ki, ki, (int)n_calib, 2.0 / (double)n_calib, 0.0,
                  kLowerTiles};
    FP4_TRY(gemm_f64(G, stream));
  }
  hipLaunchKernelGGL(gptq_damp_kernel, dim3(1), dim3(1024), 0, stream, H, ki, damp, dead, scal);
  const unsigned kk_grid = (unsigned)((k * k + 255) / 256);
  hipLaunchKernelGGL(gptq_flip_kernel, dim3(kk_grid), dim3(256), 0, stream, H, ki, dead, scal, Lf);
  const unsigned nk_grid = (unsigned)((n * k + 255) / 256);
  hipLaunchKernelGGL(gptq_zero_dead_kernel, dim3(nk_grid), dim3(256), 0, stream, Wr, n, ki, dead);
  // the inverse of the factor into H: zeros above the diagonal first
  hipLaunchKernelGGL(fill_f64_kernel, dim3(kk_grid), dim3(256), 0, stream, H, k * k);
  FP4_TRY(hipGetLastError());
  FP4_TRY(cholinv(Lf, H, ki, 0, ki, stream));
  float* ts = tscale;
  if (fmt == kFmtNV) {
    const int64_t want = (n * k + 256 * 64 - 1) / (256 * 64);
    const int np = (int)(want < kMaxParts ? want : kMaxParts);
    hipLaunchKernelGGL(gptq_amax_kernel, dim3(np), dim3(256), 0, stream, Wr, n * k, parts);
    hipLaunchKernelGGL(gptq_tscale_kernel, dim3(1), dim3(kMaxParts), 0, stream, parts, np, ts);
  }
  FP4_TRY(hipGetLastError());
  // the columns, 128 at a time, in groups of 512: each block's errs correct
  // the rest of its group at once, the group's errs (E [n, 512]) the columns
  // right of the group in one product with k = 512.  U[i][j] = X[k-1-i][k-1-j]
  const dim3 bgrid((unsigned)((n + kRows - 1) / kRows));
  for (int o0 = 0; o0 < ki; o0 += kOuter) {
    const int oe = o0 + kOuter < ki ? o0 + kOuter : ki;
    for (int c0 = o0; c0 < oe; c0 += kBC) {
      double* Eb = E + (c0 - o0);
      if (fmt == kFmtNV)
        hipLaunchKernelGGL((gptq_block_kernel<kFmtNV>), bgrid, dim3(kRows), 0, stream, Wr, n, ki,
                           c0, H, ts, Eb, codes, scales);
      else
        hipLaunchKernelGGL((gptq_block_kernel<kFmtMX>), bgrid, dim3(kRows), 0, stream, Wr, n, ki,
                           c0, H, ts, Eb, codes, scales);
      const int right = oe - c0 - kBC;
      if (right > 0) {
        // W[:, c0+128 : oe] -= E_b U[c0 : c0+128, c0+128 : oe]
        const double* ub = H + (int64_t)(k - 1 - c0) * k + (k - 1 - c0 - kBC);
        GemmArgs G = {Eb, ub, Wr + c0 + kBC, kOuter, 1, -k, -1, k, (int)n, right, kBC, -1.0, 1.0, 0};
        FP4_TRY(gemm_f64(G, stream));
      }
    }
    const int right = ki - oe;
    if (right > 0) {
      // W[:, oe:] -= E U[o0 : oe, oe:]
      const double* ub = H + (int64_t)(k - 1 - o0) * k + (k - 1 - oe);
      GemmArgs G = {E, ub, Wr + oe, kOuter, 1, -k, -1, k, (int)n, right, oe - o0, -1.0, 1.0, 0};
      FP4_TRY(gemm_f64(G, stream));
    }
  }
#undef FP4_TRY
  return hipGetLastError();
}

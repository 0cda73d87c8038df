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
//   4. L' = cholesky(H') (lower, blocked: 32-wide panels), X = L'^-1
//      (blocked by 32-row strips).  The upper Cholesky factor U of H^-1 is
//      then U[i][j] = X[k-1-i][k-1-j]: with J the reversal, H^-1 =
//      J (J H J)^-1 J = (J L'^-1 J)^T (J L'^-1 J).
//   5. NVFP4 tensor scale max |Wr| / 2688.
//   6. The columns in blocks of 128: gptq_block_kernel walks a block's
//      columns for 64 rows per workgroup (the block in LDS, U read with
//      uniform loads): block scale from the current weights at each
//      quantization block start, code, err = (w - q) / U_jj, the block's
//      later columns take -err U_jj'; then the columns right of the block
//      take -E U[block, right] in one gemm_f64 (the error correction of all
//      later columns, deferred to the block's end as one product).
#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

constexpr int kNB = 32;          // Cholesky / inverse panel width
constexpr int kBC = 128;         // GPTQ column block
constexpr int kRows = 64;        // rows per GPTQ workgroup
constexpr int kGT = 64;          // gemm_f64 tile
constexpr int kGK = 32;          // gemm_f64 k-chunk

// ---- C = beta C + alpha A B, general strides ------------------------------------
// A(i, t) = a[i * sa0 + t * sa1] (M x K), B(t, j) = b[t * sb0 + j * sb1]
// (K x N), C[i * ldc + j] (M x N).  beta == 0 never reads C.  64 x 64 tile
// per workgroup of 4 waves, each wave a 32 x 32 quarter as 2 x 2
// v_mfma_f64_16x16x4_f64 tiles (lane l: A row l % 16 / B column l % 16 at
// k-slot l / 16; C column l % 16).  The tiles go through LDS in
// chunks of 32 k; the next chunk's global loads are in flight while the
// current chunk is multiplied.  (Unlike the fp32 16 x 16 MFMAs, the fp64
// one leaves item e of lane l at row 4 e + l / 16.)
struct GemmArgs {
  const double* a;
  const double* b;
  double* c;
  int64_t sa0, sa1, sb0, sb1, ldc;
  int m, n, k;
  double alpha, beta;
};

typedef double v4d __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void gemm_f64_kernel(GemmArgs G) {
  __shared__ double As[kGK][kGT + 1];
  __shared__ double Bs[kGK][kGT + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = blockIdx.y * kGT, j0 = blockIdx.x * kGT;
  const int wr = 32 * (wave >> 1), wc = 32 * (wave & 1);
  // loaders: 2048 elements of each tile, fastest along the unit-stride side
  const bool a_i_fast = (G.sa0 < 0 ? -G.sa0 : G.sa0) <= (G.sa1 < 0 ? -G.sa1 : G.sa1);
  const bool b_j_fast = (G.sb1 < 0 ? -G.sb1 : G.sb1) <= (G.sb0 < 0 ? -G.sb0 : G.sb0);
  double ra[8], rb[8];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e;
      const int ii = a_i_fast ? (idx & 63) : (idx >> 5);
      const int tt = a_i_fast ? (idx >> 6) : (idx & 31);
      const int gi = i0 + ii, gt = t0 + tt;
      ra[e] = (gi < G.m && gt < G.k) ? G.a[gi * G.sa0 + gt * G.sa1] : 0.0;
      const int jj = b_j_fast ? (idx & 63) : (idx >> 5);
      const int tb = b_j_fast ? (idx >> 6) : (idx & 31);
      const int gj = j0 + jj, gtb = t0 + tb;
      rb[e] = (gj < G.n && gtb < G.k) ? G.b[gtb * G.sb0 + gj * G.sb1] : 0.0;
    }
  };
  v4d acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = (v4d){0.0, 0.0, 0.0, 0.0};
  fetch(0);
  for (int t0 = 0; t0 < G.k; t0 += kGK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e;
      As[a_i_fast ? (idx >> 6) : (idx & 31)][a_i_fast ? (idx & 63) : (idx >> 5)] = ra[e];
      Bs[b_j_fast ? (idx >> 6) : (idx & 31)][b_j_fast ? (idx & 63) : (idx >> 5)] = rb[e];
    }
    __syncthreads();
    if (t0 + kGK < G.k) fetch(t0 + kGK);
#pragma unroll
    for (int ks = 0; ks < kGK; ks += 4) {
      const int kk = ks + (lane >> 4), r = lane & 15;
      const double a0 = As[kk][wr + r], a1 = As[kk][wr + 16 + r];
      const double b0 = Bs[kk][wc + r], b1 = Bs[kk][wc + 16 + r];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = i0 + wr + 16 * x + 4 * e + (lane >> 4);
        const int gj = j0 + wc + 16 * y + (lane & 15);
        if (gi < G.m && gj < G.n) {
          double* p = G.c + gi * G.ldc + gj;
          *p = G.beta == 0.0 ? G.alpha * acc[x][y][e] : G.beta * *p + G.alpha * acc[x][y][e];
        }
      }
}

hipError_t gemm_f64(const GemmArgs& G, hipStream_t stream) {
  if (G.m <= 0 || G.n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((G.n + kGT - 1) / kGT), (unsigned)((G.m + kGT - 1) / kGT));
  hipLaunchKernelGGL(gemm_f64_kernel, grid, dim3(256), 0, stream, G);
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
  double v = H[(int64_t)si * k + sj];
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

// ---- Cholesky of the flipped Hessian, in place (lower) ----------------------------
// Diagonal block at (p0, p0): unblocked, in LDS.
__global__ __launch_bounds__(256) void chol_diag_kernel(double* __restrict__ A, int k, int p0) {
  __shared__ double S[kNB][kNB + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int i = e / kNB, j = e % kNB;
    S[i][j] = A[(int64_t)(p0 + i) * k + p0 + j];
  }
  __syncthreads();
  for (int c = 0; c < kNB; ++c) {
    if (tid == 0) S[c][c] = sqrt(S[c][c]);
    __syncthreads();
    if (tid > c && tid < kNB) S[tid][c] = S[tid][c] / S[c][c];
    __syncthreads();
    for (int e = tid; e < kNB * kNB; e += 256) {
      const int i = e / kNB, j = e % kNB;
      if (j > c && i >= j) S[i][j] -= S[i][c] * S[j][c];
    }
    __syncthreads();
  }
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int i = e / kNB, j = e % kNB;
    if (j <= i) A[(int64_t)(p0 + i) * k + p0 + j] = S[i][j];
  }
}

// Rows below the panel: L_ip = A_ip L_pp^-T, one thread per row.
__global__ __launch_bounds__(256) void chol_trsm_kernel(double* __restrict__ A, int k, int p0) {
  __shared__ double P[kNB][kNB + 1];
  for (int e = threadIdx.x; e < kNB * kNB; e += 256) {
    const int i = e / kNB, j = e % kNB;
    P[i][j] = j <= i ? A[(int64_t)(p0 + i) * k + p0 + j] : 0.0;
  }
  __syncthreads();
  const int row = p0 + kNB + blockIdx.x * 256 + threadIdx.x;
  if (row >= k) return;
  double* a = A + (int64_t)row * k + p0;
  double x[kNB];
#pragma unroll
  for (int c = 0; c < kNB; ++c) {
    double v = a[c];
#pragma unroll
    for (int t = 0; t < c; ++t) v -= x[t] * P[c][t];
    x[c] = v / P[c][c];
  }
#pragma unroll
  for (int c = 0; c < kNB; ++c) a[c] = x[c];
}

// ---- inverse of the lower factor, by 32-row strips ----------------------------------
// X_ii = L_ii^-1 (lower 32 x 32, zeros above its diagonal).
__global__ __launch_bounds__(256) void trtri_diag_kernel(const double* __restrict__ L,
                                                         double* __restrict__ X, int k, int i0) {
  __shared__ double S[kNB][kNB + 1];
  __shared__ double R[kNB][kNB + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int i = e / kNB, j = e % kNB;
    S[i][j] = j <= i ? L[(int64_t)(i0 + i) * k + i0 + j] : 0.0;
    R[i][j] = 0.0;
  }
  __syncthreads();
  // column c of the inverse by forward substitution, one thread per column
  if (tid < kNB) {
    const int c = tid;
    R[c][c] = 1.0 / S[c][c];
    for (int r = c + 1; r < kNB; ++r) {
      double v = 0.0;
      for (int t = c; t < r; ++t) v += S[r][t] * R[t][c];
      R[r][c] = -v / S[r][r];
    }
  }
  __syncthreads();
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int i = e / kNB, j = e % kNB;
    X[(int64_t)(i0 + i) * k + i0 + j] = R[i][j];
  }
}

// ---- the GPTQ column block ---------------------------------------------------------
// Workgroup = 64 rows (one thread each) x the block's 128 columns, kept in
// LDS as Ws[column][row].  U[i][j] = Xi[(k-1-i) k + (k-1-j)] is uniform over
// the workgroup.  Codes and scale bytes go out as they are decided; E
// [n, 128] receives err for the deferred update of the later columns.
template <int FMT>
__global__ __launch_bounds__(kRows) void gptq_block_kernel(double* __restrict__ W, int64_t n, int k,
                                                           int c0, const double* __restrict__ Xi,
                                                           const float* __restrict__ tscale,
                                                           double* __restrict__ E,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  constexpr bool NV = FMT == kFmtNV;
  constexpr int B = NV ? 16 : 32;
  __shared__ double Ws[kBC][kRows];
  const int t = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * kRows + t;
  const bool live = row < n;
  const int64_t rr = live ? row : n - 1;
  for (int j = 0; j < kBC; ++j) Ws[j][t] = W[rr * k + c0 + j];
  const float s_t = NV ? *tscale : 1.0f;
  const float d6 = 6.0f * s_t;
  float r = 0.0f;
  double deq = 0.0;
  bool usable = false;
  uint32_t pending = 0;
  for (int j = 0; j < kBC; ++j) {
    const int col = c0 + j;
    if ((j & (B - 1)) == 0) {
      // the block scale from the block's current weights, the quantizer's rule
      float a = 0.0f;
      for (int q = 0; q < B; ++q) a = fmaxf(a, fabsf((float)Ws[j + q][t]));
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
    const double w = Ws[j][t];
    const float wf = (float)w;
    uint32_t code;
    double q;
    if (usable) {
      const uint32_t pk = e2m1_pack2<0>(0u, wf * r, 0.0f) & 0xFu;
      code = pk;
      const v2f dv = e2m1_unpack2<0>(pk);
      q = (double)dv.x * deq;
    } else {
      code = (as_u(wf) >> 31) << 3;                  // sign only
      q = 0.0;
    }
    if (j & 1) {
      if (live) codes[row * (k / 2) + col / 2] = (uint8_t)(pending | (code << 4));
    } else {
      pending = code;
    }
    const double* urow = Xi + (int64_t)(k - 1 - col) * k + (k - 1 - col);   // U[col][col - x] backwards
    const double err = (w - q) / urow[0];
    if (live) E[row * kBC + j] = err;
    for (int jj = j + 1; jj < kBC; ++jj) Ws[jj][t] -= err * urow[-(jj - j)];
  }
}

}  // namespace

size_t gptq_workspace_bytes(int64_t n, int64_t k, int64_t n_calib) {
  // Wr [n, k], Xr [N, k], two k x k matrices, E [n, 128], the inverse's
  // strip product [32, k], dead flags and scalars
  const int64_t doubles = n * k + n_calib * k + 2 * k * k + n * kBC + (int64_t)kNB * k + 4;
  return (size_t)doubles * sizeof(double) + (size_t)k * sizeof(int) + 256;
}

hipError_t launch_gptq(int fmt, const void* w, int w_dtype, int64_t n, int64_t k, const void* x,
                       int x_dtype, int64_t n_calib, double damp, bool rotate, uint8_t* codes,
                       uint8_t* scales, float* tscale, void* workspace, hipStream_t stream) {
  const int bsz = fmt == kFmtNV ? 16 : 32;
  double* Wr = reinterpret_cast<double*>(workspace);
  double* Xr = Wr + n * k;
  double* H = Xr + n_calib * k;          // H, then the inverse of the factor
  double* Lf = H + k * k;                // flipped damped H, then its factor
  double* E = Lf + k * k;
  double* T = E + n * kBC;               // [32, k] strip product of the inverse
  double* scal = T + (int64_t)kNB * k;
  int* dead = reinterpret_cast<int*>(scal + 4);
  const int ki = (int)k;
  hipError_t e;
#define FP4_TRY(call) \
  if ((e = (call)) != hipSuccess) return e
  FP4_TRY(launch_rotate_f64(w, w_dtype, n * k, rotate ? bsz : 0, Wr, stream));
  FP4_TRY(launch_rotate_f64(x, x_dtype, n_calib * k, rotate ? bsz : 0, Xr, stream));
  // H = 2 / N Xr^T Xr: A(i, t) = Xr[t][i], B(t, j) = Xr[t][j]
  {
    GemmArgs G = {Xr, Xr, H, 1, k, k, 1, k, ki, ki, (int)n_calib, 2.0 / (double)n_calib, 0.0};
    FP4_TRY(gemm_f64(G, stream));
  }
  hipLaunchKernelGGL(gptq_damp_kernel, dim3(1), dim3(1024), 0, stream, H, ki, damp, dead, scal);
  const unsigned kk_grid = (unsigned)((k * k + 255) / 256);
  hipLaunchKernelGGL(gptq_flip_kernel, dim3(kk_grid), dim3(256), 0, stream, H, ki, dead, scal, Lf);
  const unsigned nk_grid = (unsigned)((n * k + 255) / 256);
  hipLaunchKernelGGL(gptq_zero_dead_kernel, dim3(nk_grid), dim3(256), 0, stream, Wr, n, ki, dead);
  FP4_TRY(hipGetLastError());
  // Cholesky of the flipped H in place
  for (int p0 = 0; p0 < ki; p0 += kNB) {
    hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, stream, Lf, ki, p0);
    const int below = ki - p0 - kNB;
    if (below > 0) {
      hipLaunchKernelGGL(chol_trsm_kernel, dim3((unsigned)((below + 255) / 256)), dim3(256), 0,
                         stream, Lf, ki, p0);
      // trailing A22 -= L21 L21^T over the full square (only its lower part is read later)
      const double* L21 = Lf + (int64_t)(p0 + kNB) * k + p0;
      GemmArgs G = {L21, L21, Lf + (int64_t)(p0 + kNB) * k + p0 + kNB, k, 1, 1, k, k,
                    below, below, kNB, -1.0, 1.0};
      FP4_TRY(gemm_f64(G, stream));
    }
  }
  // the inverse of the factor into H (zeros above the diagonal first)
  hipLaunchKernelGGL(fill_f64_kernel, dim3(kk_grid), dim3(256), 0, stream, H, k * k);
  for (int i0 = 0; i0 < ki; i0 += kNB) {
    hipLaunchKernelGGL(trtri_diag_kernel, dim3(1), dim3(256), 0, stream, Lf, H, ki, i0);
    if (i0 > 0) {
      // T = L[i0.., 0:i0] X[0:i0, 0:i0]; X[i0.., 0:i0] = -X_ii T
      GemmArgs G1 = {Lf + (int64_t)i0 * k, H, T, k, 1, k, 1, k, kNB, i0, i0, 1.0, 0.0};
      FP4_TRY(gemm_f64(G1, stream));
      GemmArgs G2 = {H + (int64_t)i0 * k + i0, T, H + (int64_t)i0 * k, k, 1, k, 1, k,
                     kNB, i0, kNB, -1.0, 0.0};
      FP4_TRY(gemm_f64(G2, stream));
    }
  }
  float* ts = tscale;
  if (fmt == kFmtNV) {
    float* parts = reinterpret_cast<float*>(T);     // the strip buffer is free again
    const int64_t want = (n * k + 256 * 64 - 1) / (256 * 64);
    const int np = (int)(want < kMaxParts ? want : kMaxParts);
    hipLaunchKernelGGL(gptq_amax_kernel, dim3(np), dim3(256), 0, stream, Wr, n * k, parts);
    hipLaunchKernelGGL(gptq_tscale_kernel, dim3(1), dim3(kMaxParts), 0, stream, parts, np, ts);
  }
  FP4_TRY(hipGetLastError());
  // the columns, 128 at a time
  const dim3 bgrid((unsigned)((n + kRows - 1) / kRows));
  for (int c0 = 0; c0 < ki; c0 += kBC) {
    if (fmt == kFmtNV)
      hipLaunchKernelGGL((gptq_block_kernel<kFmtNV>), bgrid, dim3(kRows), 0, stream, Wr, n, ki, c0,
                         H, ts, E, codes, scales);
    else
      hipLaunchKernelGGL((gptq_block_kernel<kFmtMX>), bgrid, dim3(kRows), 0, stream, Wr, n, ki, c0,
                         H, ts, E, codes, scales);
    const int right = ki - c0 - kBC;
    if (right > 0) {
      // W[:, c0+128:] -= E U[c0:c0+128, c0+128:], U[i][j] = X[k-1-i][k-1-j]
      const double* ub = H + (int64_t)(k - 1 - c0) * k + (k - 1 - c0 - kBC);
      GemmArgs G = {E, ub, Wr + c0 + kBC, kBC, 1, -k, -1, k, (int)n, right, kBC, -1.0, 1.0};
      FP4_TRY(gemm_f64(G, stream));
    }
  }
#undef FP4_TRY
  return hipGetLastError();
}

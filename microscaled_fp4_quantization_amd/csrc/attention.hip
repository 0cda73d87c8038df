// Decode attention over an FP4 (NVFP4 / MXFP4) KV cache for gfx950.
//
// hyper.ai story on the NVFP4 KV cache: the cache keeps K and V in 4-bit
// form and dequantizes them to FP8 before the attention computation.  Every
// cached element enters here as exactly the FP8 E4M3 byte the dequantize
// kernel gives it ((v * sb) * s_t rounded once to E4M3 for NVFP4,
// v * 2^(c-127) for MXFP4), and the attention of one new query token per
// sequence runs on those values:
//   out[b, j] = sum_t softmax_t(scale * K[t] . q[b, j]) V[t]
// over the first seq_lens[b] tokens of KV head j / G (grouped query heads).
//
// Dequantization by table.  The FP8 byte of an element depends only on its
// 3-bit magnitude, its sign bit and its block's scale byte, so each
// workgroup first tabulates, for all 256 scale bytes, the FP8 bytes of the
// 8 magnitudes (with the dequantize kernel's own arithmetic).  Then 4
// elements cost one v_perm_b32 (4 table bytes picked by 4 magnitudes) and a
// sign xor; FP8 -> f16 / bf16 is exact.
//
// Split-token decomposition: workgroup (bh, split) owns KV head bh % Hkv of
// sequence bh / Hkv and one chunk of its tokens; its 4 waves take 32-token
// steps in turn, each with its own running max, sum and output tile; the
// waves merge through LDS, the workgroup writes its partial (max, sum,
// unnormalized output) per query head and attn_merge_kernel merges the
// splits.  Scores live in the log2 domain: x = scale * log2(e) * (K . q),
// weights 2^(x - max).
//
// One 32-token step of a wave (lane l: r = l % 16, g = l / 16):
//   S = K Q^T, v_mfma_f32_16x16x32_{bf16,f16}, two 16-token tiles.  Row m
//     of tile T is token 16 T + 4 (m % 4) + m / 4, so the C layout (lane l
//     holds rows 4 g + e) leaves lane l the scores of tokens 4 j + g
//     (j = 4 T + e = 0..7) for query head r: exactly the k-slots of the B
//     operand of P V.  Lane
//     group g holds head-dim elements 32 g .. 32 g + 31 (16 code bytes);
//     inside a lane the k-slots follow the even/odd split of the table
//     lookup ({0, 2, 4, 6, 1, 3, 5, 7}) and Q is loaded in that order.
//   O += P V, v_mfma_f32_16x16x32_f16, 8 MFMAs: MFMA i has head-dim element
//     8 r + i in row r.  Lane l loads the 4 code bytes at 4 r of tokens
//     4 j + g (j = 0..7), looks them up and transposes the 8 x 8 FP8 bytes
//     so that fragment i holds element 8 r + i of those 8 tokens.  Every
//     cache load of a wave reads whole rows of consecutive tokens: 16 rows
//     (1 KiB) for a K tile, 4 rows for a V word.
#include "device_common.hpp"
#include "launch.hpp"

using namespace fp4dev;

namespace {

constexpr int kHeadDim = 128;
constexpr int kRowBytes = kHeadDim / 2;   // code bytes per cached token
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;                 // tokens per wave step
constexpr int kMaxGroup = 16;             // query heads per KV head (MFMA width)
constexpr int kPartPitch = kHeadDim + 4;
constexpr int64_t kTargetWorkgroups = 2048;
constexpr int64_t kMinChunk = 256;
constexpr float kLazy = 8.0f;             // log2 headroom before the running max moves

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct AttnLds {
  u32x2 lut[2][256];                           // [K, V][scale byte]: FP8 of magnitudes 0..7
  float part[kWaves][kMaxGroup][kPartPitch];   // per-wave unnormalized outputs
  float pm[kWaves][kMaxGroup];                 // per-wave running max (log2 domain)
  float pl[kWaves][kMaxGroup];                 // per-wave sum of weights
};

struct AttnArgs {
  const uint16_t* q;          // [B, Hq, 128] bf16 or f16
  const uint8_t* kc;          // [B, Hkv, t_max, 64]
  const uint8_t* ks;          // [B, Hkv, t_max, 128 / block]
  const float* kts;           // NVFP4 tensor scales (device)
  const uint8_t* vc;
  const uint8_t* vs;
  const float* vts;
  const int32_t* seq_lens;    // [B]
  float* part_o;              // [B Hkv, nsplit, G, 128]
  float* part_ml;             // [B Hkv, nsplit, G, 2]
  int64_t t_max;
  int64_t chunk;              // tokens per split (a multiple of 128)
  int hq, hkv, g, nsplit;
  float scale_log2;           // softmax scale * log2(e)
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Code word w (8 E2M1 codes) + table row -> FP8 bytes of the even elements
// (0, 2, 4, 6) and of the odd ones (1, 3, 5, 7).
__device__ __forceinline__ void lookup8(uint32_t w, u32x2 t, uint32_t& ev, uint32_t& od) {
  ev = perm(t.y, t.x, w & 0x07070707u) ^ ((w << 4) & 0x80808080u);
  od = perm(t.y, t.x, (w >> 4) & 0x07070707u) ^ (w & 0x80808080u);
}

// T_a = byte a of x0, x1, x2, x3 (a 4 x 4 byte transpose).
__device__ __forceinline__ void transpose4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                           uint32_t t[4]) {
  const uint32_t u01l = perm(x1, x0, 0x05010400u), u01h = perm(x1, x0, 0x07030602u);
  const uint32_t u23l = perm(x3, x2, 0x05010400u), u23h = perm(x3, x2, 0x07030602u);
  t[0] = perm(u23l, u01l, 0x05040100u);
  t[1] = perm(u23l, u01l, 0x07060302u);
  t[2] = perm(u23h, u01h, 0x05040100u);
  t[3] = perm(u23h, u01h, 0x07060302u);
}

// Max over the 4 lane groups of 16 (lanes l, l ^ 16, l ^ 32, l ^ 48):
// gfx950's row swaps, no LDS round trip.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// FP8 bytes 2 HI, 2 HI + 1 of x -> two f16 / bf16 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t f8_to_f16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HI));
}

template <bool HI>
__device__ __forceinline__ uint32_t f8_to_bf16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
}

template <int QDT>
__device__ __forceinline__ v4f mfma_qk(u32x4 a, u32x4 b, v4f c) {
  if (QDT == kInBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                               __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

struct AttnState {
  float m;                  // running max of the scaled scores (log2 domain)
  v4f ol;                   // sum of the weights (every row of this tile holds it)
  v4f o[8];                 // unnormalized output: o[i] row 4 g + e = element 32 g + 8 e + i
};

struct AttnPtrs {
  const uint8_t* kc;        // this (sequence, head)'s K codes, K scales, V codes, V scales
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  uint32_t koff, voff;      // this lane's byte offsets (token 0 of the step)
  int t_end;
};

// The cache words of one step, loaded a step ahead.
struct StepRegs {
  u32x4 kw[2];              // K codes: tiles T = 0, 1
  uint32_t ksb[2];          // their scale bytes (NVFP4: two blocks in 16 bits)
  uint32_t vw[8];           // V codes of tokens 4 j + g
  uint32_t vsb[8];          // their scale bytes
};

// K (V) words of the step at tokens t0 .. t0 + 31.  A step inside the live
// range addresses the cache through a uniform base plus this lane's
// offsets; a step running past t_end reads token t_end - 1 for the tokens
// beyond it (finite values; their weights are 0).
template <int FMT>
__device__ __forceinline__ void load_k(const AttnPtrs& P, int t0, int r, int g, StepRegs& R) {
  constexpr bool NV = FMT == kFmtNV;
  constexpr int kScaleBytes = NV ? kHeadDim / 16 : kHeadDim / 32;
  constexpr int kSShift = NV ? 3 : 4;       // code offset -> scale offset
  if (t0 + kStep <= P.t_end) {
    const uint8_t* kc = P.kc + (uint32_t)t0 * kRowBytes;
    const uint8_t* ks = P.ks + (uint32_t)t0 * kScaleBytes;
    const uint32_t kso = P.koff >> kSShift;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      R.kw[T] = *reinterpret_cast<const u32x4*>(kc + P.koff + 16 * T * kRowBytes);
      if (NV) R.ksb[T] = *reinterpret_cast<const uint16_t*>(ks + kso + 16 * T * kScaleBytes);
      else R.ksb[T] = ks[kso + 16 * T * kScaleBytes];
    }
  } else {
    const int t_last = P.t_end - 1;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      int tk = t0 + 16 * T + 4 * (r & 3) + (r >> 2);
      tk = tk < t_last ? tk : t_last;
      const uint32_t o = (uint32_t)tk * kRowBytes + 16 * g;
      R.kw[T] = *reinterpret_cast<const u32x4*>(P.kc + o);
      if (NV) R.ksb[T] = *reinterpret_cast<const uint16_t*>(P.ks + (o >> kSShift));
      else R.ksb[T] = P.ks[o >> kSShift];
    }
  }
}

template <int FMT>
__device__ __forceinline__ void load_v(const AttnPtrs& P, int t0, int r, int g, StepRegs& R) {
  constexpr bool NV = FMT == kFmtNV;
  constexpr int kScaleBytes = NV ? kHeadDim / 16 : kHeadDim / 32;
  constexpr int kSShift = NV ? 3 : 4;
  if (t0 + kStep <= P.t_end) {
    const uint8_t* vc = P.vc + (uint32_t)t0 * kRowBytes;
    const uint8_t* vs = P.vs + (uint32_t)t0 * kScaleBytes;
    const uint32_t vso = P.voff >> kSShift;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      R.vw[j] = *reinterpret_cast<const uint32_t*>(vc + P.voff + 4 * j * kRowBytes);
      R.vsb[j] = vs[vso + 4 * j * kScaleBytes];
    }
  } else {
    const int t_last = P.t_end - 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int tv = t0 + 4 * j + g;
      tv = tv < t_last ? tv : t_last;
      const uint32_t o = (uint32_t)tv * kRowBytes + 4 * r;
      R.vw[j] = *reinterpret_cast<const uint32_t*>(P.vc + o);
      R.vsb[j] = P.vs[o >> kSShift];
    }
  }
}

// One 32-token step of a wave at tokens t0 .. t0 + 31 on the words in R;
// refills R with the words of the wave's next step tn as soon as each part
// has been used (K after the scores, V after its table lookups), so those
// loads run under this step's arithmetic.  TAIL: the step runs past t_end
// and its scores beyond it are masked to weight 0.
template <int FMT, int QDT, bool TAIL>
__device__ __forceinline__ void attn_step(const AttnLds& L, const AttnPtrs& P, const u32x4 qf[4],
                                          float c2, int t0, int tn, int r, int g, StepRegs& R,
                                          AttnState& st) {
  constexpr bool NV = FMT == kFmtNV;
  const bool more = tn < P.t_end;
  const u32x4 kw[2] = {R.kw[0], R.kw[1]};
  const uint32_t ksb[2] = {R.ksb[0], R.ksb[1]};

  // ---- S = K Q^T ----------------------------------------------------------------
  v4f s[2];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    s[T] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t sb = NV ? ((c < 2) ? (ksb[T] & 0xFFu) : (ksb[T] >> 8)) : ksb[T];
      uint32_t ev, od;
      lookup8(kw[T][c], L.lut[0][sb], ev, od);
      u32x4 kf;
      if (QDT == kInBF16) {
        kf = (u32x4){f8_to_bf16x2<false>(ev), f8_to_bf16x2<true>(ev),
                     f8_to_bf16x2<false>(od), f8_to_bf16x2<true>(od)};
      } else {
        kf = (u32x4){f8_to_f16x2<false>(ev), f8_to_f16x2<true>(ev),
                     f8_to_f16x2<false>(od), f8_to_f16x2<true>(od)};
      }
      s[T] = mfma_qk<QDT>(kf, qf[c], s[T]);
    }
  }
  if (more) load_k<FMT>(P, tn, r, g, R);

  // ---- V fragments: element 8 r + i of tokens 4 j + g, j = 0..7 ---------------------
  uint32_t ev[8], od[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lookup8(R.vw[j], L.lut[1][R.vsb[j]], ev[j], od[j]);
  if (more) load_v<FMT>(P, tn, r, g, R);
  uint32_t te0[4], te1[4], to0[4], to1[4];
  transpose4(ev[0], ev[1], ev[2], ev[3], te0);
  transpose4(ev[4], ev[5], ev[6], ev[7], te1);
  transpose4(od[0], od[1], od[2], od[3], to0);
  transpose4(od[4], od[5], od[6], od[7], to1);

  // ---- online softmax, log2 domain: weight 2^(c2 s - m).  The running max m
  // moves only when the step's scores exceed it by more than kLazy, so the
  // weights stay below 2^kLazy (well inside fp16) and rescales are rare ------
  float sv[8];
  float mx = -__builtin_inff();
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = s[T][e];
      if (TAIL && t0 + 16 * T + 4 * e + g >= P.t_end) v = -__builtin_inff();
      sv[4 * T + e] = v;
      mx = fmaxf(mx, v);
    }
  mx = max_over_groups(mx) * c2;
  if (__any(mx > st.m + kLazy)) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.ol *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.o[i] *= alpha;
    st.m = m_new;
  }
  const float nm = -st.m;
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[j], c2, nm));
  const v8h pf = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                  (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};

  // ---- O += P V; the weights' sum on the matrix cores as well (ones x P) ------------
  const v8h ones = {1, 1, 1, 1, 1, 1, 1, 1};
  st.ol = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf, st.ol, 0, 0, 0);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const u32x4 fe = {f8_to_f16x2<false>(te0[a]), f8_to_f16x2<true>(te0[a]),
                      f8_to_f16x2<false>(te1[a]), f8_to_f16x2<true>(te1[a])};
    st.o[2 * a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, fe), pf, st.o[2 * a], 0, 0, 0);
    const u32x4 fo = {f8_to_f16x2<false>(to0[a]), f8_to_f16x2<true>(to0[a]),
                      f8_to_f16x2<false>(to1[a]), f8_to_f16x2<true>(to1[a])};
    st.o[2 * a + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, fo), pf, st.o[2 * a + 1], 0, 0, 0);
  }
}

// 4 waves per SIMD (16 per CU, 4 workgroups: the LDS of a CU holds 4): the
// register budget that leaves keeps the accumulators out of AGPRs.
template <int FMT, int QDT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attn_decode_kernel(AttnArgs A) {
  __shared__ AttnLds L;
  constexpr bool NV = FMT == kFmtNV;
  constexpr int kScaleBytes = NV ? kHeadDim / 16 : kHeadDim / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t b = bh / A.hkv;
  const int h = (int)(bh - b * A.hkv);

  // ---- FP8 table: thread tid owns scale byte tid --------------------------------
  {
    const v2f m01 = e2m1_unpack2<0>(0x76543210u), m23 = e2m1_unpack2<1>(0x76543210u);
    const v2f m45 = e2m1_unpack2<2>(0x76543210u), m67 = e2m1_unpack2<3>(0x76543210u);
    const float mag[8] = {m01.x, m01.y, m23.x, m23.y, m45.x, m45.y, m67.x, m67.y};
    const float sv = block_scale_value<NV>((uint32_t)tid);
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      float y[8];
      const float s_t = NV ? (kv ? *A.vts : *A.kts) : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = mag[i] * sv;     // exact
        y[i] = NV ? t * s_t : t;
      }
      L.lut[kv][tid] = (u32x2){pack_e4m3x4(y), pack_e4m3x4(y + 4)};
    }
  }

  // ---- this workgroup's tokens (offsets inside this (sequence, head)'s cache) --------
  int64_t len = A.seq_lens[b];
  if (len < 0) len = 0;
  if (len > A.t_max) len = A.t_max;
  const int64_t tb = (int64_t)split * A.chunk;
  const int t_begin = (int)(tb < len ? tb : len);
  const int t_end = (int)(tb + A.chunk < len ? tb + A.chunk : len);
  const int64_t row0 = bh * A.t_max;
  const uint8_t* kcb = A.kc + row0 * kRowBytes;
  const uint8_t* ksb_ = A.ks + row0 * kScaleBytes;
  const uint8_t* vcb = A.vc + row0 * kRowBytes;
  const uint8_t* vsb_ = A.vs + row0 * kScaleBytes;

  // ---- Q fragments: query head r (zero for r >= G), elements 32 g + 8 c + {0,2,4,6,1,3,5,7}
  u32x4 qf[4];
  {
    const bool live = r < A.g;
    const uint16_t* qrow = A.q + (b * A.hq + (int64_t)h * A.g + (live ? r : 0)) * kHeadDim + 32 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (live) w = *reinterpret_cast<const u32x4*>(qrow + 8 * c);
      qf[c] = (u32x4){perm(w.y, w.x, 0x05040100u), perm(w.w, w.z, 0x05040100u),
                      perm(w.y, w.x, 0x07060302u), perm(w.w, w.z, 0x07060302u)};
      if (A.scale_log2 < 0.0f) qf[c] ^= 0x80008000u;  // scale * (K . q) = |scale| * (K . -q), exact
    }
  }
  const float c2 = fabsf(A.scale_log2);
  __syncthreads();                                    // the table is complete

  AttnState st;
  st.m = -__builtin_inff();
  st.ol = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i) st.o[i] = (v4f){0.f, 0.f, 0.f, 0.f};
  // loop-invariant byte offsets of this lane's first K row (tile T adds 16 T
  // rows), first V row (word j adds 4 j rows) and their scale bytes
  const uint32_t koff = (uint32_t)(4 * (r & 3) + (r >> 2)) * kRowBytes + 16 * g;
  const uint32_t voff = (uint32_t)g * kRowBytes + 4 * r;
  const AttnPtrs P = {kcb, ksb_, vcb, vsb_, koff, voff, t_end};

  int t0 = t_begin + wave * kStep;
  StepRegs R;
  if (t0 < t_end) {
    load_k<FMT>(P, t0, r, g, R);
    load_v<FMT>(P, t0, r, g, R);
  }
  for (; t0 + kStep <= t_end; t0 += kWaves * kStep)
    attn_step<FMT, QDT, false>(L, P, qf, c2, t0, t0 + kWaves * kStep, r, g, R, st);
  if (t0 < t_end) attn_step<FMT, QDT, true>(L, P, qf, c2, t0, t_end, r, g, R, st);
  const float m = st.m;
  const float l = st.ol[0];                           // sum of the fp16 weights, all lane groups

  // ---- merge the 4 waves, write this split's partial ----------------------------------
  if (r < A.g) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) L.part[wave][r][32 * g + 8 * e + i] = st.o[i][e];
    if (g == 0) {
      L.pm[wave][r] = m;
      L.pl[wave][r] = l;
    }
  }
  __syncthreads();
  const int64_t pbase = (bh * A.nsplit + split) * A.g;
  for (int idx = tid; idx < A.g * kHeadDim; idx += kThreads) {
    const int qh = idx >> 7, d = idx & (kHeadDim - 1);
    float M = L.pm[0][qh];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, L.pm[w][qh]);
    float acc = 0.0f;
    if (M > -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) acc += L.part[w][qh][d] * __builtin_amdgcn_exp2f(L.pm[w][qh] - M);
    }
    A.part_o[(pbase + qh) * kHeadDim + d] = acc;
  }
  if (tid < A.g) {
    float M = L.pm[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, L.pm[w][tid]);
    float s = 0.0f;
    if (M > -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += L.pl[w][tid] * __builtin_amdgcn_exp2f(L.pm[w][tid] - M);
    }
    A.part_ml[(pbase + tid) * 2] = M;
    A.part_ml[(pbase + tid) * 2 + 1] = s;
  }
}

// One wave per (sequence, query head): merges the splits' partials; a
// sequence with no tokens gives zeros.  Lane l owns elements 2 l, 2 l + 1.
template <int OUT>
__global__ __launch_bounds__(64) void attn_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        int nsplit, int g, int hkv, int hq,
                                                        void* __restrict__ out) {
  const int64_t bq = blockIdx.x;                      // b * hq + query head
  const int64_t b = bq / hq;
  const int j = (int)(bq - b * hq);
  const int64_t bh = b * hkv + j / g;
  const int qh = j % g;
  const int lane = threadIdx.x;
  float M = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((bh * nsplit + s) * g + qh) * 2]);
  float o0 = 0.0f, o1 = 0.0f;
  if (M > -__builtin_inff()) {
    float sum = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const int64_t p = (bh * nsplit + s) * g + qh;
      const float w = __builtin_amdgcn_exp2f(part_ml[p * 2] - M);
      sum += part_ml[p * 2 + 1] * w;
      const v2f v = *reinterpret_cast<const v2f*>(part_o + p * kHeadDim + 2 * lane);
      o0 += v.x * w;
      o1 += v.y * w;
    }
    o0 = o0 / sum;
    o1 = o1 / sum;
  }
  const int64_t idx = bq * kHeadDim + 2 * lane;
  if (OUT == kInF32) {
    *reinterpret_cast<v2f*>(reinterpret_cast<float*>(out) + idx) = (v2f){o0, o1};
  } else {
    const v2bf v = {(__bf16)o0, (__bf16)o1};
    *reinterpret_cast<v2bf*>(reinterpret_cast<__bf16*>(out) + idx) = v;
  }
}

void split_plan(int64_t bh, int64_t t_max, int* nsplit, int64_t* chunk) {
  int64_t want = (kTargetWorkgroups + bh - 1) / bh;
  const int64_t most = (t_max + kMinChunk - 1) / kMinChunk;
  if (want > most) want = most;
  if (want < 1) want = 1;
  int64_t c = (t_max + want - 1) / want;
  c = (c + 127) / 128 * 128;
  *chunk = c;
  *nsplit = (int)((t_max + c - 1) / c);
}

}  // namespace

size_t attention_workspace_bytes(int64_t batch, int64_t q_heads, int64_t kv_heads, int64_t t_max) {
  int ns;
  int64_t chunk;
  const int64_t bh = batch * kv_heads;
  split_plan(bh, t_max, &ns, &chunk);
  return (size_t)(bh * ns * (q_heads / kv_heads)) * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_attention_decode(int fmt, const void* q, int q_dtype, int64_t batch,
                                   int64_t q_heads, int64_t kv_heads, const uint8_t* k_codes,
                                   const uint8_t* k_scales, const float* k_tscale,
                                   const uint8_t* v_codes, const uint8_t* v_scales,
                                   const float* v_tscale, int64_t t_max, const int32_t* seq_lens,
                                   float softmax_scale, void* out, int out_dtype, void* workspace,
                                   hipStream_t stream) {
  AttnArgs a;
  const int64_t bh = batch * kv_heads;
  int ns;
  int64_t chunk;
  split_plan(bh, t_max, &ns, &chunk);
  const int g = (int)(q_heads / kv_heads);
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.kc = k_codes;
  a.ks = k_scales;
  a.kts = k_tscale;
  a.vc = v_codes;
  a.vs = v_scales;
  a.vts = v_tscale;
  a.seq_lens = seq_lens;
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_ml = a.part_o + bh * ns * g * kHeadDim;
  a.t_max = t_max;
  a.chunk = chunk;
  a.hq = (int)q_heads;
  a.hkv = (int)kv_heads;
  a.g = g;
  a.nsplit = ns;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  const dim3 grid((unsigned)bh, (unsigned)ns);
  if (fmt == kFmtNV) {
    if (q_dtype == kInBF16) hipLaunchKernelGGL((attn_decode_kernel<kFmtNV, kInBF16>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((attn_decode_kernel<kFmtNV, kInF16>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (q_dtype == kInBF16) hipLaunchKernelGGL((attn_decode_kernel<kFmtMX, kInBF16>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((attn_decode_kernel<kFmtMX, kInF16>), grid, dim3(kThreads), 0, stream, a);
  }
  const dim3 mgrid((unsigned)(batch * q_heads));
  if (out_dtype == kInF32) {
    hipLaunchKernelGGL((attn_merge_kernel<kInF32>), mgrid, dim3(64), 0, stream, a.part_o, a.part_ml, ns, g,
                       (int)kv_heads, (int)q_heads, out);
  } else {
    hipLaunchKernelGGL((attn_merge_kernel<kInBF16>), mgrid, dim3(64), 0, stream, a.part_o, a.part_ml, ns, g,
                       (int)kv_heads, (int)q_heads, out);
  }
  return hipGetLastError();
}

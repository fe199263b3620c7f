// Chunked (WY / UT) evaluation of the gated delta rule for prefill, with the
// q/k L2 norm fused in front and the gated-RMSNorm epilogue fused behind.
//
// The "chunked" linear-attention operation of LightLLM #1097 "[model] Support
// Qwen3next" (Highlights, "Specialized Triton Kernels"), over the GDN layer of
// LightLLM PR #1184.  The math follows from unrolling the gated delta rule
// S_t = e^{g_t} S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T (row form, S in
// R^{d_v x d_k}) over a chunk of n tokens with incoming state S0 and inclusive
// cumulative log-decay G_i = g_1 + ... + g_i:
//   A_ij = b_i e^{G_i - G_j} (k_i . k_j)   for i > j, else 0
//   T    = (I + A)^{-1}                    (unit lower triangular)
//   W    = T diag(b e^G) K,   Ut = T diag(b) V        (independent of S0)
//   U    = Ut - W S0^T                     (the chunk's delta-rule updates u_i)
//   O    = diag(e^G) Q S0^T + (M o Q K^T) U,  M_ij = e^{G_i - G_j} for j <= i
//   S    = e^{G_n} S0 + U^T diag(e^{G_n - G}) K
// Every exponent is a non-positive difference and is masked before exp.
//
// MI355X design (v1: one workgroup per (sequence, V head) chain):
//  * The state is held transposed, S^T [d_k x d_v], in MFMA accumulators that
//    never leave registers between chunks: wave w owns d_v columns
//    [32w, 32w+32) and all d_k rows.  The accumulator tile layout (lane l holds
//    rows 4(l/16)+i of column l%16) is also a valid B operand of the
//    contraction over d_k, so W S0^T and Q S0^T take S^T straight from
//    registers; likewise U (tokens x d_v) feeds (M o QK^T) U and K^T U.
//  * The chunk's q, k (row-major and transposed) and v (transposed) are staged
//    once in LDS in the operand precision; the small C x C matrices (A and T
//    in fp32, P = M o QK^T, T diag(b e^G), T diag(b) in operand precision)
//    live in LDS too.  All contractions run on MFMA: bf16 16x16x32 (fp32
//    accumulate) in bf16 mode, fp32 16x16x4 in the all-fp32 mode.
//  * T: 16x16 diagonal blocks by forward substitution in registers, then
//    off-diagonal blocks by block forward substitution on fp32 MFMA.
#include <stdlib.h>
#include <string.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

// waves per workgroup: one per 32 d_v columns (at least one)
template <int D>
constexpr int kChunkThreads = (D >= 128 ? 4 : (D >= 64 ? 2 : 1)) * 64;

template <typename Op, int D, int C>
struct Cfg {
  static constexpr int NT = D / 16;  // 16-wide tiles along d
  static constexpr int CT = C / 16;  // 16-token tiles per chunk
  static constexpr int THREADS = kChunkThreads<D>;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int DVT = NT / WAVES;  // d_v tiles per wave
  static constexpr int LD_D = D + 4;      // row stride (elements) of [C][D] operand tiles
  static constexpr int LD_C = C + 4;      // row stride of [D][C] and [C][C] operand tiles
  static constexpr int LD_F = C + 4;      // row stride of fp32 [C][C] tiles
  static constexpr int LPR = D / 8;       // lanes per row when loading (8 elements each)
  // LDS carve-up (bytes; every piece a multiple of 16)
  static constexpr int Q_OFF = 0;
  static constexpr int K_OFF = Q_OFF + C * LD_D * (int)sizeof(Op);   // k^ row-major, later W
  static constexpr int KT_OFF = K_OFF + C * LD_D * (int)sizeof(Op);  // k^ transposed [D][C]
  static constexpr int VT_OFF = KT_OFF + D * LD_C * (int)sizeof(Op); // v transposed [D][C]
  static constexpr int A_OFF = VT_OFF + D * LD_C * (int)sizeof(Op);  // fp32 A
  static constexpr int T_OFF = A_OFF + C * LD_F * 4;                 // fp32 T
  static constexpr int TK_OFF = T_OFF + C * LD_F * 4;                // T diag(b e^G)
  static constexpr int TV_OFF = TK_OFF + C * LD_C * (int)sizeof(Op); // T diag(b)
  static constexpr int P_OFF = TV_OFF + C * LD_C * (int)sizeof(Op);  // M o QK^T
  static constexpr int G_OFF = P_OFF + C * LD_C * (int)sizeof(Op);   // G, e^G, beta
  static constexpr int RED_OFF = G_OFF + 3 * C * 4;                  // [WAVES][C] row sums
  static constexpr int BYTES = RED_OFF + WAVES * C * 4;
};

template <typename Op>
__device__ __forceinline__ typename Frag<Op>::type neg(typename Frag<Op>::type f) {
  typename Frag<Op>::type r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = -f[i];
  return r;
}

template <typename T, typename Op, int D, int C>
__global__ __launch_bounds__(kChunkThreads<D>) void chunk_prefill_kernel(
    const T* __restrict__ qkv, const float* __restrict__ g_in, const float* __restrict__ beta_in,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const uint8_t* __restrict__ has_init,
    float* __restrict__ state, int32_t n_slots, T* __restrict__ o, const T* __restrict__ z,
    const T* __restrict__ norm_w, float norm_eps, float scale, int64_t t_total, int32_t h_k, int32_t h_v) {
  using K = Cfg<Op, D, C>;
  using FragT = typename Frag<Op>::type;
  constexpr int NT = K::NT, CT = K::CT, WAVES = K::WAVES, DVT = K::DVT;
  constexpr int LD_D = K::LD_D, LD_C = K::LD_C, LD_F = K::LD_F, LPR = K::LPR;

  __shared__ __attribute__((aligned(16))) unsigned char smem[K::BYTES];
  Op* sQ = reinterpret_cast<Op*>(smem + K::Q_OFF);
  Op* sK = reinterpret_cast<Op*>(smem + K::K_OFF);
  Op* sKT = reinterpret_cast<Op*>(smem + K::KT_OFF);
  Op* sVT = reinterpret_cast<Op*>(smem + K::VT_OFF);
  float* sA = reinterpret_cast<float*>(smem + K::A_OFF);
  float* sT = reinterpret_cast<float*>(smem + K::T_OFF);
  Op* sTk = reinterpret_cast<Op*>(smem + K::TK_OFF);
  Op* sTv = reinterpret_cast<Op*>(smem + K::TV_OFF);
  Op* sP = reinterpret_cast<Op*>(smem + K::P_OFF);
  float* sG = reinterpret_cast<float*>(smem + K::G_OFF);
  float* sEG = sG + C;
  float* sB = sG + 2 * C;
  float* sRed = reinterpret_cast<float*>(smem + K::RED_OFF);

  const int n = blockIdx.x / h_v;
  const int h = blockIdx.x % h_v;
  const int hk = h / (h_v / h_k);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int c_ch = 2 * h_k * D + h_v * D;
  const int64_t o_ld = (int64_t)h_v * D;  // row stride of o and z

  const int64_t lo = min((int64_t)cu[n], t_total);
  const int64_t hi = min(max((int64_t)cu[n + 1], lo), t_total);
  const int32_t slot = slots[n];
  if (!slot_ok(slot, n_slots)) {  // padding entry: zero rows
    for (int64_t t = lo; t < hi; ++t)
      for (int r = tid; r < D; r += K::THREADS) o[t * o_ld + h * D + r] = from_f32<T>(0.0f);
    return;
  }
  const bool init = has_init == nullptr || has_init[n] != 0;
  float* st_ptr = state + ((int64_t)slot * h_v + h) * D * D;

  // S^T accumulators: Sacc[mt][j] = S^T tile (d_k tile mt, d_v tile wave*DVT+j)
  f32x4 Sacc[NT][DVT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int j = 0; j < DVT; ++j) {
      const int dv = 16 * (wave * DVT + j) + l16;
      if (init) {
        const float4 v = *reinterpret_cast<const float4*>(st_ptr + dv * D + 16 * mt + 4 * g4);
        Sacc[mt][j] = f32x4{v.x, v.y, v.z, v.w};
      } else {
        Sacc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

  // Each thread owns RPT rows of each of q, k, v (8 elements each) per chunk.
  // Their raw bits sit in registers: the next chunk's loads are issued as soon
  // as the current chunk is staged in LDS and land while it is computed.
  constexpr int RPP = K::THREADS / LPR;     // rows per pass of the workgroup
  constexpr int RPT = (C + RPP - 1) / RPP;  // rows per thread per kind
  const int e0 = (tid % LPR) * 8;
  const int r0 = tid / LPR;
  const int64_t cols[3] = {(int64_t)hk * D, (int64_t)(h_k + hk) * D, (int64_t)(2 * h_k + h) * D};
  Raw8<T> pre[3][RPT];
  float pre_g = 0.f, pre_b = 0.f;
  // (a macro rather than a lambda: a captured array would be moved to LDS)
#define GDN_ISSUE_CHUNK_LOADS(cs)                                                         \
  {                                                                                       \
    const int nv_ = (int)min((int64_t)C, hi - (cs));                                      \
    _Pragma("unroll") for (int kind = 0; kind < 3; ++kind)                                \
    _Pragma("unroll") for (int j = 0; j < RPT; ++j) {                                     \
      const int r = r0 + j * RPP;                                                         \
      if (r < nv_) pre[kind][j].load(qkv + ((cs) + r) * c_ch + cols[kind] + e0);          \
      else pre[kind][j].zero();                                                           \
    }                                                                                     \
    if (wave == 0) {                                                                      \
      pre_g = lane < nv_ ? g_in[((cs) + lane) * h_v + h] : 0.f;                           \
      pre_b = lane < nv_ ? beta_in[((cs) + lane) * h_v + h] : 0.f;                        \
    }                                                                                     \
  }
  if (lo < hi) GDN_ISSUE_CHUNK_LOADS(lo);
  Raw8<T> zpre[RPT];
  float nw[DVT];
#pragma unroll
  for (int j = 0; j < DVT; ++j) nw[j] = z ? to_f32(norm_w[16 * (wave * DVT + j) + l16]) : 1.f;

  for (int64_t c0 = lo; c0 < hi; c0 += C) {
    const int nvalid = (int)min((int64_t)C, hi - c0);

    // ---------------- phase 1: stage q^, k^ (normalised) and v; cumulative gates
    {
#pragma unroll
      for (int kind = 0; kind < 3; ++kind)
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          const int r = r0 + j * RPP;
          float v[8];
          pre[kind][j].to_f32(v);
          if (kind < 2) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
            ss = group_sum<LPR>(ss);
            const float rn = fast_rsq(ss + 1e-6f);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= rn;
          }
          if (r < C) {
            if (kind == 0) {
              *reinterpret_cast<FragT*>(sQ + r * LD_D + e0) = FragT{from_f32<Op>(v[0]), from_f32<Op>(v[1]), from_f32<Op>(v[2]), from_f32<Op>(v[3])};
              *reinterpret_cast<FragT*>(sQ + r * LD_D + e0 + 4) = FragT{from_f32<Op>(v[4]), from_f32<Op>(v[5]), from_f32<Op>(v[6]), from_f32<Op>(v[7])};
            } else if (kind == 1) {
              *reinterpret_cast<FragT*>(sK + r * LD_D + e0) = FragT{from_f32<Op>(v[0]), from_f32<Op>(v[1]), from_f32<Op>(v[2]), from_f32<Op>(v[3])};
              *reinterpret_cast<FragT*>(sK + r * LD_D + e0 + 4) = FragT{from_f32<Op>(v[4]), from_f32<Op>(v[5]), from_f32<Op>(v[6]), from_f32<Op>(v[7])};
#pragma unroll
              for (int e = 0; e < 8; ++e) sKT[(e0 + e) * LD_C + r] = from_f32<Op>(v[e]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) sVT[(e0 + e) * LD_C + r] = from_f32<Op>(v[e]);
            }
          }
        }
      if (wave == 0) {
        // inclusive scan of g over the chunk (padded tokens: g = 0, beta = 0)
        float gv = pre_g;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float up = __shfl_up(gv, off);
          if (lane >= off) gv += up;
        }
        if (lane < C) {
          sG[lane] = gv;
          sEG[lane] = fast_exp(gv);
          sB[lane] = pre_b;
        }
      }
      if (c0 + C < hi) GDN_ISSUE_CHUNK_LOADS(c0 + C);  // next chunk's loads overlap this chunk's compute
      if (z) {  // this chunk's gate rows, consumed by the epilogue
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          const int r = r0 + j * RPP;
          if (r < nvalid) zpre[j].load(z + (c0 + r) * o_ld + h * D + e0);
          else zpre[j].zero();
        }
      }
    }
    __syncthreads();

    // ---------------- phase 2: Gram tiles -> A (fp32, strict lower) and P (lower incl. diagonal)
    {
      constexpr int NLT = CT * (CT + 1) / 2;  // lower-triangular tiles per matrix
      constexpr int PER_WAVE = (2 * NLT + WAVES - 1) / WAVES;
#pragma unroll
      for (int k = 0; k < PER_WAVE; ++k) {
        const int q = wave + k * WAVES;
        if (q < 2 * NLT) {
          const bool is_p = q >= NLT;
          const int idx = is_p ? q - NLT : q;
          int ti = 0;
          while ((ti + 1) * (ti + 2) / 2 <= idx) ++ti;
          const int tj = idx - ti * (ti + 1) / 2;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const Op* arow = (is_p ? sQ : sK) + (16 * ti + l16) * LD_D;
          const Op* brow = sK + (16 * tj + l16) * LD_D;
          int kb = 0;
#pragma unroll
          for (; kb + 1 < NT; kb += 2)
            mma_k32(acc, lds_frag<Op>(arow + 16 * kb + 4 * g4), lds_frag<Op>(arow + 16 * kb + 16 + 4 * g4),
                    lds_frag<Op>(brow + 16 * kb + 4 * g4), lds_frag<Op>(brow + 16 * kb + 16 + 4 * g4));
          if (kb < NT) mma_k16(acc, lds_frag<Op>(arow + 16 * kb + 4 * g4), lds_frag<Op>(brow + 16 * kb + 4 * g4));
          const int cc = 16 * tj + l16;
          const float gc = sG[cc];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * ti + 4 * g4 + i;
            const float dec = fast_exp(fminf(sG[r] - gc, 0.f));
            if (is_p) sP[r * LD_C + cc] = from_f32<Op>(r >= cc ? dec * acc[i] : 0.f);
            else sA[r * LD_F + cc] = r > cc ? sB[r] * dec * acc[i] : 0.f;
          }
        }
      }
      // upper blocks: A and P are zero there, and so is T
      for (int e = tid; e < C * C; e += K::THREADS) {
        const int r = e / C, cc = e % C;
        if ((r >> 4) < (cc >> 4)) {
          sA[r * LD_F + cc] = 0.f;
          sT[r * LD_F + cc] = 0.f;
          sP[r * LD_C + cc] = from_f32<Op>(0.f);
        }
      }
    }
    __syncthreads();

    // ---------------- phase 3: T = (I + A)^-1
    // (a) diagonal 16x16 blocks: forward substitution, one lane per column
    if (tid < CT * 16) {
      const int b = tid >> 4, c = tid & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* arow = sA + (16 * b + r) * LD_F + 16 * b;
        float acc = r == c ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < r; ++j) acc = fmaf(-arow[j], x[j], acc);
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(16 * b + r) * LD_F + 16 * b + c] = x[r];
    }
    __syncthreads();
    // (b) off-diagonal blocks, block row by block row: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
#pragma unroll
    for (int bi = 1; bi < CT; ++bi) {
      for (int bj = wave; bj < bi; bj += WAVES) {
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
        for (int bk = bj; bk < bi; ++bk) {
          const f32x4 a = lds_frag<float>(sA + (16 * bi + l16) * LD_F + 16 * bk + 4 * g4);
          f32x4 b;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) b[jj] = sT[(16 * bk + 4 * g4 + jj) * LD_F + 16 * bj + l16];
          mma_k16(X, a, b);
        }
        f32x4 Y = {0.f, 0.f, 0.f, 0.f};
        mma_k16(Y, lds_frag<float>(sT + (16 * bi + l16) * LD_F + 16 * bi + 4 * g4), X);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sT[(16 * bi + 4 * g4 + jj) * LD_F + 16 * bj + l16] = -Y[jj];
      }
      __syncthreads();
    }
    // (c) column-scaled copies in operand precision: Tk = T diag(b e^G), Tv = T diag(b)
    for (int e = tid; e < C * C; e += K::THREADS) {
      const int r = e / C, cc = e % C;
      const float t = sT[r * LD_F + cc];
      sTk[r * LD_C + cc] = from_f32<Op>(t * sB[cc] * sEG[cc]);
      sTv[r * LD_C + cc] = from_f32<Op>(t * sB[cc]);
    }
    __syncthreads();

    // ---------------- phase 4: W = Tk K -> LDS (over k^'s slot), Ut = Tv V -> registers
    for (int q = wave; q < CT * NT; q += WAVES) {
      const int mt = q / NT, nt = q % NT;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const Op* arow = sTk + (16 * mt + l16) * LD_C;
      const Op* brow = sKT + (16 * nt + l16) * LD_C;
      int kb = 0;
      for (; kb + 1 <= mt; kb += 2)  // T is lower triangular: k blocks beyond mt are zero
        mma_k32(acc, lds_frag<Op>(arow + 16 * kb + 4 * g4), lds_frag<Op>(arow + 16 * kb + 16 + 4 * g4),
                lds_frag<Op>(brow + 16 * kb + 4 * g4), lds_frag<Op>(brow + 16 * kb + 16 + 4 * g4));
      if (kb <= mt) mma_k16(acc, lds_frag<Op>(arow + 16 * kb + 4 * g4), lds_frag<Op>(brow + 16 * kb + 4 * g4));
#pragma unroll
      for (int i = 0; i < 4; ++i) sK[(16 * mt + 4 * g4 + i) * LD_D + 16 * nt + l16] = from_f32<Op>(acc[i]);
    }
    f32x4 Uacc[CT][DVT];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int j = 0; j < DVT; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const Op* arow = sTv + (16 * mt + l16) * LD_C;
        const Op* brow = sVT + (16 * (wave * DVT + j) + l16) * LD_C;
        int kb = 0;
#pragma unroll
        for (; kb + 1 <= mt; kb += 2)
          mma_k32(acc, lds_frag<Op>(arow + 16 * kb + 4 * g4), lds_frag<Op>(arow + 16 * kb + 16 + 4 * g4),
                  lds_frag<Op>(brow + 16 * kb + 4 * g4), lds_frag<Op>(brow + 16 * kb + 16 + 4 * g4));
        if (kb <= mt) mma_k16(acc, lds_frag<Op>(arow + 16 * kb + 4 * g4), lds_frag<Op>(brow + 16 * kb + 4 * g4));
        Uacc[mt][j] = acc;
      }
    __syncthreads();

    // ---------------- phase 5: the state contractions
    // S^T as B operand of the contraction over d_k (old state, before update)
    FragT Sf[NT][DVT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < DVT; ++j) Sf[mt][j] = frag_from<Op>(Sacc[mt][j]);

    f32x4 Oacc[CT][DVT];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt) {
      const Op* wrow = sK + (16 * mt + l16) * LD_D;  // W
      const Op* qrow = sQ + (16 * mt + l16) * LD_D;
#pragma unroll
      for (int j = 0; j < DVT; ++j) {
        f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
        int kb = 0;
#pragma unroll
        for (; kb + 1 < NT; kb += 2) {
          // U = Ut - W S^T ;  O = Q S^T
          mma_k32(Uacc[mt][j], neg<Op>(lds_frag<Op>(wrow + 16 * kb + 4 * g4)),
                  neg<Op>(lds_frag<Op>(wrow + 16 * kb + 16 + 4 * g4)), Sf[kb][j], Sf[kb + 1][j]);
          mma_k32(oacc, lds_frag<Op>(qrow + 16 * kb + 4 * g4), lds_frag<Op>(qrow + 16 * kb + 16 + 4 * g4), Sf[kb][j],
                  Sf[kb + 1][j]);
        }
        if (kb < NT) {
          mma_k16(Uacc[mt][j], neg<Op>(lds_frag<Op>(wrow + 16 * kb + 4 * g4)), Sf[kb][j]);
          mma_k16(oacc, lds_frag<Op>(qrow + 16 * kb + 4 * g4), Sf[kb][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[i] *= sEG[16 * mt + 4 * g4 + i];
        Oacc[mt][j] = oacc;
      }
    }
    // O += (M o QK^T) U  (P lower triangular by token tiles)
    {
      FragT Uf[CT][DVT];
#pragma unroll
      for (int kt = 0; kt < CT; ++kt)
#pragma unroll
        for (int j = 0; j < DVT; ++j) Uf[kt][j] = frag_from<Op>(Uacc[kt][j]);
#pragma unroll
      for (int mt = 0; mt < CT; ++mt) {
        const Op* prow = sP + (16 * mt + l16) * LD_C;
#pragma unroll
        for (int j = 0; j < DVT; ++j) {
          int kb = 0;
#pragma unroll
          for (; kb + 1 <= mt; kb += 2)
            mma_k32(Oacc[mt][j], lds_frag<Op>(prow + 16 * kb + 4 * g4), lds_frag<Op>(prow + 16 * kb + 16 + 4 * g4),
                    Uf[kb][j], Uf[kb + 1][j]);
          if (kb <= mt) mma_k16(Oacc[mt][j], lds_frag<Op>(prow + 16 * kb + 4 * g4), Uf[kb][j]);
        }
      }
    }
    // S^T <- e^{G_n} S^T + K^T diag(e^{G_n - G}) U
    {
      const float g_last = sG[C - 1];
      const float eg_last = fast_exp(g_last);
      FragT Uf[CT][DVT];
#pragma unroll
      for (int kt = 0; kt < CT; ++kt) {
        f32x4 d;
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = fast_exp(g_last - sG[16 * kt + 4 * g4 + i]);
#pragma unroll
        for (int j = 0; j < DVT; ++j) {
          f32x4 u = Uacc[kt][j];
#pragma unroll
          for (int i = 0; i < 4; ++i) u[i] *= d[i];
          Uf[kt][j] = frag_from<Op>(u);
        }
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const Op* krow = sKT + (16 * mt + l16) * LD_C;
#pragma unroll
        for (int j = 0; j < DVT; ++j) {
          f32x4 acc = Sacc[mt][j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] *= eg_last;
          int kb = 0;
#pragma unroll
          for (; kb + 1 < CT; kb += 2)
            mma_k32(acc, lds_frag<Op>(krow + 16 * kb + 4 * g4), lds_frag<Op>(krow + 16 * kb + 16 + 4 * g4),
                    Uf[kb][j], Uf[kb + 1][j]);
          if (kb < CT) mma_k16(acc, lds_frag<Op>(krow + 16 * kb + 4 * g4), Uf[kb][j]);
          Sacc[mt][j] = acc;
        }
      }
    }

    // ---------------- phase 6: epilogue (scale, optional gated RMSNorm) and store
    // The output tile is staged in LDS (over the v / A tiles, dead by now) so that
    // z is read and o written as whole 16-byte row pieces.
    {
      T* sZ = reinterpret_cast<T*>(smem + K::VT_OFF);
      if (z) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          const int r = r0 + j * RPP;
          if (r < C) {
            float v[8];
            zpre[j].to_f32(v);
            store8(sZ + r * LD_D + e0, v);
          }
        }
#pragma unroll
        for (int mt = 0; mt < CT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < DVT; ++j) ss = fmaf(Oacc[mt][j][i], Oacc[mt][j][i], ss);
            ss = group_sum<16>(ss);
            if (l16 == 0) sRed[wave * C + 16 * mt + 4 * g4 + i] = ss;
          }
      }
      __syncthreads();
      if (z) {
        float f[CT][4];
        float zz[CT][DVT][4];
#pragma unroll
        for (int mt = 0; mt < CT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * mt + 4 * g4 + i;
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) tot += sRed[w * C + t];
            f[mt][i] = scale * fast_rsq(tot * scale * scale * (1.0f / D) + norm_eps);
#pragma unroll
            for (int j = 0; j < DVT; ++j) zz[mt][j][i] = to_f32(sZ[t * LD_D + 16 * (wave * DVT + j) + l16]);
          }
#pragma unroll
        for (int mt = 0; mt < CT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < DVT; ++j)
              sZ[(16 * mt + 4 * g4 + i) * LD_D + 16 * (wave * DVT + j) + l16] =
                  from_f32<T>(Oacc[mt][j][i] * f[mt][i] * nw[j] * fast_silu(zz[mt][j][i]));
      } else {
#pragma unroll
        for (int mt = 0; mt < CT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < DVT; ++j)
              sZ[(16 * mt + 4 * g4 + i) * LD_D + 16 * (wave * DVT + j) + l16] = from_f32<T>(Oacc[mt][j][i] * scale);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int r = r0 + j * RPP;
        if (r < nvalid) {
          float v[8];
          load8(sZ + r * LD_D + e0, v);
          store8(o + (c0 + r) * o_ld + h * D + e0, v);
        }
      }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }

#undef GDN_ISSUE_CHUNK_LOADS
  // final state back to the slot
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int j = 0; j < DVT; ++j) {
      const int dv = 16 * (wave * DVT + j) + l16;
      *reinterpret_cast<float4*>(st_ptr + dv * D + 16 * mt + 4 * g4) =
          make_float4(Sacc[mt][j][0], Sacc[mt][j][1], Sacc[mt][j][2], Sacc[mt][j][3]);
    }
}

template <typename T, typename Op, int D, int C>
hipError_t impl(const ChunkArgs& a, hipStream_t st) {
  using K = Cfg<Op, D, C>;
  static_assert(K::BYTES <= 160 * 1024, "LDS budget");
  static_assert(C * K::LD_D * (int)sizeof(T) <= K::T_OFF - K::VT_OFF, "output tile fits over the v and A tiles");
  if (a.n_seq == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_prefill_kernel<T, Op, D, C>), dim3((unsigned)((int64_t)a.n_seq * a.s.h_v)),
                     dim3(K::THREADS), 0, st, (const T*)a.qkv, a.g, a.beta, a.cu_seqlens, a.slots, a.has_init,
                     a.state, a.n_slots, (T*)a.o, (const T*)a.z, (const T*)a.norm_w, a.norm_eps, a.scale,
                     a.t_total, a.s.h_k, a.s.h_v);
  return hipGetLastError();
}

template <typename T, typename Op, int D>
hipError_t by_chunk(const ChunkArgs& a, hipStream_t st) {
  switch (a.chunk) {
    case 16: return impl<T, Op, D, 16>(a, st);
    case 32: return impl<T, Op, D, 32>(a, st);
    case 64:
      if constexpr (sizeof(Op) == 2 || D <= 64) return impl<T, Op, D, 64>(a, st);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool chunk_supported(int d, int chunk, bool bf16) {
  if (d != 16 && d != 32 && d != 64 && d != 128) return false;
  if (chunk != 16 && chunk != 32 && chunk != 64) return false;
  if (!bf16 && d == 128 && chunk == 64) return false;  // exceeds LDS in fp32
  return true;
}

namespace {
// Which evaluation runs: GDN_PREFILL_PATH=fused|split (read once), default split.
bool use_split() {
  static const int mode = [] {
    const char* e = getenv("GDN_PREFILL_PATH");
    return (e && strcmp(e, "fused") == 0) ? 0 : 1;
  }();
  return mode == 1;
}
}  // namespace

size_t chunk_workspace_size(const Shape& s, bool bf16, int32_t n_seq, int64_t t_total, int32_t chunk) {
  return use_split() ? chunk_split_workspace_size(s, bf16, n_seq, t_total, chunk) : 0;
}

hipError_t launch_chunk_prefill(const ChunkArgs& a, hipStream_t st) {
  return use_split() ? launch_chunk_split(a, st) : launch_chunk_fused(a, st);
}

hipError_t launch_chunk_fused(const ChunkArgs& a, hipStream_t st) {
  switch (a.s.d) {
    case 16: return a.bf16 ? by_chunk<bf16, bf16, 16>(a, st) : by_chunk<float, float, 16>(a, st);
    case 32: return a.bf16 ? by_chunk<bf16, bf16, 32>(a, st) : by_chunk<float, float, 32>(a, st);
    case 64: return a.bf16 ? by_chunk<bf16, bf16, 64>(a, st) : by_chunk<float, float, 64>(a, st);
    case 128: return a.bf16 ? by_chunk<bf16, bf16, 128>(a, st) : by_chunk<float, float, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

// Chunked gated delta rule, split into a chunk-parallel preparation pass and
// a state pass that runs per (sequence, V head, 16-column d_v tile).  Same math
// as chunk_prefill.hip (the chunked WY / UT form of the gated delta rule):
//   A = strict-lower(b_i e^{G_i-G_j} k_i.k_j),  T = (I + A)^{-1},
//   W = T diag(b e^G) K,  Ut = T diag(b) V,  P = M o Q K^T        (no state)
//   U = Ut - W S0^T,  O = diag(e^G) Q S0^T + P U,
//   S = e^{G_n} S0 + K^T diag(e^{G_n - G}) U                       (the chain)
//
// Why this shape on MI355X: the first line depends only on the chunk's own
// tokens, so it runs as one workgroup per (chunk, V head) across the GPU.  In
// the chain, the rows of S (the d_v index) never mix: every contraction runs
// over d_k or over tokens.  So one wave owns a 16-wide slice of d_v for all of
// d_k, holding its S^T slice in MFMA accumulators, and a single 4096-token
// sequence with 32 V heads already gives 256 independent waves, one per CU,
// with no LDS and no barrier in the loop.  The prep pass writes every operand
// the chain reads as ready-made MFMA fragments:
//   -W and Q' = scale diag(e^G) Q (A operands, contraction over d_k)
//   K'^T = (diag(e^{G_n-G}) K)^T   (A operand, contraction over the chunk)
//   scale P                        (A operand, lower triangle)
//   Ut                            (accumulator layout)
// so each wave streams them with 16-byte loads one chunk ahead.  The gated
// RMSNorm needs the whole d_v row, which is spread over the waves of a head:
// the chain writes scale * O and a small row-wise pass finishes the norm in
// place.
//
//   chunk_index_kernel  first global chunk of every sequence (block scan)
//   chunk_prep_kernel   per (chunk, V head): q/k L2 norm, gates, Gram, T and
//                       the operand fragments above
//   chunk_state_kernel  per (sequence, V head, d_v tile): the chunk loop
//   gated_norm_kernel   per (token, V head): RMSNorm over d_v times w silu(z)
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace split {

template <int D>
constexpr int kThreads = (D >= 128 ? 4 : (D >= 64 ? 2 : 1)) * 64;

template <typename Op, int D, int C>
struct Cfg {
  static constexpr int NT = D / 16;
  static constexpr int CT = C / 16;
  static constexpr int THREADS = kThreads<D>;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int DVT = NT / WAVES;
  static constexpr int LD_D = D + 4;   // row stride of [C][D] operand tiles (elements)
  static constexpr int LD_C = C + 4;   // row stride of [C][C] operand tiles
  static constexpr int LD_F = C + 4;   // row stride of the fp32 A / T tile
  static constexpr int LPR = D / 8;    // lanes per row piece of 8 elements
  static constexpr int RPP = THREADS / LPR;
  static constexpr int RPT = (C + RPP - 1) / RPP;
  // Pair fragments: an A operand tile of 16 rows and a 32-wide step of the
  // contraction, 8 values per lane (two 16-blocks, 4 each), zero past the end.
  static constexpr int NPD = (NT + 1) / 2;  // 32-steps over d_k
  static constexpr int NPC = (CT + 1) / 2;  // 32-steps over the chunk
  static constexpr int PAIR = 64 * 8;       // elements per pair tile
  // workspace unit per (chunk, V head), bytes
  static constexpr int W_OFF = 0;                                   // -W     [CT][NPD] pairs
  static constexpr int Q_OFF = W_OFF + CT * NPD * PAIR * (int)sizeof(Op);   // Q'  [CT][NPD]
  static constexpr int KT_OFF = Q_OFF + CT * NPD * PAIR * (int)sizeof(Op);  // K'^T [NT][NPC]
  static constexpr int P_OFF = KT_OFF + NT * NPC * PAIR * (int)sizeof(Op);  // P   [CT][NPC]
  static constexpr int UT_OFF = P_OFF + CT * NPC * PAIR * (int)sizeof(Op);  // Ut  [CT][NT][64][4]
  static constexpr int F_OFF = UT_OFF + C * D * (int)sizeof(Op);            // e^{G_n}
  static constexpr int UNIT = (F_OFF + 16 + 255) / 256 * 256;
  // prep kernel LDS
  static constexpr int PQ = 0;                                     // q^ rows, later W
  static constexpr int PK = PQ + C * LD_D * (int)sizeof(Op);       // k^ rows
  static constexpr int PV = PK + C * LD_D * (int)sizeof(Op);       // v rows
  static constexpr int PA = PV + C * LD_D * (int)sizeof(Op);       // fp32 A, then T in place
  static constexpr int PP = PA + C * LD_F * 4;                     // P
  static constexpr int PG = PP + C * LD_C * (int)sizeof(Op);       // G, beta, beta e^G
  static constexpr int PREP_BYTES = PG + 3 * C * 4;
};

__device__ __forceinline__ int32_t seq_of_chunk(const int32_t* __restrict__ cstart, int32_t n_seq, int32_t gc) {
  int32_t lo = 0, hi = n_seq - 1;  // largest i with cstart[i] <= gc
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (cstart[mid] <= gc) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// cstart[i] = sum over j < i of ceil(len_j / C), for i = 0..n_seq.  One block.
__global__ __launch_bounds__(1024) void chunk_index_kernel(const int32_t* __restrict__ cu, int32_t n_seq,
                                                           int64_t t_total, int32_t chunk,
                                                           int32_t* __restrict__ cstart) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (n_seq + 1023) / 1024;
  const int i0 = min(tid * per, n_seq), i1 = min(i0 + per, n_seq);
  int32_t s = 0;
  for (int i = i0; i < i1; ++i) {
    const int64_t lo = min((int64_t)cu[i], t_total);
    const int64_t hi = min(max((int64_t)cu[i + 1], lo), t_total);
    s += (int32_t)((hi - lo + chunk - 1) / chunk);
  }
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = tid == 0 ? 0 : part[tid - 1];
  for (int i = i0; i < i1; ++i) {
    cstart[i] = run;
    const int64_t lo = min((int64_t)cu[i], t_total);
    const int64_t hi = min(max((int64_t)cu[i + 1], lo), t_total);
    run += (int32_t)((hi - lo + chunk - 1) / chunk);
  }
  if (tid == 1023) cstart[n_seq] = part[1023];
}

template <typename Op>
__device__ __forceinline__ typename Frag<Op>::type frag_scaled(const float* p, const float* s) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  typename Frag<Op>::type r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = from_f32<Op>(v[i] * s[i]);
  return r;
}
// 4 values down a column of a row-major tile (contraction index = row).
template <typename Op>
__device__ __forceinline__ typename Frag<Op>::type frag_col(const Op* p, int ld) {
  typename Frag<Op>::type r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = p[i * ld];
  return r;
}

template <typename Op>
__device__ __forceinline__ typename Frag<Op>::type zero_frag() {
  typename Frag<Op>::type r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = from_f32<Op>(0.f);
  return r;
}
template <typename Op>
__device__ __forceinline__ typename Frag<Op>::type frag_mul(const typename Frag<Op>::type& a, float f) {
  typename Frag<Op>::type r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = from_f32<Op>(to_f32(a[i]) * f);
  return r;
}
template <typename Op>
__device__ __forceinline__ void store_pair(Op* dst, const typename Frag<Op>::type& lo,
                                           const typename Frag<Op>::type& hi);
template <>
__device__ __forceinline__ void store_pair<bf16>(bf16* dst, const bf16x4& lo, const bf16x4& hi) {
  *reinterpret_cast<bf16x8*>(dst) = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <>
__device__ __forceinline__ void store_pair<float>(float* dst, const f32x4& lo, const f32x4& hi) {
  reinterpret_cast<f32x4*>(dst)[0] = lo;
  reinterpret_cast<f32x4*>(dst)[1] = hi;
}

// A pair fragment in registers: one 16x16x32 bf16 MFMA, or two 16-blocks of
// 16x16x4 fp32 MFMAs.  B is the two matching 16-blocks in accumulator layout.
template <typename Op> struct Pair;
template <> struct Pair<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ void mma(f32x4& acc, const bf16x4& b0, const bf16x4& b1) const {
    const bf16x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, b, acc, 0, 0, 0);
  }
};
template <> struct Pair<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = reinterpret_cast<const f32x4*>(p)[0];
    hi = reinterpret_cast<const f32x4*>(p)[1];
  }
  __device__ __forceinline__ void mma(f32x4& acc, const f32x4& b0, const f32x4& b1) const {
    mma_k32(acc, lo, hi, b0, b1);
  }
};

// ------------------------------------------------------------------ prep
template <typename T, typename Op, int D, int C>
__global__ __launch_bounds__(kThreads<D>) void chunk_prep_kernel(
    const T* __restrict__ qkv, const float* __restrict__ g_in, const float* __restrict__ beta_in,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const int32_t* __restrict__ cstart,
    int32_t n_slots, int32_t n_seq, int64_t t_total, int32_t h_k, int32_t h_v, float scale,
    unsigned char* __restrict__ ws) {
  using K = Cfg<Op, D, C>;
  using FragT = typename Frag<Op>::type;
  constexpr int NT = K::NT, CT = K::CT, WAVES = K::WAVES, LPR = K::LPR, RPP = K::RPP, RPT = K::RPT;
  constexpr int LD_D = K::LD_D, LD_C = K::LD_C, LD_F = K::LD_F;
  __shared__ __attribute__((aligned(16))) unsigned char smem[K::PREP_BYTES];
  Op* sQ = reinterpret_cast<Op*>(smem + K::PQ);
  Op* sK = reinterpret_cast<Op*>(smem + K::PK);
  Op* sV = reinterpret_cast<Op*>(smem + K::PV);
  float* sAT = reinterpret_cast<float*>(smem + K::PA);
  Op* sP = reinterpret_cast<Op*>(smem + K::PP);
  float* sG = reinterpret_cast<float*>(smem + K::PG);
  float* sB = sG + C;
  float* sBE = sG + 2 * C;

  const int gc = blockIdx.x / h_v;
  const int h = blockIdx.x % h_v;
  if (gc >= cstart[n_seq]) return;
  const int n = seq_of_chunk(cstart, n_seq, gc);
  if (!slot_ok(slots[n], n_slots)) return;  // padding entry: nothing to prepare
  const int hk = h / (h_v / h_k);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int c_ch = 2 * h_k * D + h_v * D;
  const int64_t seq_lo = min((int64_t)cu[n], t_total);
  const int64_t seq_hi = min(max((int64_t)cu[n + 1], seq_lo), t_total);
  const int64_t c0 = seq_lo + (int64_t)(gc - cstart[n]) * C;
  const int nvalid = (int)min((int64_t)C, seq_hi - c0);
  unsigned char* unit = ws + ((int64_t)gc * h_v + h) * K::UNIT;

  // ---- stage q^, k^ (normalised) and v row-major; gates
  {
    const int e0 = (tid % LPR) * 8, r0 = tid / LPR;
    const int64_t cols[3] = {(int64_t)hk * D, (int64_t)(h_k + hk) * D, (int64_t)(2 * h_k + h) * D};
    Raw8<T> raw[3][RPT];
#pragma unroll
    for (int kind = 0; kind < 3; ++kind)
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int r = r0 + j * RPP;
        if (r < nvalid) raw[kind][j].load(qkv + (c0 + r) * c_ch + cols[kind] + e0);
        else raw[kind][j].zero();
      }
    float gv = 0.f, bv = 0.f;
    if (wave == 0 && lane < nvalid) {
      gv = g_in[(c0 + lane) * h_v + h];
      bv = beta_in[(c0 + lane) * h_v + h];
    }
#pragma unroll
    for (int kind = 0; kind < 3; ++kind)
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int r = r0 + j * RPP;
        float v[8];
        raw[kind][j].to_f32(v);
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
          Op* dst = (kind == 0 ? sQ : (kind == 1 ? sK : sV)) + r * LD_D + e0;
          *reinterpret_cast<FragT*>(dst) = FragT{from_f32<Op>(v[0]), from_f32<Op>(v[1]), from_f32<Op>(v[2]), from_f32<Op>(v[3])};
          *reinterpret_cast<FragT*>(dst + 4) = FragT{from_f32<Op>(v[4]), from_f32<Op>(v[5]), from_f32<Op>(v[6]), from_f32<Op>(v[7])};
        }
      }
    if (wave == 0) {
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float up = __shfl_up(gv, off);
        if (lane >= off) gv += up;
      }
      if (lane < C) {
        sG[lane] = gv;
        sB[lane] = bv;
        sBE[lane] = bv * fast_exp(gv);
      }
      if (lane == C - 1) reinterpret_cast<float*>(unit + K::F_OFF)[0] = fast_exp(gv);
    }
  }
  __syncthreads();

  // ---- Gram tiles (lower triangle): K K^T -> A (fp32), Q K^T -> P
  {
    constexpr int NLT = CT * (CT + 1) / 2;
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
        const float gc_ = sG[cc];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ti + 4 * g4 + i;
          const float dec = fast_exp(fminf(sG[r] - gc_, 0.f));
          if (is_p) sP[r * LD_C + cc] = from_f32<Op>(r >= cc ? dec * acc[i] : 0.f);
          else sAT[r * LD_F + cc] = r > cc ? sB[r] * dec * acc[i] : 0.f;
        }
      }
    }
    for (int e = tid; e < C * C; e += K::THREADS) {  // upper blocks
      const int r = e / C, cc = e % C;
      if ((r >> 4) < (cc >> 4)) {
        sAT[r * LD_F + cc] = 0.f;
        sP[r * LD_C + cc] = from_f32<Op>(0.f);
      }
    }
  }
  __syncthreads();

  // ---- Q' = scale diag(e^G) Q^, K'^T = (diag(e^{G_n - G}) K^)^T and scale P as pair fragments.
  // sQ, sK, sP and sG stay unchanged until the W phase, behind later barriers.
  {
    constexpr int NPD = K::NPD, NPC = K::NPC, NQ = CT * NPD, NK = NT * NPC, NP = CT * NPC;
    const float g_n = sG[C - 1];
    for (int q = wave; q < NQ + NK + NP; q += WAVES) {
      FragT lo, hi;
      Op* dst;
      if (q < NQ) {
        const int mt = q / NPD, sp = q % NPD, r = 16 * mt + l16;
        const float f = scale * fast_exp(sG[r]);
        const Op* src = sQ + r * LD_D + 32 * sp + 4 * g4;
        lo = frag_mul<Op>(lds_frag<Op>(src), f);
        hi = 32 * sp + 16 < D ? frag_mul<Op>(lds_frag<Op>(src + 16), f) : zero_frag<Op>();
        dst = reinterpret_cast<Op*>(unit + K::Q_OFF) + (q * 64 + lane) * 8;
      } else if (q < NQ + NK) {
        const int idx = q - NQ, mt = idx / NPC, sp = idx % NPC;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t0 = 32 * sp + 4 * g4 + i, t1 = t0 + 16;
          lo[i] = from_f32<Op>(t0 < C ? to_f32(sK[t0 * LD_D + 16 * mt + l16]) * fast_exp(g_n - sG[t0]) : 0.f);
          hi[i] = from_f32<Op>(t1 < C ? to_f32(sK[t1 * LD_D + 16 * mt + l16]) * fast_exp(g_n - sG[t1]) : 0.f);
        }
        dst = reinterpret_cast<Op*>(unit + K::KT_OFF) + (idx * 64 + lane) * 8;
      } else {
        const int idx = q - NQ - NK, mt = idx / NPC, sp = idx % NPC;
        const Op* src = sP + (16 * mt + l16) * LD_C + 32 * sp + 4 * g4;
        lo = frag_mul<Op>(lds_frag<Op>(src), scale);
        hi = 32 * sp + 16 < C ? frag_mul<Op>(lds_frag<Op>(src + 16), scale) : zero_frag<Op>();
        dst = reinterpret_cast<Op*>(unit + K::P_OFF) + (idx * 64 + lane) * 8;
      }
      store_pair<Op>(dst, lo, hi);
    }
  }

  // ---- T = (I + A)^-1 in place.  (a) diagonal 16x16 blocks, one lane per column
  if (tid < CT * 16) {
    const int b = tid >> 4, c = tid & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* arow = sAT + (16 * b + r) * LD_F + 16 * b;
      float acc = r == c ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) acc = fmaf(-arow[j], x[j], acc);
      x[r] = acc;
    }
    // every read of this block above precedes these writes in the wave's program order
#pragma unroll
    for (int r = 0; r < 16; ++r) sAT[(16 * b + r) * LD_F + 16 * b + c] = x[r];
  }
  __syncthreads();
  // (b) block rows: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.  The A blocks of the
  // row are read into registers before any wave overwrites them with T.
#pragma unroll
  for (int bi = 1; bi < CT; ++bi) {
    f32x4 a_row[CT];
#pragma unroll
    for (int bk = 0; bk < CT; ++bk)
      if (bk < bi) a_row[bk] = lds_frag<float>(sAT + (16 * bi + l16) * LD_F + 16 * bk + 4 * g4);
    __syncthreads();
    for (int bj = wave; bj < bi; bj += WAVES) {
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bk = 0; bk < CT; ++bk)
        if (bk >= bj && bk < bi) {
          f32x4 b;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) b[jj] = sAT[(16 * bk + 4 * g4 + jj) * LD_F + 16 * bj + l16];
          mma_k16(X, a_row[bk], b);
        }
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
      mma_k16(Y, lds_frag<float>(sAT + (16 * bi + l16) * LD_F + 16 * bi + 4 * g4), X);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sAT[(16 * bi + 4 * g4 + jj) * LD_F + 16 * bj + l16] = -Y[jj];
    }
    __syncthreads();
  }

  // ---- W = T diag(b e^G) K -> LDS over q^ (dead), Ut = T diag(b) V -> workspace (fragment order)
  {
    Op* ut = reinterpret_cast<Op*>(unit + K::UT_OFF);
    for (int q = wave; q < 2 * CT * NT; q += WAVES) {
      const bool is_u = q >= CT * NT;
      const int idx = is_u ? q - CT * NT : q;
      const int mt = idx / NT, nt = idx % NT;
      const float* scl = is_u ? sB : sBE;
      const Op* src = is_u ? sV : sK;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* trow = sAT + (16 * mt + l16) * LD_F;
      for (int kb = 0; kb <= mt; ++kb) {  // T is lower triangular
        const FragT a = frag_scaled<Op>(trow + 16 * kb + 4 * g4, scl + 16 * kb + 4 * g4);
        const FragT b = frag_col<Op>(src + (16 * kb + 4 * g4) * LD_D + 16 * nt + l16, LD_D);
        mma_k16(acc, a, b);
      }
      if (is_u) {
        // lane-fragment order: [mt][nt][lane][4], as the state kernel's accumulators
        *reinterpret_cast<FragT*>(ut + ((mt * NT + nt) * 64 + lane) * 4) = frag_from<Op>(acc);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) sQ[(16 * mt + 4 * g4 + i) * LD_D + 16 * nt + l16] = from_f32<Op>(acc[i]);
      }
    }
  }
  __syncthreads();
  // ---- -W as pair fragments (the chain adds -W S^T to Ut)
  {
    constexpr int NPD = K::NPD;
    for (int q = wave; q < CT * NPD; q += WAVES) {
      const int mt = q / NPD, sp = q % NPD;
      const Op* src = sQ + (16 * mt + l16) * LD_D + 32 * sp + 4 * g4;
      const FragT lo = frag_mul<Op>(lds_frag<Op>(src), -1.f);
      const FragT hi = 32 * sp + 16 < D ? frag_mul<Op>(lds_frag<Op>(src + 16), -1.f) : zero_frag<Op>();
      store_pair<Op>(reinterpret_cast<Op*>(unit + K::W_OFF) + (q * 64 + lane) * 8, lo, hi);
    }
  }
}

// ----------------------------------------------------------------- state
// One wave: the chain of one sequence's chunks for one V head and NTW 16-wide
// tiles of d_v.  S^T[d_k][d_v-slice] lives in accumulators (lane: d_k rows
// 4g..4g+3 of each 16-block, d_v column l16), which is also the B operand
// layout for every product that contracts over d_k.  Operands of chunk c+1 are
// loaded right after chunk c consumed the same registers.  Block order puts
// all tiles of one (sequence, head) on one XCD, so its fragments are fetched
// into that XCD's L2 once.
template <typename Op, int D, int C, int NTW>
__global__ __launch_bounds__(64) void chunk_state_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const uint8_t* __restrict__ has_init,
    const int32_t* __restrict__ cstart, const unsigned char* __restrict__ ws, float* __restrict__ state,
    int32_t n_slots, Op* __restrict__ o, int64_t t_total, int32_t n_seq, int32_t h_v) {
  using K = Cfg<Op, D, C>;
  using FragT = typename Frag<Op>::type;
  constexpr int NT = K::NT, CT = K::CT, NPD = K::NPD, NPC = K::NPC, NTILE = NT / NTW;
  const int xcd = blockIdx.x & 7, kq = blockIdx.x >> 3, tile = kq % NTILE;
  const int64_t grp = (int64_t)(kq / NTILE) * 8 + xcd;
  if (grp >= (int64_t)n_seq * h_v) return;
  const int n = (int)(grp / h_v), h = (int)(grp % h_v);
  const int lane = threadIdx.x, g4 = lane >> 4, l16 = lane & 15;
  const int col0 = h * D + 16 * NTW * tile;  // first output column of this wave
  const int64_t o_ld = (int64_t)h_v * D;
  const int64_t lo = min((int64_t)cu[n], t_total);
  const int64_t hi = min(max((int64_t)cu[n + 1], lo), t_total);
  const int32_t slot = slots[n];
  if (!slot_ok(slot, n_slots)) {  // padding entry: zero outputs
    for (int64_t e = lane; e < (hi - lo) * 16 * NTW; e += 64)
      o[(lo + e / (16 * NTW)) * o_ld + col0 + e % (16 * NTW)] = from_f32<Op>(0.f);
    return;
  }
  const bool init = has_init == nullptr || has_init[n] != 0;
  float* st_ptr = state + ((int64_t)slot * h_v + h) * D * D;

  f32x4 Sacc[NT][NTW];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int dv = 16 * (NTW * tile + j) + l16;
      if (init) {
        const float4 v = *reinterpret_cast<const float4*>(st_ptr + dv * D + 16 * mt + 4 * g4);
        Sacc[mt][j] = f32x4{v.x, v.y, v.z, v.w};
      } else {
        Sacc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

  Pair<Op> wn[CT][NPD], qp[CT][NPD], kt[NT][NPC], pp[CT][NPC];
  FragT ut[CT][NTW];
  float egn = 0.f;
#define GDN_LOAD_WU(u)                                                                              \
  {                                                                                                 \
    const Op* w_ = reinterpret_cast<const Op*>((u) + K::W_OFF);                                     \
    _Pragma("unroll") for (int mt = 0; mt < CT; ++mt)                                               \
    _Pragma("unroll") for (int sp = 0; sp < NPD; ++sp) wn[mt][sp].load(w_ + ((mt * NPD + sp) * 64 + lane) * 8); \
    const Op* u_ = reinterpret_cast<const Op*>((u) + K::UT_OFF);                                    \
    _Pragma("unroll") for (int mt = 0; mt < CT; ++mt)                                               \
    _Pragma("unroll") for (int j = 0; j < NTW; ++j)                                                 \
      ut[mt][j] = *reinterpret_cast<const FragT*>(u_ + ((mt * NT + NTW * tile + j) * 64 + lane) * 4); \
  }
#define GDN_LOAD_Q(u)                                                                               \
  {                                                                                                 \
    const Op* q_ = reinterpret_cast<const Op*>((u) + K::Q_OFF);                                     \
    _Pragma("unroll") for (int mt = 0; mt < CT; ++mt)                                               \
    _Pragma("unroll") for (int sp = 0; sp < NPD; ++sp) qp[mt][sp].load(q_ + ((mt * NPD + sp) * 64 + lane) * 8); \
  }
#define GDN_LOAD_P(u)                                                                               \
  {                                                                                                 \
    const Op* p_ = reinterpret_cast<const Op*>((u) + K::P_OFF);                                     \
    _Pragma("unroll") for (int mt = 0; mt < CT; ++mt)                                               \
    _Pragma("unroll") for (int sp = 0; sp < NPC; ++sp)                                              \
      if (2 * sp <= mt) pp[mt][sp].load(p_ + ((mt * NPC + sp) * 64 + lane) * 8);                    \
  }
#define GDN_LOAD_KT(u)                                                                              \
  {                                                                                                 \
    const Op* k_ = reinterpret_cast<const Op*>((u) + K::KT_OFF);                                    \
    _Pragma("unroll") for (int mt = 0; mt < NT; ++mt)                                               \
    _Pragma("unroll") for (int sp = 0; sp < NPC; ++sp) kt[mt][sp].load(k_ + ((mt * NPC + sp) * 64 + lane) * 8); \
    egn = *reinterpret_cast<const float*>((u) + K::F_OFF);                                          \
  }
  int32_t gcx = cstart[n];
  if (lo < hi) {
    const unsigned char* u0 = ws + ((int64_t)gcx * h_v + h) * K::UNIT;
    GDN_LOAD_WU(u0);
    GDN_LOAD_Q(u0);
    GDN_LOAD_P(u0);
    GDN_LOAD_KT(u0);
  }
  const FragT zf = zero_frag<Op>();
  const int32_t lane_off = (int32_t)(4 * g4 * o_ld) + l16;  // lane's row 4g and column within the tile

  for (int64_t c0 = lo; c0 < hi; c0 += C, ++gcx) {
    const int nvalid = (int)min((int64_t)C, hi - c0);
    // The next chunk's operands are loaded unconditionally (the last chunk
    // re-reads its own unit), so the wait counts stay exact: a load under a
    // branch makes the compiler wait for every load issued after it as well.
    // Scheduling fences keep each group right after the phase that frees its
    // registers, a full iteration ahead of its use.
    const unsigned char* un = ws + ((int64_t)(c0 + C < hi ? gcx + 1 : gcx) * h_v + h) * K::UNIT;

    FragT Sf[NT][NTW];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < NTW; ++j) Sf[mt][j] = frag_from<Op>(Sacc[mt][j]);

    // U = Ut - W S^T
    f32x4 Uacc[CT][NTW];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = to_f32(ut[mt][j][i]);
#pragma unroll
        for (int sp = 0; sp < NPD; ++sp) wn[mt][sp].mma(acc, Sf[2 * sp][j], 2 * sp + 1 < NT ? Sf[2 * sp + 1][j] : zf);
        Uacc[mt][j] = acc;
      }
    __builtin_amdgcn_sched_barrier(0);
    GDN_LOAD_WU(un);
    __builtin_amdgcn_sched_barrier(0);

    // O = Q' S^T
    f32x4 Oacc[CT][NTW];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < NPD; ++sp) qp[mt][sp].mma(acc, Sf[2 * sp][j], 2 * sp + 1 < NT ? Sf[2 * sp + 1][j] : zf);
        Oacc[mt][j] = acc;
      }
    __builtin_amdgcn_sched_barrier(0);
    GDN_LOAD_Q(un);
    __builtin_amdgcn_sched_barrier(0);

    // O += P U
    FragT Uf[CT][NTW];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int j = 0; j < NTW; ++j) Uf[mt][j] = frag_from<Op>(Uacc[mt][j]);
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int sp = 0; sp < NPC; ++sp)
          if (2 * sp <= mt) pp[mt][sp].mma(Oacc[mt][j], Uf[2 * sp][j], 2 * sp + 1 < CT ? Uf[2 * sp + 1][j] : zf);
    __builtin_amdgcn_sched_barrier(0);
    GDN_LOAD_P(un);
    __builtin_amdgcn_sched_barrier(0);

    // S^T <- e^{G_n} S^T + K'^T U
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        f32x4 acc = Sacc[mt][j];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= egn;
#pragma unroll
        for (int sp = 0; sp < NPC; ++sp) kt[mt][sp].mma(acc, Uf[2 * sp][j], 2 * sp + 1 < CT ? Uf[2 * sp + 1][j] : zf);
        Sacc[mt][j] = acc;
      }
    __builtin_amdgcn_sched_barrier(0);
    GDN_LOAD_KT(un);
    __builtin_amdgcn_sched_barrier(0);

    // O out (the scale is in Q' and P).  Row bases are uniform, the lane part
    // is loop-invariant; a full chunk stores without per-row guards.
    if (nvalid == C) {
#pragma unroll
      for (int mt = 0; mt < CT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Op* orow = o + (c0 + 16 * mt + i) * o_ld + col0;
#pragma unroll
          for (int j = 0; j < NTW; ++j) orow[lane_off + 16 * j] = from_f32<Op>(Oacc[mt][j][i]);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < CT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Op* orow = o + (c0 + 16 * mt + i) * o_ld + col0;
          if (16 * mt + 4 * g4 + i < nvalid) {
#pragma unroll
            for (int j = 0; j < NTW; ++j) orow[lane_off + 16 * j] = from_f32<Op>(Oacc[mt][j][i]);
          }
        }
    }
  }
#undef GDN_LOAD_WU
#undef GDN_LOAD_Q
#undef GDN_LOAD_P
#undef GDN_LOAD_KT

#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int dv = 16 * (NTW * tile + j) + l16;
      *reinterpret_cast<float4*>(st_ptr + dv * D + 16 * mt + 4 * g4) =
          make_float4(Sacc[mt][j][0], Sacc[mt][j][1], Sacc[mt][j][2], Sacc[mt][j][3]);
    }
}

// ------------------------------------------------------------------ norm
// out = o / sqrt(mean_dv(o^2) + eps) * w * silu(z) in place, o = scale * O as
// the chain wrote it.  D / 8 lanes hold one (token, V head) row.  Tokens
// outside [cu[0], cu[n_seq]) are left alone, as the chain leaves them.
template <typename T, int D>
__global__ __launch_bounds__(256) void gated_norm_kernel(T* __restrict__ o, const T* __restrict__ z,
                                                         const T* __restrict__ norm_w,
                                                         const int32_t* __restrict__ cu, int32_t n_seq,
                                                         int64_t t_total, int32_t h_v, float eps) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int e0 = (threadIdx.x % LPR) * 8;
  const int64_t t = row / h_v;
  const int64_t t_lo = max((int64_t)cu[0], (int64_t)0), t_hi = min((int64_t)cu[n_seq], t_total);
  const bool live = t >= t_lo && t < t_hi;
  float v[8], zz[8], w[8];
  if (live) {
    load8(o + row * D + e0, v);
    load8(z + row * D + e0, zz);
    load8(norm_w + e0, w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = zz[e] = w[e] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  ss = group_sum<LPR>(ss);  // LPR lanes of a row are an aligned group
  const float rstd = fast_rsq(ss * (1.0f / D) + eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = v[e] * rstd * w[e] * fast_silu(zz[e]);
  if (live) store8(o + row * D + e0, v);
}

// Tiles of d_v per wave: one for a single long sequence is the most
// parallel chain.
template <typename Op, int D>
constexpr int kTileW = 1;

// workspace: [chunk index][units]
inline size_t idx_bytes(int32_t n_seq) { return (((size_t)n_seq + 1) * 4 + 255) / 256 * 256; }

template <typename T, typename Op, int D, int C>
size_t ws_bytes(int32_t n_seq, int64_t t_total, int32_t h_v) {
  using K = Cfg<Op, D, C>;
  const int64_t max_chunks = t_total / C + n_seq;
  return idx_bytes(n_seq) + (size_t)max_chunks * h_v * K::UNIT;
}

template <typename T, typename Op, int D, int C>
hipError_t run(const ChunkArgs& a, hipStream_t st) {
  using K = Cfg<Op, D, C>;
  static_assert(sizeof(T) == sizeof(Op), "the chain writes O in the activation type");
  static_assert(K::PREP_BYTES <= 160 * 1024, "LDS budget");
  constexpr int NTW = kTileW<Op, D>, NTILE = K::NT / NTW;
  if (a.n_seq == 0) return hipSuccess;
  int32_t* cstart = reinterpret_cast<int32_t*>(a.workspace);
  unsigned char* units = reinterpret_cast<unsigned char*>(a.workspace) + idx_bytes(a.n_seq);
  hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.n_seq, a.t_total, (int32_t)C,
                     cstart);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t max_chunks = a.t_total / C + a.n_seq;
  if (max_chunks > 0) {
    hipLaunchKernelGGL((chunk_prep_kernel<T, Op, D, C>), dim3((unsigned)(max_chunks * a.s.h_v)), dim3(K::THREADS), 0,
                       st, (const T*)a.qkv, a.g, a.beta, a.cu_seqlens, a.slots, cstart, a.n_slots, a.n_seq, a.t_total,
                       a.s.h_k, a.s.h_v, a.scale, units);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const int64_t groups = ((int64_t)a.n_seq * a.s.h_v + 7) / 8 * 8;
  hipLaunchKernelGGL((chunk_state_kernel<Op, D, C, NTW>), dim3((unsigned)(groups * NTILE)), dim3(64), 0, st,
                     a.cu_seqlens, a.slots, a.has_init, cstart, units, a.state, a.n_slots, (Op*)a.o, a.t_total,
                     a.n_seq, a.s.h_v);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (a.z != nullptr && a.t_total > 0) {
    constexpr int RPB = 256 / (D / 8);
    const int64_t rows = a.t_total * a.s.h_v;
    hipLaunchKernelGGL((gated_norm_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                       (T*)a.o, (const T*)a.z, (const T*)a.norm_w, a.cu_seqlens, a.n_seq, a.t_total, a.s.h_v,
                       a.norm_eps);
  }
  return hipGetLastError();
}

template <typename T, typename Op, int D>
hipError_t by_chunk(const ChunkArgs& a, hipStream_t st) {
  switch (a.chunk) {
    case 16: return run<T, Op, D, 16>(a, st);
    case 32: return run<T, Op, D, 32>(a, st);
    case 64: return run<T, Op, D, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename Op, int D>
size_t ws_by_chunk(int chunk, int32_t n_seq, int64_t t_total, int32_t h_v) {
  switch (chunk) {
    case 16: return ws_bytes<T, Op, D, 16>(n_seq, t_total, h_v);
    case 32: return ws_bytes<T, Op, D, 32>(n_seq, t_total, h_v);
    case 64: return ws_bytes<T, Op, D, 64>(n_seq, t_total, h_v);
  }
  return 0;
}

}  // namespace split

size_t chunk_split_workspace_size(const Shape& s, bool is_bf16, int32_t n_seq, int64_t t_total, int32_t chunk) {
  switch (s.d) {
    case 16: return is_bf16 ? split::ws_by_chunk<bf16, bf16, 16>(chunk, n_seq, t_total, s.h_v)
                         : split::ws_by_chunk<float, float, 16>(chunk, n_seq, t_total, s.h_v);
    case 32: return is_bf16 ? split::ws_by_chunk<bf16, bf16, 32>(chunk, n_seq, t_total, s.h_v)
                         : split::ws_by_chunk<float, float, 32>(chunk, n_seq, t_total, s.h_v);
    case 64: return is_bf16 ? split::ws_by_chunk<bf16, bf16, 64>(chunk, n_seq, t_total, s.h_v)
                         : split::ws_by_chunk<float, float, 64>(chunk, n_seq, t_total, s.h_v);
    case 128: return is_bf16 ? split::ws_by_chunk<bf16, bf16, 128>(chunk, n_seq, t_total, s.h_v)
                          : split::ws_by_chunk<float, float, 128>(chunk, n_seq, t_total, s.h_v);
  }
  return 0;
}

hipError_t launch_chunk_split(const ChunkArgs& a, hipStream_t st) {
  switch (a.s.d) {
    case 16: return a.bf16 ? split::by_chunk<bf16, bf16, 16>(a, st) : split::by_chunk<float, float, 16>(a, st);
    case 32: return a.bf16 ? split::by_chunk<bf16, bf16, 32>(a, st) : split::by_chunk<float, float, 32>(a, st);
    case 64: return a.bf16 ? split::by_chunk<bf16, bf16, 64>(a, st) : split::by_chunk<float, float, 64>(a, st);
    case 128: return a.bf16 ? split::by_chunk<bf16, bf16, 128>(a, st) : split::by_chunk<float, float, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

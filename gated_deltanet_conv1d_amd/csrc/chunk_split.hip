// Chunked gated delta rule, split into a chunk-parallel preparation pass and
// a per-sequence state pass.  Same math as chunk_prefill.hip (the chunked
// WY / UT form of the gated delta rule over 64-token chunks):
//   A = strict-lower(b_i e^{G_i-G_j} k_i.k_j),  T = (I + A)^{-1},
//   W = T diag(b e^G) K,  Ut = T diag(b) V,  P = M o Q K^T        (no state)
//   U = Ut - W S0^T,  O = diag(e^G) Q S0^T + P U,
//   S = e^{G_n} S0 + K^T diag(e^{G_n - G}) U                       (the chain)
//
// Why split on MI355X: everything in the first line depends only on the
// chunk's own tokens, so it runs as one workgroup per (chunk, V head) across
// the whole GPU (thousands of workgroups, two per CU by LDS), while the serial
// chain per (sequence, V head) keeps only the three state contractions and
// the epilogue.  The price is a workspace round trip of W, Ut, P and G
// (bf16 for the operands: 40 KiB per chunk and head at d = 128, C = 64).
//
//   chunk_index_kernel  first global chunk of every sequence (block scan)
//   chunk_prep_kernel   per (chunk, V head): q/k L2 norm, gates, Gram, T, W, Ut, P
//   chunk_state_kernel  per (sequence, V head): S^T in MFMA accumulators, the
//                       chunk loop with prefetched operands, gated-RMSNorm epilogue
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
  // workspace unit per (chunk, V head), bytes
  static constexpr int W_OFF = 0;
  static constexpr int UT_OFF = W_OFF + C * D * (int)sizeof(Op);
  static constexpr int P_OFF = UT_OFF + C * D * (int)sizeof(Op);
  static constexpr int G_OFF = P_OFF + C * C * (int)sizeof(Op);
  static constexpr int RQ_OFF = G_OFF + C * 4;   // 1 / sqrt(|q_t|^2 + eps)
  static constexpr int RK_OFF = RQ_OFF + C * 4;  // 1 / sqrt(|k_t|^2 + eps)
  static constexpr int UNIT = RK_OFF + C * 4;
  // prep kernel LDS
  static constexpr int PQ = 0;                                     // q^ rows, later W
  static constexpr int PK = PQ + C * LD_D * (int)sizeof(Op);       // k^ rows
  static constexpr int PV = PK + C * LD_D * (int)sizeof(Op);       // v rows
  static constexpr int PA = PV + C * LD_D * (int)sizeof(Op);       // fp32 A, then T in place
  static constexpr int PP = PA + C * LD_F * 4;                     // P
  static constexpr int PG = PP + C * LD_C * (int)sizeof(Op);       // G, beta, beta e^G
  static constexpr int PREP_BYTES = PG + 3 * C * 4;
  // state kernel LDS
  static constexpr int SQ = 0;                                     // raw q rows
  static constexpr int SK = SQ + C * LD_D * (int)sizeof(Op);       // raw k rows
  static constexpr int SW = SK + C * LD_D * (int)sizeof(Op);
  static constexpr int SP = SW + C * LD_D * (int)sizeof(Op);
  static constexpr int SG = SP + C * LD_C * (int)sizeof(Op);       // G, e^G r_q, e^(G_n - G) r_k
  static constexpr int SR = SG + 3 * C * 4;                        // [WAVES][C] row sums
  static constexpr int STATE_BYTES = SR + WAVES * C * 4;
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

// ------------------------------------------------------------------ prep
template <typename T, typename Op, int D, int C>
__global__ __launch_bounds__(kThreads<D>) void chunk_prep_kernel(
    const T* __restrict__ qkv, const float* __restrict__ g_in, const float* __restrict__ beta_in,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const int32_t* __restrict__ cstart,
    int32_t n_slots, int32_t n_seq, int64_t t_total, int32_t h_k, int32_t h_v, unsigned char* __restrict__ ws) {
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
          if (r < C && tid % LPR == 0) reinterpret_cast<float*>(unit + (kind == 0 ? K::RQ_OFF : K::RK_OFF))[r] = rn;
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
        reinterpret_cast<float*>(unit + K::G_OFF)[lane] = gv;
      }
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
  // ---- W and P rows to the workspace, 16-byte pieces
  {
    Op* wdst = reinterpret_cast<Op*>(unit + K::W_OFF);
    for (int e = tid; e < C * D / 8; e += K::THREADS) {
      const int r = e / (D / 8), c8 = (e % (D / 8)) * 8;
      float v[8];
      load8(sQ + r * LD_D + c8, v);
      store8(wdst + r * D + c8, v);
    }
    Op* pdst = reinterpret_cast<Op*>(unit + K::P_OFF);
    for (int e = tid; e < C * C / 8; e += K::THREADS) {
      const int r = e / (C / 8), c8 = (e % (C / 8)) * 8;
      float v[8];
      load8(sP + r * LD_C + c8, v);
      store8(pdst + r * C + c8, v);
    }
  }
}

// ----------------------------------------------------------------- state
// 8 raw activations into LDS unchanged (activation and operand types agree).
template <typename T>
__device__ __forceinline__ void raw_store(const Raw8<T>& r, T* dst);
template <>
__device__ __forceinline__ void raw_store<bf16>(const Raw8<bf16>& r, bf16* dst) {
  reinterpret_cast<uint2*>(dst)[0] = make_uint2(r.u.x, r.u.y);
  reinterpret_cast<uint2*>(dst)[1] = make_uint2(r.u.z, r.u.w);
}
template <>
__device__ __forceinline__ void raw_store<float>(const Raw8<float>& r, float* dst) {
  reinterpret_cast<uint4*>(dst)[0] = r.u[0];
  reinterpret_cast<uint4*>(dst)[1] = r.u[1];
}

// The chain over one sequence's chunks for one V head.  q and k stay raw in LDS:
// their L2 norms (from the prep pass) are folded into the rows of the products,
//   diag(r_q) Q S^T  and  (diag(r_k) K)^T U' = K^T (diag(r_k) U'),
// so staging is a plain copy.  The epilogue works from registers: z arrives in
// accumulator layout with the prefetch and o leaves straight from the tiles;
// only the gated RMSNorm's cross-wave row sums go through LDS.
template <typename T, typename Op, int D, int C>
__global__ __launch_bounds__(kThreads<D>) void chunk_state_kernel(
    const T* __restrict__ qkv, const int32_t* __restrict__ cu, const int32_t* __restrict__ slots,
    const uint8_t* __restrict__ has_init, const int32_t* __restrict__ cstart, const unsigned char* __restrict__ ws,
    float* __restrict__ state, int32_t n_slots, T* __restrict__ o, const T* __restrict__ z,
    const T* __restrict__ norm_w, float norm_eps, float scale, int64_t t_total, int32_t h_k, int32_t h_v) {
  static_assert(sizeof(T) == sizeof(Op), "activations are staged unchanged as MFMA operands");
  using K = Cfg<Op, D, C>;
  using FragT = typename Frag<Op>::type;
  constexpr int NT = K::NT, CT = K::CT, WAVES = K::WAVES, DVT = K::DVT, LPR = K::LPR, RPP = K::RPP;
  constexpr int RPT = K::RPT, LD_D = K::LD_D, LD_C = K::LD_C;
  constexpr int WPT = (C * D / 8 + K::THREADS - 1) / K::THREADS;  // W pieces per thread
  constexpr int PPT = (C * C / 8 + K::THREADS - 1) / K::THREADS;  // P pieces per thread
  __shared__ __attribute__((aligned(16))) unsigned char smem[K::STATE_BYTES];
  Op* sQ = reinterpret_cast<Op*>(smem + K::SQ);
  Op* sK = reinterpret_cast<Op*>(smem + K::SK);
  Op* sW = reinterpret_cast<Op*>(smem + K::SW);
  Op* sP = reinterpret_cast<Op*>(smem + K::SP);
  float* sG = reinterpret_cast<float*>(smem + K::SG);
  float* sFQ = sG + C;      // e^{G_t} r_q[t]
  float* sFK = sG + 2 * C;  // e^{G_n - G_t} r_k[t]
  float* sRed = reinterpret_cast<float*>(smem + K::SR);

  const int n = blockIdx.x / h_v;
  const int h = blockIdx.x % h_v;
  const int hk = h / (h_v / h_k);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int c_ch = 2 * h_k * D + h_v * D;
  const int64_t o_ld = (int64_t)h_v * D;
  const int64_t lo = min((int64_t)cu[n], t_total);
  const int64_t hi = min(max((int64_t)cu[n + 1], lo), t_total);
  const int32_t slot = slots[n];
  if (!slot_ok(slot, n_slots)) {
    for (int64_t t = lo; t < hi; ++t)
      for (int r = tid; r < D; r += K::THREADS) o[t * o_ld + h * D + r] = from_f32<T>(0.0f);
    return;
  }
  const bool init = has_init == nullptr || has_init[n] != 0;
  float* st_ptr = state + ((int64_t)slot * h_v + h) * D * D;
  const int32_t gc0 = cstart[n];

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
  float nw[DVT];
#pragma unroll
  for (int j = 0; j < DVT; ++j) nw[j] = z ? to_f32(norm_w[16 * (wave * DVT + j) + l16]) : 1.f;

  // operands of the next chunk, prefetched into registers in two groups
  const int e0 = (tid % LPR) * 8, r0 = tid / LPR;
  const int64_t col_q = (int64_t)hk * D, col_k = (int64_t)(h_k + hk) * D;
  Raw8<T> pq[RPT], pk[RPT];
  Raw8<Op> pw[WPT], pp[PPT];
  FragT put[CT][DVT];
  T pz[CT][DVT][4];
  float pg = 0.f, prq = 0.f, prk = 0.f;
#define GDN_PREFETCH_A(cs, gcx)                                                                  \
  {                                                                                              \
    const int nv_ = (int)min((int64_t)C, hi - (cs));                                             \
    const unsigned char* unit_ = ws + ((int64_t)(gcx) * h_v + h) * K::UNIT;                      \
    _Pragma("unroll") for (int j = 0; j < RPT; ++j) {                                            \
      const int r = r0 + j * RPP;                                                                \
      if (r < nv_) {                                                                             \
        pq[j].load(qkv + ((cs) + r) * c_ch + col_q + e0);                                        \
        pk[j].load(qkv + ((cs) + r) * c_ch + col_k + e0);                                        \
      } else {                                                                                   \
        pq[j].zero(); pk[j].zero();                                                              \
      }                                                                                          \
    }                                                                                            \
    const Op* w_ = reinterpret_cast<const Op*>(unit_ + K::W_OFF);                                \
    _Pragma("unroll") for (int j = 0; j < WPT; ++j) {                                            \
      const int e = tid + j * K::THREADS;                                                        \
      if (e < C * D / 8) pw[j].load(w_ + (e / (D / 8)) * D + (e % (D / 8)) * 8); else pw[j].zero(); \
    }                                                                                            \
  }
#define GDN_PREFETCH_B(cs, gcx)                                                                  \
  {                                                                                              \
    const int nv_ = (int)min((int64_t)C, hi - (cs));                                             \
    const unsigned char* unit_ = ws + ((int64_t)(gcx) * h_v + h) * K::UNIT;                      \
    const Op* p_ = reinterpret_cast<const Op*>(unit_ + K::P_OFF);                                \
    _Pragma("unroll") for (int j = 0; j < PPT; ++j) {                                            \
      const int e = tid + j * K::THREADS;                                                        \
      if (e < C * C / 8) pp[j].load(p_ + (e / (C / 8)) * C + (e % (C / 8)) * 8); else pp[j].zero(); \
    }                                                                                            \
    const Op* u_ = reinterpret_cast<const Op*>(unit_ + K::UT_OFF);                               \
    _Pragma("unroll") for (int mt = 0; mt < CT; ++mt)                                            \
    _Pragma("unroll") for (int j = 0; j < DVT; ++j)                                              \
      put[mt][j] = *reinterpret_cast<const FragT*>(u_ + ((mt * NT + wave * DVT + j) * 64 + lane) * 4); \
    if (wave == 0 && lane < C) {                                                                 \
      pg = reinterpret_cast<const float*>(unit_ + K::G_OFF)[lane];                               \
      prq = reinterpret_cast<const float*>(unit_ + K::RQ_OFF)[lane];                             \
      prk = reinterpret_cast<const float*>(unit_ + K::RK_OFF)[lane];                             \
    }                                                                                            \
    if (z) {                                                                                     \
      _Pragma("unroll") for (int mt = 0; mt < CT; ++mt)                                          \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                            \
        const int t = 16 * mt + 4 * g4 + i;                                                      \
        _Pragma("unroll") for (int j = 0; j < DVT; ++j)                                          \
          pz[mt][j][i] = t < nv_ ? z[((cs) + t) * o_ld + h * D + 16 * (wave * DVT + j) + l16]    \
                                 : from_f32<T>(0.f);                                             \
      }                                                                                          \
    }                                                                                            \
  }
  if (lo < hi) {
    GDN_PREFETCH_A(lo, gc0);
    GDN_PREFETCH_B(lo, gc0);
  }

  int32_t gcx = gc0;
  for (int64_t c0 = lo; c0 < hi; c0 += C, ++gcx) {
    const int nvalid = (int)min((int64_t)C, hi - c0);
    const bool more = c0 + C < hi;
    // ---- prefetched registers -> LDS; Ut -> accumulators; per-token factors
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = r0 + j * RPP;
      if (r < C) {
        raw_store<Op>(*reinterpret_cast<const Raw8<Op>*>(&pq[j]), sQ + r * LD_D + e0);
        raw_store<Op>(*reinterpret_cast<const Raw8<Op>*>(&pk[j]), sK + r * LD_D + e0);
      }
    }
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int e = tid + j * K::THREADS;
      if (e < C * D / 8) raw_store<Op>(pw[j], sW + (e / (D / 8)) * LD_D + (e % (D / 8)) * 8);
    }
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int e = tid + j * K::THREADS;
      if (e < C * C / 8) raw_store<Op>(pp[j], sP + (e / (C / 8)) * LD_C + (e % (C / 8)) * 8);
    }
    f32x4 Uacc[CT][DVT];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int j = 0; j < DVT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) Uacc[mt][j][i] = to_f32(put[mt][j][i]);
    float zz[CT][DVT][4];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int j = 0; j < DVT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) zz[mt][j][i] = to_f32(pz[mt][j][i]);
    if (wave == 0) {
      const float g_last = __shfl(pg, C - 1);
      if (lane < C) {
        sG[lane] = pg;
        sFQ[lane] = fast_exp(pg) * prq;
        sFK[lane] = fast_exp(g_last - pg) * prk;
      }
    }
    __syncthreads();
    if (more) GDN_PREFETCH_A(c0 + C, gcx + 1);

    // ---- U = Ut - W S^T ;  O = diag(e^G r_q) Q S^T
    FragT Sf[NT][DVT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < DVT; ++j) Sf[mt][j] = frag_from<Op>(Sacc[mt][j]);
    f32x4 Oacc[CT][DVT];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt) {
      const Op* wrow = sW + (16 * mt + l16) * LD_D;
      const Op* qrow = sQ + (16 * mt + l16) * LD_D;
#pragma unroll
      for (int j = 0; j < DVT; ++j) {
        f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
        int kb = 0;
#pragma unroll
        for (; kb + 1 < NT; kb += 2) {
          FragT w0 = lds_frag<Op>(wrow + 16 * kb + 4 * g4), w1 = lds_frag<Op>(wrow + 16 * kb + 16 + 4 * g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) { w0[i] = -w0[i]; w1[i] = -w1[i]; }
          mma_k32(Uacc[mt][j], w0, w1, Sf[kb][j], Sf[kb + 1][j]);
          mma_k32(oacc, lds_frag<Op>(qrow + 16 * kb + 4 * g4), lds_frag<Op>(qrow + 16 * kb + 16 + 4 * g4), Sf[kb][j],
                  Sf[kb + 1][j]);
        }
        if (kb < NT) {
          FragT w0 = lds_frag<Op>(wrow + 16 * kb + 4 * g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) w0[i] = -w0[i];
          mma_k16(Uacc[mt][j], w0, Sf[kb][j]);
          mma_k16(oacc, lds_frag<Op>(qrow + 16 * kb + 4 * g4), Sf[kb][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[i] *= sFQ[16 * mt + 4 * g4 + i];
        Oacc[mt][j] = oacc;
      }
    }
    if (more) GDN_PREFETCH_B(c0 + C, gcx + 1);
    // ---- O += P U
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
    // ---- S^T <- e^{G_n} S^T + K^T diag(e^{G_n - G} r_k) U   (K^T read down k's columns)
    {
      const float eg_last = fast_exp(sG[C - 1]);
      FragT Uf[CT][DVT];
#pragma unroll
      for (int kt = 0; kt < CT; ++kt) {
        const f32x4 d = *reinterpret_cast<const f32x4*>(sFK + 16 * kt + 4 * g4);
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
        FragT ka[CT];
#pragma unroll
        for (int kt = 0; kt < CT; ++kt) ka[kt] = frag_col<Op>(sK + (16 * kt + 4 * g4) * LD_D + 16 * mt + l16, LD_D);
#pragma unroll
        for (int j = 0; j < DVT; ++j) {
          f32x4 acc = Sacc[mt][j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] *= eg_last;
          int kb = 0;
#pragma unroll
          for (; kb + 1 < CT; kb += 2) mma_k32(acc, ka[kb], ka[kb + 1], Uf[kb][j], Uf[kb + 1][j]);
          if (kb < CT) mma_k16(acc, ka[kb], Uf[kb][j]);
          Sacc[mt][j] = acc;
        }
      }
    }

    // ---- epilogue: scale, gated RMSNorm over d_v, stores from the tiles
    float f[CT][4];
    if (z) {
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
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < CT; ++mt) {
        f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
          const f32x4 part = *reinterpret_cast<const f32x4*>(sRed + w * C + 16 * mt + 4 * g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) tot[i] += part[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) f[mt][i] = scale * fast_rsq(tot[i] * scale * scale * (1.0f / D) + norm_eps);
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < CT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) f[mt][i] = scale;
    }
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g4 + i;
        if (t < nvalid) {
          T* orow = o + (c0 + t) * o_ld + h * D;
#pragma unroll
          for (int j = 0; j < DVT; ++j) {
            float v = Oacc[mt][j][i] * f[mt][i];
            if (z) v *= nw[j] * fast_silu(zz[mt][j][i]);
            orow[16 * (wave * DVT + j) + l16] = from_f32<T>(v);
          }
        }
      }
    __syncthreads();  // LDS is rewritten by the next chunk
  }
#undef GDN_PREFETCH_A
#undef GDN_PREFETCH_B

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
size_t ws_bytes(int32_t n_seq, int64_t t_total, int32_t h_v) {
  using K = Cfg<Op, D, C>;
  const int64_t max_chunks = t_total / C + n_seq;
  const size_t idx = (((size_t)n_seq + 1) * 4 + 255) / 256 * 256;
  return idx + (size_t)max_chunks * h_v * K::UNIT;
}

template <typename T, typename Op, int D, int C>
hipError_t run(const ChunkArgs& a, hipStream_t st) {
  using K = Cfg<Op, D, C>;
  static_assert(K::PREP_BYTES <= 160 * 1024 && K::STATE_BYTES <= 160 * 1024, "LDS budget");
  if (a.n_seq == 0) return hipSuccess;
  int32_t* cstart = reinterpret_cast<int32_t*>(a.workspace);
  unsigned char* units = reinterpret_cast<unsigned char*>(a.workspace) + (((size_t)a.n_seq + 1) * 4 + 255) / 256 * 256;
  hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.n_seq, a.t_total, (int32_t)C,
                     cstart);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t max_chunks = a.t_total / C + a.n_seq;
  if (max_chunks > 0) {
    hipLaunchKernelGGL((chunk_prep_kernel<T, Op, D, C>), dim3((unsigned)(max_chunks * a.s.h_v)), dim3(K::THREADS), 0,
                       st, (const T*)a.qkv, a.g, a.beta, a.cu_seqlens, a.slots, cstart, a.n_slots, a.n_seq, a.t_total,
                       a.s.h_k, a.s.h_v, units);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((chunk_state_kernel<T, Op, D, C>), dim3((unsigned)((int64_t)a.n_seq * a.s.h_v)),
                     dim3(K::THREADS), 0, st, (const T*)a.qkv, a.cu_seqlens, a.slots, a.has_init, cstart, units,
                     a.state, a.n_slots, (T*)a.o, (const T*)a.z, (const T*)a.norm_w, a.norm_eps, a.scale, a.t_total,
                     a.s.h_k, a.s.h_v);
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

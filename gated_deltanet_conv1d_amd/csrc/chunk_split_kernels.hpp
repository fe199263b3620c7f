// Chunked gated delta rule, split into a chunk-parallel preparation pass and
// a state pass that runs per (sequence, V head, 16-column d_v tile).  The
// math is the chunked WY / UT form of the gated delta rule, from unrolling
// S_t = e^{g_t} S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T (row form, S in
// R^{d_v x d_k}) over a chunk with incoming state S0 and inclusive cumulative
// log-decay G_i = g_1 + ... + g_i:
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
// with no LDS and no barrier in the loop.  The chain keeps only what is
// serial, U and the state update; it records S at every chunk start (h) and
// U, and the output O = diag(f_q) Q h^T + P U with its gated RMSNorm is again
// chunk-parallel.  The prep pass writes the operands as ready-made MFMA
// fragments:
//   -W                             (A operand, contraction over d_k)
//   K^T                            (A operand, contraction over the chunk; raw k,
//                                   so one copy per QK head, in the unit of
//                                   its first V head)
//   scale P                        (A operand, lower triangle; bf16 as hi + lo)
//   Ut                             (accumulator layout; the chain turns it into U)
//   f_q = scale e^G r_q            (per token; the output pass reads raw q)
//   f_k = e^{G_n-G} r_k            (per token; the chain scales U's rows by it)
// so every load is a 16- or 8-byte lane-contiguous vector.  The state update
// K'^T U with K' = diag(f_k) K runs as K^T (diag(f_k) U): k enters exactly as
// the bf16 conv output, and the one rounding is that of the scaled U.
//
//   chunk_index_kernel  first global chunk of every sequence (block scan) and
//                       the sequences longest first; only with more than 8
//                       sequences, else each wave scans
//   chunk_prep_kernel   per (chunk, V head, or both V heads of a QK head when
//                       h_v = 2 h_k): q/k L2 norm, gates, Gram, T and the
//                       operand fragments above
//   chunk_state_kernel  per (sequence, V head, d_v tile): the chunk loop; in
//                       the single-call prefill also the final conv windows
//   chunk_out_kernel    per (chunk, V head): O, gated RMSNorm over d_v, store
//   chunk_chain_out_kernel  many chains: per (sequence, V head), the chunk
//                       loop over all of d_v that also computes the output
//                       (then no output pass runs)
#pragma once
#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "launch_table.hpp"

namespace gdn {
namespace split {

template <int D>
constexpr int kThreads = (D >= 128 ? 4 : (D >= 64 ? 2 : 1)) * 64;
constexpr int kMaxConvW = 4;

template <typename Op, int D, int C>
struct Cfg {
  static constexpr int NT = D / 16;
  static constexpr int CT = C / 16;
  static constexpr int THREADS = kThreads<D>;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int DVT = NT / WAVES;
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
  static constexpr int KT_OFF = W_OFF + CT * NPD * PAIR * (int)sizeof(Op);  // K^T  [NT][NPC]
  static constexpr int P_OFF = KT_OFF + NT * NPC * PAIR * (int)sizeof(Op);  // P   [CT][NPC]
  // bf16 operands: P as a hi + lo pair (the low part, P - bf16(P), next)
  static constexpr int P_PARTS = sizeof(Op) == 2 ? 2 : 1;
  static constexpr int UT_OFF = P_OFF + P_PARTS * CT * NPC * PAIR * (int)sizeof(Op);  // Ut  [CT][NT][64][4]
  static constexpr int H_OFF = UT_OFF + C * D * (int)sizeof(Op);            // S^T at chunk start, [NPD][NT] pairs
  static constexpr int F_OFF = H_OFF + NPD * NT * PAIR * (int)sizeof(Op);   // e^{G_n}, then f_q [C]
  static constexpr int FQ_OFF = F_OFF + 16;                                 // scale e^{G_t} r_q[t]
  // fused-input, a sequence's first chunk only: the old conv window of the q
  // channels, [D][kMaxConvW - 1] like the conv state, for the output pass
  static constexpr int FK_OFF = FQ_OFF + C * 4;                             // e^{G_n-G_t} r_k[t]
  static constexpr int HALO_OFF = FK_OFF + C * 4;
  static constexpr int UNIT = (HALO_OFF + D * (kMaxConvW - 1) * (int)sizeof(Op) + 255) / 256 * 256;
  // output kernel LDS: raw q rows, then (over them) the fp32 O tile, row-major
  static constexpr int LD_Q = D + 8;
  static constexpr int LD_O = D + 4;
  static constexpr int OUT_BYTES = C * LD_O * 4 > C * LD_Q * (int)sizeof(Op) ? C * LD_O * 4 : C * LD_Q * (int)sizeof(Op);
  // prep kernel LDS.  Row strides are padded so that the fragment reads of a
  // wave (16 rows x 4 column groups) spread over the banks: 68 words per row
  // of k / q / v (the 16 rows start 4 banks apart), 68 words per row of A
  // and T.
  static constexpr int LDR = D + 8;    // raw k rows (elements)
  static constexpr int LDA = C + 4;    // fp32 A, then T in place
  static constexpr int LDT = C + 8;    // T diag(b e^G r_k) and T diag(b), operand type
};

__device__ __forceinline__ int32_t seq_of_chunk(const int32_t* __restrict__ cstart, int32_t n_seq, int32_t gc) {
  int32_t lo = 0, hi = n_seq - 1;  // largest i with cstart[i] <= gc
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (cstart[mid] <= gc) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Chunk bookkeeping.  With more than kScanSeqs sequences, chunk_index_kernel
// writes cstart (the first global chunk of every sequence) to the workspace.
// Otherwise no index kernel runs (cstart == nullptr): every wave derives the
// same numbers from cu_seqlens with a short scan in registers.  (Over 64
// sequences of a varlen batch, 140k workgroups each scanning cost more than
// the one-block index kernel they replace.)
constexpr int kScanSeqs = 8;

struct SeqScan {
  int32_t excl, incl;  // this lane's sequence: first global chunk, one past its last
};
template <int C>
__device__ __forceinline__ SeqScan seq_scan(const int32_t* __restrict__ cu, int32_t n_seq, int64_t t_total) {
  const int lane = threadIdx.x & 63;
  int32_t cnt = 0;
  if (lane < n_seq) {
    const int64_t lo = min((int64_t)cu[lane], t_total);
    const int64_t hi = min(max((int64_t)cu[lane + 1], lo), t_total);
    cnt = (int32_t)((hi - lo + C - 1) / C);
  }
  int32_t incl = cnt;
  for (int off = 1; off < n_seq; off <<= 1) {  // (none for one sequence)
    const int32_t up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  return {incl - cnt, incl};
}

// The sequence n holding global chunk gc and its first global chunk; n ==
// n_seq when gc lies past the last chunk.  Wave-uniform; every lane calls it.
template <int C>
__device__ __forceinline__ void locate_chunk(const int32_t* __restrict__ cstart, const int32_t* __restrict__ cu,
                                             int32_t n_seq, int64_t t_total, int32_t gc, int& n, int32_t& first) {
  if (cstart) {
    if (gc >= cstart[n_seq]) {
      n = n_seq;
      first = 0;
      return;
    }
    n = seq_of_chunk(cstart, n_seq, gc);
    first = cstart[n];
    return;
  }
  const SeqScan sc = seq_scan<C>(cu, n_seq, t_total);
  const int lane = threadIdx.x & 63;
  n = __builtin_amdgcn_readfirstlane((int)__popcll(__ballot(lane < n_seq && sc.incl <= gc)));
  first = __builtin_amdgcn_readfirstlane(__shfl(sc.excl, n < 64 ? n : 63));
}

// First global chunk of sequence n.  Every lane calls it.
template <int C>
__device__ __forceinline__ int32_t first_chunk(const int32_t* __restrict__ cstart, const int32_t* __restrict__ cu,
                                               int32_t n_seq, int64_t t_total, int n) {
  if (cstart) return cstart[n];
  return __builtin_amdgcn_readfirstlane(__shfl(seq_scan<C>(cu, n_seq, t_total).excl, n));
}

// cstart[i] = sum over j < i of ceil(len_j / C), for i = 0..n_seq, and
// order[0..n_seq): the sequences by chunk count, longest first (ties by
// index; index order above kOrderSeqs sequences).  One block.
//
// The chain with output runs one workgroup per (sequence, V head) for the
// whole sequence and takes its sequence from order: with lengths spread over a
// batch, dispatching the long chains first keeps the last round of workgroups
// from being one long chain started late (on 64 sequences of 128..8192
// tokens, 256 concurrent chains: 580 chunk steps per slot in index order, 537
// longest first, 534 ideal).
constexpr int kOrderSeqs = 1024;
static __global__ __launch_bounds__(1024) void chunk_index_kernel(const int32_t* __restrict__ cu, int32_t n_seq,
                                                           int64_t t_total, int32_t chunk,
                                                           int32_t* __restrict__ cstart,
                                                           int32_t* __restrict__ order) {
  __shared__ int32_t part[1024];
  __shared__ int32_t cnt[kOrderSeqs];
  const int tid = threadIdx.x;
  const int per = (n_seq + 1023) / 1024;
  const int i0 = min(tid * per, n_seq), i1 = min(i0 + per, n_seq);
  int32_t s = 0;
  for (int i = i0; i < i1; ++i) {
    const int64_t lo = min((int64_t)cu[i], t_total);
    const int64_t hi = min(max((int64_t)cu[i + 1], lo), t_total);
    const int32_t c = (int32_t)((hi - lo + chunk - 1) / chunk);
    if (n_seq <= kOrderSeqs) cnt[i] = c;  // (then i == tid)
    s += c;
  }
  part[tid] = s;
  __syncthreads();
  if (n_seq <= kOrderSeqs) {
    if (tid < n_seq) {
      const int32_t mine = cnt[tid];
      int32_t rank = 0;
      for (int j = 0; j < n_seq; ++j) {
        const int32_t c = cnt[j];
        rank += c > mine || (c == mine && j < tid);
      }
      order[rank] = tid;
    }
  } else {
    for (int i = i0; i < i1; ++i) order[i] = i;
  }
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
// Nontemporal vector access for the output pass's single-use streams (its
// workspace reads, z, the output rows).  Workspace writes stay plain: the
// next pass reads them back, and at single-sequence sizes the whole
// workspace stays in the 256 MiB memory-side cache, which the latency-bound
// chain depends on (nontemporal workspace writes slowed it by 15%).
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
  __device__ __forceinline__ void load_nt(const bf16* p) { v = nt_ld(reinterpret_cast<const bf16x8*>(p)); }
  __device__ __forceinline__ void split(bf16x4& a, bf16x4& b) const {
    a = bf16x4{v[0], v[1], v[2], v[3]};
    b = bf16x4{v[4], v[5], v[6], v[7]};
  }
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
  __device__ __forceinline__ void load_nt(const float* p) {
    lo = nt_ld(reinterpret_cast<const f32x4*>(p));
    hi = nt_ld(reinterpret_cast<const f32x4*>(p) + 1);
  }
  __device__ __forceinline__ void split(f32x4& a, f32x4& b) const {
    a = lo;
    b = hi;
  }
  __device__ __forceinline__ void mma(f32x4& acc, const f32x4& b0, const f32x4& b1) const {
    mma_k32(acc, lo, hi, b0, b1);
  }
};

// A wave-uniform 64-bit value kept in SGPRs (the compiler cannot always prove
// the uniformity of a computed offset).
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Address of a workspace vector: uniform base plus a 32-bit unsigned byte
// offset, which lets the compiler use SGPR-base addressing with no 64-bit
// VALU arithmetic per load.
template <typename V>
__device__ __forceinline__ const V* at(const unsigned char* base, uint32_t off) {
  return reinterpret_cast<const V*>(base + off);
}
template <typename V>
__device__ __forceinline__ V* at(unsigned char* base, uint32_t off) {
  return reinterpret_cast<V*>(base + off);
}

// ------------------------------------------------------------------ prep
// 8 raw activations into LDS unchanged (activation and operand types agree).
template <typename T>
__device__ __forceinline__ void raw_store(const Raw8<T>& r, T* dst);
template <>
__device__ __forceinline__ void raw_store<bf16>(const Raw8<bf16>& r, bf16* dst) {
  *reinterpret_cast<uint4*>(dst) = r.u;
}
template <>
__device__ __forceinline__ void raw_store<float>(const Raw8<float>& r, float* dst) {
  reinterpret_cast<uint4*>(dst)[0] = r.u[0];
  reinterpret_cast<uint4*>(dst)[1] = r.u[1];
}

// Fused-input mode: rows [0, C) of NP channel parts of y = silu(bias +
// causal conv1d(x)) for the chunk at c0, computed exactly as the conv1d
// kernel does (bias, then the window oldest first, fp32 FMA; SiLU; rounded to
// the operand type), written to LDS row-major (part p at dst[p], row stride
// LDR).  Before the sequence start the window reads the slot's conv state
// (zeros without history); rows at or past nvalid are zero.  One item = one
// 8-channel group of one part over RB consecutive rows, the window sliding
// in registers (RB + W - 1 row loads per RB rows).
struct ConvIn {
  const void* x;
  const void* w;
  const void* bias;
  const void* state;   // [rows][W-1] windows, channel c of this sequence at row state_row0 + c
  int64_t state_row0;
  bool init;
  int64_t seq_lo;
};
template <typename T, typename Op, int D, int C, int W, int NP, int RB, int THREADS>
__device__ __forceinline__ void stage_conv(const ConvIn& ci, int c_ch, const int (&col)[NP], int64_t c0, int nvalid,
                                           Op* base, const int (&dst)[NP], int ldr, int tid) {
  constexpr int NG = D / 8, NRB = C / RB, ITEMS = NP * NG * NRB;
  static_assert(C % RB == 0, "row blocks");
  const T* x = reinterpret_cast<const T*>(ci.x);
  const T* wt = reinterpret_cast<const T*>(ci.w);
  const T* bias = reinterpret_cast<const T*>(ci.bias);
  const T* cst = reinterpret_cast<const T*>(ci.state);
  for (int it = tid; it < ITEMS; it += THREADS) {
    const int p = it / (NG * NRB), rem = it % (NG * NRB), cg = rem % NG, rb = rem / NG;
    const int ch = col[p] + 8 * cg;
    if (rb * RB >= nvalid) {  // rows past the sequence's end: zeros, and no window to read
      const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < RB; ++k) store8(base + dst[p] + (rb * RB + k) * ldr + 8 * cg, zero);
      continue;
    }
    // the 8 channels' taps are 8W consecutive weights: W vector loads, issued
    // before the rows, so that waiting for them does not wait for every row
    // (loads retire in issue order) and row k's outputs need only rows up to
    // k + W - 1.  From here every window position lies in
    // [seq_lo - (W-1), c0 + nvalid).  All RB + W - 1 rows are loaded,
    // unconditionally (an out-of-window row re-reads row c0, which is always
    // in range), so the loads overlap.
    Raw8<T> wr[W], br;
#pragma unroll
    for (int j = 0; j < W; ++j) wr[j].load(wt + (int64_t)ch * W + 8 * j);
    if (bias) br.load(bias + ch);
    constexpr int NR = RB + W - 1;
    const int64_t p0 = c0 + rb * RB - (W - 1);  // position of window row 0
    Raw8<T> raw[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int64_t pos = p0 + k;
      const bool in_x = pos >= ci.seq_lo && pos < c0 + nvalid;
      raw[k].load(x + (in_x ? pos : c0) * c_ch + ch);
    }
    float w[W][8], b[8];
    {
      float wf[W * 8];
#pragma unroll
      for (int j = 0; j < W; ++j) wr[j].to_f32(wf + 8 * j);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < W; ++j) w[j][i] = wf[i * W + j];
      if (bias) {
        br.to_f32(b);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = 0.0f;
      }
    }
    float win[W][8];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int64_t pos = p0 + j;
      if (pos >= ci.seq_lo) {
        raw[j].to_f32(win[j]);
      } else {
        const int64_t back = ci.seq_lo - pos;  // 1 .. W-1 steps before the sequence start
#pragma unroll
        for (int i = 0; i < 8; ++i)
          win[j][i] = ci.init ? to_f32(cst[(ci.state_row0 + ch + i) * (W - 1) + (W - 1 - back)]) : 0.0f;
      }
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int r = rb * RB + k;
      float out[8];
      raw[W - 1 + k].to_f32(win[W - 1]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float acc = b[i];
#pragma unroll
        for (int j = 0; j < W; ++j) acc = fmaf(w[j][i], win[j][i], acc);
        out[i] = r < nvalid ? fast_silu(acc) : 0.0f;
      }
      store8(base + dst[p] + r * ldr + 8 * cg, out);
#pragma unroll
      for (int j = 0; j < W - 1; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) win[j][i] = win[j + 1][i];
    }
  }
}

// Gate inputs of the fused-input mode: g, beta from a, b exactly as the gating
// kernel computes them.
struct GateIn {
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
};

// LDS layout of the prep kernel for G V heads per workgroup (one QK head when
// G = h_v / h_k = 2).  Shared: the k rows (and, fused-input, the q rows); per
// V head: its v rows (fused-input), its fp32 A/T tile, G and b.  The A tiles
// overlay the q and v rows in the fused-input mode (those are read into
// registers first); the scaled T copies overlay each A tile when they fit.
template <typename Op, int D, int C, bool FUSE, int G>
struct PrepLDS {
  using K = Cfg<Op, D, C>;
  static constexpr int S = (int)sizeof(Op);
  static constexpr int ROWS = C * K::LDR * S;       // one [C][LDR] row tile
  static constexpr int ATILE = C * K::LDA * 4;      // one fp32 A/T tile
  static constexpr int TTILE = C * K::LDT * S;      // the scaled T copy of W
  static constexpr int KR = 0;
  static constexpr int QR = ROWS;                   // fused-input only
  static constexpr int VR = 2 * ROWS;               // fused-input only, + s * ROWS
  static constexpr int A0 = FUSE ? QR : ROWS;       // + s * ATILE
  static constexpr int END_ROWS = FUSE ? (2 + G) * ROWS : ROWS;
  static constexpr int END_A = A0 + G * ATILE;
  // r_k [C], then per head G, b, f_K, f_W [C] each
  static constexpr int SM = (END_ROWS > END_A ? END_ROWS : END_A);
  static constexpr int SMALL = (1 + 4 * G) * C * 4;
  static constexpr bool T_OVER_A = TTILE <= ATILE;
  static constexpr int T0 = T_OVER_A ? A0 : SM + SMALL;  // + s * (T_OVER_A ? ATILE : TTILE)
  static constexpr int TSTEP = T_OVER_A ? ATILE : TTILE;
  static constexpr int BYTES = T_OVER_A ? SM + SMALL : T0 + G * TSTEP;
};

// Per (chunk, QK head's group of G V heads).  Everything runs on the raw q, k,
// v of the chunk; the L2 norms enter as per-token factors
// r = 1/sqrt(|x|^2 + 1e-6), and per V head s (gates G_s, b_s):
//   A_ij  = b_i r_k[i] r_k[j] e^{G_i-G_j} (k_i.k_j), i > j;   T = (I + A)^{-1}
//   P_ij  = scale r_q[i] r_k[j] e^{G_i-G_j} (q_i.k_j), i >= j
//   W     = T diag(b e^G r_k) K,   Ut = T diag(b) V,   K' = diag(e^{G_n-G} r_k) K
// and f_q = scale e^G r_q, which the output pass applies to Q S^T.  The raw
// products k_i.k_j and q_i.k_j and the loads (or convolutions) of q and k are
// shared by the G V heads of the QK head.
// No fragment is ever read down an LDS column.  P is formed as P^T = K Q^T,
// whose accumulator layout is P's A-fragment layout; W is formed as
// W^T = K^T (T diag(..))^T, whose accumulator layout is W's A-fragment layout;
// K and V blocks reach the column (B operand) layout through one MFMA with an
// identity operand, which is exact.  Only k (and, fused-input, q and v) is
// staged in LDS; otherwise each wave loads its q blocks and v tiles as
// register fragments.
template <typename T, typename Op, int D, int C, bool FUSE = false, int W = 4, int G = 1>
__global__ __launch_bounds__(kThreads<D>) void chunk_prep_kernel(
    const T* __restrict__ qkv, const float* __restrict__ g_in, const float* __restrict__ beta_in,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const int32_t* __restrict__ cstart,
    int32_t n_slots, int32_t n_seq, int64_t t_total, int32_t h_k, int32_t h_v, float scale,
    unsigned char* __restrict__ ws, ConvIn conv, GateIn gate, const uint8_t* __restrict__ has_init, int32_t q_out) {
  static_assert(sizeof(T) == sizeof(Op), "raw activations are MFMA operands");
  using K = Cfg<Op, D, C>;
  using L = PrepLDS<Op, D, C, FUSE, G>;
  using FragT = typename Frag<Op>::type;
  constexpr int NT = K::NT, CT = K::CT, WAVES = K::WAVES, DVT = K::DVT, LPR = K::LPR, RPP = K::RPP, RPT = K::RPT;
  constexpr int NPD = K::NPD, NPC = K::NPC, LDR = K::LDR, LDA = K::LDA, LDT = K::LDT;
  constexpr int QB = (CT + WAVES - 1) / WAVES;  // q blocks per wave: blocks wave, wave + WAVES, ...
  constexpr uint32_t PB = K::PAIR * sizeof(Op);
  static_assert(DVT == 1 || DVT == 2, "a wave's d tiles form one pair fragment");
  static_assert(G >= 1 && G <= 2, "V heads per workgroup");
  static_assert(L::BYTES <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
  Op* sK = reinterpret_cast<Op*>(smem + L::KR);
  float* sRK = reinterpret_cast<float*>(smem + L::SM);
  // per V head s (s may be a runtime value: addresses, not pointer arrays)
  auto sA = [&](int s) { return reinterpret_cast<float*>(smem + L::A0 + s * L::ATILE); };
  auto sG = [&](int s) { return sRK + C + 4 * s * C; };
  auto sB = [&](int s) { return sRK + 2 * C + 4 * s * C; };
  auto sFW = [&](int s) { return sRK + 4 * C + 4 * s * C; };  // b_t e^{G_t} r_k[t]
  auto sTW = [&](int s) { return reinterpret_cast<Op*>(smem + L::T0 + s * L::TSTEP); };

  const int hgroups = h_v / G;
  const int gc = blockIdx.x / hgroups;
  const int h0 = (blockIdx.x % hgroups) * G;  // first V head; G > 1 only when G == h_v / h_k
  int n;
  int32_t first;
  locate_chunk<C>(cstart, cu, n_seq, t_total, gc, n, first);
  if (n >= n_seq) return;
  if (!slot_ok(slots[n], n_slots)) return;  // padding entry: nothing to prepare
  const int hk = h0 / (h_v / h_k);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int c_ch = 2 * h_k * D + h_v * D;
  const int64_t seq_lo = min((int64_t)cu[n], t_total);
  const int64_t seq_hi = min(max((int64_t)cu[n + 1], seq_lo), t_total);
  const int64_t c0 = seq_lo + (int64_t)(gc - first) * C;
  const int nvalid = (int)min((int64_t)C, seq_hi - c0);
  auto unit = [&](int s) { return ws + ((int64_t)gc * h_v + h0 + s) * K::UNIT; };
  const uint32_t lp = lane * 8 * sizeof(Op), lf = lane * 4 * sizeof(Op);
  const FragT zf = zero_frag<Op>();
  FragT eye;  // B fragment of the 16x16 identity
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = from_f32<Op>(4 * g4 + i == l16 ? 1.f : 0.f);

  // gates of V head h0 + s into LDS (and e^{G_n} to its unit), on one wave:
  // from g, beta, or (fused-input) from a, b exactly as the gating kernel
  auto gates = [&](int s) {
    const int h = h0 + s;
    float gv = 0.f, bv = 0.f;
    if (lane < nvalid) {
      const int64_t i = (c0 + lane) * h_v + h;
      if constexpr (FUSE) {
        gv = -expf(gate.A_log[h]) * softplusf_(to_f32(reinterpret_cast<const T*>(gate.a)[i]) + gate.dt_bias[h]);
        bv = sigmoidf_(to_f32(reinterpret_cast<const T*>(gate.b)[i]));
      } else {
        gv = g_in[i];
        bv = beta_in[i];
      }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float up = __shfl_up(gv, off);
      if (lane >= off) gv += up;
    }
    if (lane < C) {
      sG(s)[lane] = gv;
      sB(s)[lane] = bv;
    }
    if (lane == C - 1) *at<float>(unit(s), K::F_OFF) = fast_exp(gv);
  };

  FragT Qb[QB][NPD][2], Va[G][CT][DVT];
  if constexpr (!FUSE) {
    // ---- register fragments straight from memory: this wave's q blocks (B
    // operand of P^T, row l16) and v tiles of each V head (A layout, row l16)
    {
      const T* qbase = qkv + (int64_t)hk * D + 4 * g4;
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int r = 16 * (wave + b * WAVES) + l16;
        const bool ok = wave + b * WAVES < CT && r < nvalid;
#pragma unroll
        for (int sp = 0; sp < NPD; ++sp) {
          Qb[b][sp][0] = ok ? *reinterpret_cast<const FragT*>(qbase + (c0 + r) * c_ch + 32 * sp) : zf;
          Qb[b][sp][1] = ok && 32 * sp + 16 < D ? *reinterpret_cast<const FragT*>(qbase + (c0 + r) * c_ch + 32 * sp + 16) : zf;
        }
      }
#pragma unroll
      for (int s = 0; s < G; ++s) {
        const T* vbase = qkv + (int64_t)(2 * h_k + h0 + s) * D + 16 * wave * DVT + 4 * g4;
#pragma unroll
        for (int kb = 0; kb < CT; ++kb)
#pragma unroll
          for (int j = 0; j < DVT; ++j) {
            const int r = 16 * kb + l16;
            Va[s][kb][j] = r < nvalid ? *reinterpret_cast<const FragT*>(vbase + (c0 + r) * c_ch + 16 * j) : zf;
          }
      }
    }
    // ---- raw k rows into LDS with their inverse norms; gates
    {
      const int e0 = (tid % LPR) * 8, r0 = tid / LPR;
      Raw8<T> raw[RPT];
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int r = r0 + j * RPP;
        if (r < nvalid) raw[j].load(qkv + (c0 + r) * c_ch + (int64_t)(h_k + hk) * D + e0);
        else raw[j].zero();
      }
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int r = r0 + j * RPP;
        float v[8];
        raw[j].to_f32(v);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
        ss = group_sum<LPR>(ss);
        if (r < C) {
          raw_store<Op>(*reinterpret_cast<const Raw8<Op>*>(&raw[j]), sK + r * LDR + e0);
          if (tid % LPR == 0) sRK[r] = fast_rsq(ss + 1e-6f);
        }
      }
#pragma unroll
      for (int s = 0; s < G; ++s)
        if (wave == s % WAVES) gates(s);
    }
    __syncthreads();
  } else {
    // ---- conv1d + SiLU of x into LDS: k and q of this QK head, v of each V head
    Op* sQf = reinterpret_cast<Op*>(smem + L::QR);
    {
      const int32_t slot = slots[n];
      const bool init = has_init == nullptr || has_init[n] != 0;
      const ConvIn ci{conv.x, conv.w, conv.bias, conv.state, (int64_t)slot * c_ch, init, seq_lo};
      // A sequence's first chunk keeps the old conv window of its q channels
      // in its units: the chain pass stores the new windows before the output
      // pass recomputes q.
      if (gc == first && init) {
        const T* cst = reinterpret_cast<const T*>(conv.state) + ((int64_t)slot * c_ch + hk * D) * (W - 1);
        for (int e = tid; e < D * (W - 1); e += K::THREADS) {
          const T v = cst[e];
#pragma unroll
          for (int s = 0; s < G; ++s) *at<T>(unit(s), K::HALO_OFF + e * (int)sizeof(T)) = v;
        }
      }
      // (destinations as element offsets from the LDS base, so the stores
      // stay LDS stores whichever part a thread's item falls in)
      int cols[2 + G], dst[2 + G];
      cols[0] = (h_k + hk) * D;
      dst[0] = L::KR / (int)sizeof(Op);
      cols[1] = hk * D;
      dst[1] = L::QR / (int)sizeof(Op);
#pragma unroll
      for (int s = 0; s < G; ++s) {
        cols[2 + s] = (2 * h_k + h0 + s) * D;
        dst[2 + s] = (L::VR + s * L::ROWS) / (int)sizeof(Op);
      }
      stage_conv<T, Op, D, C, W, 2 + G, 16, K::THREADS>(ci, c_ch, cols, c0, nvalid, reinterpret_cast<Op*>(smem), dst,
                                                        LDR, tid);
    }
    // gates on the waves with the fewest conv items (the last ones)
#pragma unroll
    for (int s = 0; s < G; ++s)
      if (wave == WAVES - 1 - s % WAVES) gates(s);
    __syncthreads();
    // the same fragments and norms as the unfused path, read from LDS
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int r = 16 * (wave + b * WAVES) + l16;
      const bool ok = wave + b * WAVES < CT && r < nvalid;
#pragma unroll
      for (int sp = 0; sp < NPD; ++sp) {
        Qb[b][sp][0] = ok ? lds_frag<Op>(sQf + r * LDR + 32 * sp + 4 * g4) : zf;
        Qb[b][sp][1] = ok && 32 * sp + 16 < D ? lds_frag<Op>(sQf + r * LDR + 32 * sp + 16 + 4 * g4) : zf;
      }
    }
#pragma unroll
    for (int s = 0; s < G; ++s) {
      const Op* sVf = reinterpret_cast<const Op*>(smem + L::VR + s * L::ROWS);
#pragma unroll
      for (int kb = 0; kb < CT; ++kb)
#pragma unroll
        for (int j = 0; j < DVT; ++j) {
          const int r = 16 * kb + l16;
          Va[s][kb][j] = r < nvalid ? lds_frag<Op>(sVf + r * LDR + 16 * (wave * DVT + j) + 4 * g4) : zf;
        }
    }
    {
      const int e0 = (tid % LPR) * 8, r0 = tid / LPR;
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int r = r0 + j * RPP;
        float v[8];
        if (r < C) load8(sK + r * LDR + e0, v);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.f;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
        ss = group_sum<LPR>(ss);
        if (r < C && tid % LPR == 0) sRK[r] = fast_rsq(ss + 1e-6f);
      }
    }
    __syncthreads();  // r_k visible; q and v rows are read before the A tiles overlay them
  }

  // ---- for the chain that computes the output itself: the chunk's raw q
  // rows as A-operand pairs [C/16][D/32], once per QK head, in the S^T area of
  // the unit of its first V head (that chain writes no S^T)
  if (q_out && h0 % (h_v / h_k) == 0) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int ib = wave + b * WAVES;
      if (ib >= CT) break;
#pragma unroll
      for (int sp = 0; sp < NPD; ++sp)
        store_pair<Op>(at<Op>(unit(0), K::H_OFF + (uint32_t)(ib * NPD + sp) * PB + lp), Qb[b][sp][0], Qb[b][sp][1]);
    }
  }

  // ---- Gram work.  Wave w: the P^T tiles of its q blocks ib (pairs of
  // column blocks -> P fragments of each V head) and f_q of those rows; then
  // K K^T tiles -> A of each V head, taken in the order that evens out the
  // per-wave tile count.  Each raw product is formed once for the G V heads.
  {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int ib = wave + b * WAVES;
      if (ib >= CT) break;
      // r_q of row 16 ib + l16: the row's 32 pair values per lane, 4 lanes per row
      float ss = 0.f;
#pragma unroll
      for (int sp = 0; sp < NPD; ++sp)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = to_f32(Qb[b][sp][hh][e]);
            ss = fmaf(x, x, ss);
          }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const int i = 16 * ib + l16;
      const float fi = scale * fast_rsq(ss + 1e-6f);  // scale r_q[i]
      if (g4 == 0)
#pragma unroll
        for (int s = 0; s < G; ++s) *at<float>(unit(s), K::FQ_OFF + 4 * i) = fi * fast_exp(sG(s)[i]);
#pragma unroll
      for (int sp = 0; sp < NPC; ++sp) {
        if (2 * sp > ib) break;
        f32x4 raw[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int jb = 2 * sp + hh;
          raw[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (jb > ib) continue;
          const Op* arow = sK + (16 * jb + l16) * LDR + 4 * g4;
#pragma unroll
          for (int s2 = 0; s2 < NPD; ++s2) {
            if (32 * s2 + 16 < D)
              mma_k32(raw[hh], lds_frag<Op>(arow + 32 * s2), lds_frag<Op>(arow + 32 * s2 + 16), Qb[b][s2][0],
                      Qb[b][s2][1]);
            else
              mma_k16(raw[hh], lds_frag<Op>(arow + 32 * s2), Qb[b][s2][0]);
          }
        }
#pragma unroll
        for (int s = 0; s < G; ++s) {
          const float gi = sG(s)[i];
          FragT half[2], low[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const int jj = 16 * (2 * sp + hh) + 4 * g4 + ii;
              const float pv = 2 * sp + hh <= ib && i >= jj
                                   ? fi * sRK[jj] * fast_exp(fminf(gi - sG(s)[jj], 0.f)) * raw[hh][ii]
                                   : 0.f;
              half[hh][ii] = from_f32<Op>(pv);
              low[hh][ii] = from_f32<Op>(pv - to_f32(half[hh][ii]));
            }
          store_pair<Op>(at<Op>(unit(s), K::P_OFF + (uint32_t)(ib * NPC + sp) * PB + lp), half[0], half[1]);
          if constexpr (K::P_PARTS == 2)
            store_pair<Op>(at<Op>(unit(s), K::P_OFF + (uint32_t)((CT + ib) * NPC + sp) * PB + lp), low[0], low[1]);
        }
      }
    }
    // A tiles (ib, jb), jb <= ib: block row ib (ib + 1 tiles) goes to wave
    // CT - 1 - ib (mod WAVES), so with CT == WAVES every wave has CT + 1 tiles
    // in all (w + 1 P tiles and CT - w A tiles)
    for (int ib = CT - 1 - (int)wave; ib >= 0; ib -= WAVES)
#pragma unroll
      for (int jb = 0; jb < CT; ++jb) {
        if (jb > ib) break;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const Op* arow = sK + (16 * ib + l16) * LDR + 4 * g4;
        const Op* brow = sK + (16 * jb + l16) * LDR + 4 * g4;
#pragma unroll
        for (int s2 = 0; s2 < NPD; ++s2) {
          if (32 * s2 + 16 < D)
            mma_k32(acc, lds_frag<Op>(arow + 32 * s2), lds_frag<Op>(arow + 32 * s2 + 16), lds_frag<Op>(brow + 32 * s2),
                    lds_frag<Op>(brow + 32 * s2 + 16));
          else
            mma_k16(acc, lds_frag<Op>(arow + 32 * s2), lds_frag<Op>(brow + 32 * s2));
        }
        const int j = 16 * jb + l16;
        const float rj = sRK[j];
#pragma unroll
        for (int s = 0; s < G; ++s) {
          const float gj = sG(s)[j];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * ib + 4 * g4 + ii;
            sA(s)[i * LDA + j] = i > j ? sB(s)[i] * sRK[i] * rj * fast_exp(fminf(sG(s)[i] - gj, 0.f)) * acc[ii] : 0.f;
          }
        }
      }
  }
  __syncthreads();

  // per-token column factors of W (LDS) and K' (f_k, to the unit), once per (V head, token)
  for (int e = tid; e < G * C; e += K::THREADS) {
    const int s = e / C, t = e % C;
    const float gt = sG(s)[t], rk = sRK[t];
    *at<float>(unit(s), K::FK_OFF + 4 * t) = fast_exp(sG(s)[C - 1] - gt) * rk;
    sFW(s)[t] = sB(s)[t] * fast_exp(gt) * rk;
  }
  // ---- T = (I + A)^-1 in place, per V head.  (a) diagonal 16x16 blocks, one
  // lane per column
  if (tid < G * CT * 16) {
    const int s = tid / (CT * 16), b = (tid / 16) % CT, c = tid & 15;
    // the block's rows into registers first, so the substitution chain runs
    // on registers (16-byte reads; the upper triangle is read but unused)
    float blk[16][16];
#pragma unroll
    for (int r = 1; r < 16; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (4 * q < r)
          *reinterpret_cast<f32x4*>(&blk[r][4 * q]) = *reinterpret_cast<const f32x4*>(sA(s) + (16 * b + r) * LDA + 16 * b + 4 * q);
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == c ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) acc = fmaf(-blk[r][j], x[j], acc);
      x[r] = acc;
    }
    // every read of this block above precedes these writes in the wave's program order
#pragma unroll
    for (int r = 0; r < 16; ++r) sA(s)[(16 * b + r) * LDA + 16 * b + c] = x[r];
  }
  __syncthreads();
  // (b) block rows: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.  The A blocks of the
  // row are read into registers before any wave overwrites them with T.
#pragma unroll
  for (int bi = 1; bi < CT; ++bi) {
    f32x4 a_row[G][CT];
#pragma unroll
    for (int s = 0; s < G; ++s)
#pragma unroll
      for (int bk = 0; bk < CT; ++bk)
        if (bk < bi) a_row[s][bk] = lds_frag<float>(sA(s) + (16 * bi + l16) * LDA + 16 * bk + 4 * g4);
    __syncthreads();
    for (int it = wave; it < G * bi; it += WAVES) {
      const int s = it / bi, bj = it % bi;
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bk = 0; bk < CT; ++bk)
        if (bk >= bj && bk < bi) {
          f32x4 b;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) b[jj] = sA(s)[(16 * bk + 4 * g4 + jj) * LDA + 16 * bj + l16];
          f32x4 av = a_row[0][bk];
#pragma unroll
          for (int s2 = 1; s2 < G; ++s2)
            if (s == s2) av = a_row[s2][bk];
          mma_k16(X, av, b);
        }
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
      mma_k16(Y, lds_frag<float>(sA(s) + (16 * bi + l16) * LDA + 16 * bi + 4 * g4), X);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sA(s)[(16 * bi + 4 * g4 + jj) * LDA + 16 * bj + l16] = -Y[jj];
    }
    __syncthreads();
  }

  // ---- Ut = T diag(b) V (this wave's d tiles) straight from the fp32 T tile.  T can have large
  // entries of both signs (it inverts I + A), and Ut cancels them, so the
  // operand keeps T diag(b) to fp32 accuracy: in bf16 as a hi + lo pair, two
  // MFMAs per block.  (W's T diag(b e^G r_k) enters a product whose result the
  // chain and output passes combine with the state; one bf16 copy suffices.)
#pragma unroll
  for (int s = 0; s < G; ++s) {
    FragT Vc[CT][DVT];
#pragma unroll
    for (int kb = 0; kb < CT; ++kb)
#pragma unroll
      for (int j = 0; j < DVT; ++j) {
        f32x4 b = {0.f, 0.f, 0.f, 0.f};
        mma_k16(b, Va[s][kb][j], eye);
        Vc[kb][j] = frag_from<Op>(b);
      }
#pragma unroll
    for (int mt = 0; mt < CT; ++mt) {
      f32x4 uacc[DVT];
#pragma unroll
      for (int j = 0; j < DVT; ++j) uacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* trow = sA(s) + (16 * mt + l16) * LDA + 4 * g4;
#pragma unroll
      for (int s2 = 0; s2 < NPC; ++s2)
        if (2 * s2 <= mt) {
          const bool two = 2 * s2 + 1 <= mt;  // (block 2 s2 + 1 above the diagonal is zero)
          f32x4 t0 = lds_frag<float>(trow + 32 * s2), t1 = two ? lds_frag<float>(trow + 32 * s2 + 16) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            t0[i] *= sB(s)[32 * s2 + 4 * g4 + i];
            t1[i] *= two ? sB(s)[32 * s2 + 16 + 4 * g4 + i] : 0.f;
          }
#pragma unroll
          for (int j = 0; j < DVT; ++j) {
            const FragT v0 = Vc[2 * s2][j], v1 = two ? Vc[2 * s2 + 1][j] : zf;
            if constexpr (sizeof(Op) == 2) {
              const FragT h0 = frag_from<Op>(t0), h1 = frag_from<Op>(t1);
              f32x4 r0, r1;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                r0[i] = t0[i] - to_f32(h0[i]);
                r1[i] = t1[i] - to_f32(h1[i]);
              }
              mma_k32(uacc[j], h0, h1, v0, v1);
              mma_k32(uacc[j], frag_from<Op>(r0), frag_from<Op>(r1), v0, v1);
            } else {
              mma_k32(uacc[j], frag_from<Op>(t0), frag_from<Op>(t1), v0, v1);
            }
          }
        }
#pragma unroll
      for (int j = 0; j < DVT; ++j)
        *at<FragT>(unit(s), K::UT_OFF + (uint32_t)(mt * NT + wave * DVT + j) * PB / 2 + lf) = frag_from<Op>(uacc[j]);
    }
  }

  // ---- T_W = T diag(b e^G r_k) in the operand type, zero above the diagonal
  // blocks.  It may overlay T itself: all of T is read first.
  {
    constexpr int PER = (G * C * C / 4 + K::THREADS - 1) / K::THREADS;
    FragT tw[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + k * K::THREADS;
      if (e < G * C * C / 4) {
        const int s = e / (C * C / 4), er = e % (C * C / 4);
        const int r = er / (C / 4), c4 = (er % (C / 4)) * 4;
        const bool keep = (c4 >> 4) <= (r >> 4);
        const f32x4 t = keep ? *reinterpret_cast<const f32x4*>(sA(s) + r * LDA + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) tw[k][i] = from_f32<Op>(t[i] * sFW(s)[c4 + i]);
      }
    }
    if (L::T_OVER_A) __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + k * K::THREADS;
      if (e < G * C * C / 4) {
        const int s = e / (C * C / 4), er = e % (C * C / 4);
        const int r = er / (C / 4), c4 = (er % (C / 4)) * 4;
        *reinterpret_cast<FragT*>(sTW(s) + r * LDT + c4) = tw[k];
      }
    }
  }
  __syncthreads();

  // ---- this wave's d tiles of K as column (B operand) fragments; per V head
  // W^T and K^T
  FragT Kc[CT][DVT];
#pragma unroll
  for (int kb = 0; kb < CT; ++kb)
#pragma unroll
    for (int j = 0; j < DVT; ++j) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      mma_k16(a, lds_frag<Op>(sK + (16 * kb + l16) * LDR + 16 * (wave * DVT + j) + 4 * g4), eye);
      Kc[kb][j] = frag_from<Op>(a);
    }
  {
    const int sp_w = wave;  // the pair of d tiles this wave owns (DVT == 2), or pair 0 (DVT == 1)
#pragma unroll
    for (int s = 0; s < G; ++s) {
#pragma unroll
      for (int mt = 0; mt < CT; ++mt) {
        f32x4 wacc[DVT];
#pragma unroll
        for (int j = 0; j < DVT; ++j) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const Op* twrow = sTW(s) + (16 * mt + l16) * LDT + 4 * g4;
#pragma unroll
          for (int s2 = 0; s2 < NPC; ++s2)
            if (2 * s2 <= mt) {
              const bool two = 2 * s2 + 1 < CT;
              const FragT b0 = lds_frag<Op>(twrow + 32 * s2), b1 = two ? lds_frag<Op>(twrow + 32 * s2 + 16) : zf;
              mma_k32(acc, Kc[2 * s2][j], two ? Kc[2 * s2 + 1][j] : zf, b0, b1);
            }
          wacc[j] = acc;
        }
        store_pair<Op>(at<Op>(unit(s), K::W_OFF + (uint32_t)(mt * NPD + sp_w) * PB + lp), frag_from<Op>(wacc[0], -1.f),
                       DVT == 2 ? frag_from<Op>(wacc[DVT - 1], -1.f) : zf);
      }
      // raw K^T is the same for every V head of the QK head: stored once, in
      // the unit of the group's first V head, where the chain reads it
      if ((h0 + s) % (h_v / h_k) == 0) {
#pragma unroll
        for (int j = 0; j < DVT; ++j)
#pragma unroll
          for (int sp = 0; sp < NPC; ++sp) {
            store_pair<Op>(at<Op>(unit(s), K::KT_OFF + (uint32_t)((wave * DVT + j) * NPC + sp) * PB + lp),
                           Kc[2 * sp][j], 2 * sp + 1 < CT ? Kc[2 * sp + 1 < CT ? 2 * sp + 1 : 0][j] : zf);
          }
      }
    }
  }
}

// ----------------------------------------------------------------- state
// The chain of one sequence's chunks for one V head and NTW 16-wide tiles of
// d_v, on one workgroup of NPD waves (NPD = d_k / 32, at least one).  The rows
// of S^T[d_k][tiles] are split over the waves: wave w holds d_k tiles 2w and
// 2w + 1 in accumulators (lane: d_k rows 4g..4g+3 of each 16-block, d_v
// column l16), which is pair w of the B operand of every product over d_k.
// Per chunk:
//   h = bf16(S^T): each wave's pairs -> workspace and LDS;             barrier
//   U = Ut - W S^T: wave w the chunk row tiles w, w + NPD, ... with all of h
//       from LDS -> workspace (over Ut) and LDS;                         barrier
//   S^T <- e^{G_n} S^T + K^T (diag(f_k) U): each wave its d_k tiles, all of the
//       scaled U from LDS.
// A wave streams only the operand rows it uses (one row tile of -W and Ut,
// two of K^T), PD - 1 chunks ahead in registers, so a chunk's loads and its
// MFMA work are spread over the CU's four SIMDs; NTW tiles share each -W and
// K^T load.  Block order puts all tiles of one (sequence, head) on one XCD,
// so W and K^T reach that XCD's L2 once.
template <int D>
constexpr int kChainThreads = 64 * ((D / 16 + 1) / 2);  // one wave per h pair

template <typename Op, int D, int C, int NTW, int PD>
__global__ __launch_bounds__(kChainThreads<D>) void chunk_state_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const uint8_t* __restrict__ has_init,
    const int32_t* __restrict__ cstart, unsigned char* __restrict__ ws, float* __restrict__ state,
    int32_t n_slots, Op* __restrict__ o, int64_t t_total, int32_t n_seq, int32_t h_v, int32_t kt_group,
    const Op* __restrict__ conv_x, Op* __restrict__ conv_state, int32_t c_ch, int32_t conv_w) {
  using K = Cfg<Op, D, C>;
  using FragT = typename Frag<Op>::type;
  constexpr int NT = K::NT, CT = K::CT, NPD = K::NPD, NPC = K::NPC, NTILE = NT / NTW;
  constexpr int MW = NPD;                   // waves
  static_assert(64 * MW == kChainThreads<D>, "one wave per h pair");
  static_assert(PD >= 2, "a chunk's loads go to a stage other than its own");
  static_assert(NT % NTW == 0, "whole d_v tiles per workgroup");
  constexpr int SM = NT >= 2 ? 2 : 1;       // d_k tiles of S^T per wave
  constexpr int UPW = (CT + MW - 1) / MW;   // chunk row tiles of U per wave
  constexpr uint32_t PB = K::PAIR * sizeof(Op);  // bytes per pair tile
  __shared__ __attribute__((aligned(16))) Op sH[NPD][NTW][64 * 8];  // h, pairs
  __shared__ __attribute__((aligned(16))) Op sU[CT][NTW][64 * 4];   // U, accumulator layout
  const int xcd = blockIdx.x & 7, kq = blockIdx.x >> 3, tile = kq % NTILE;
  const int64_t grp = (int64_t)(kq / NTILE) * 8 + xcd;
  if (grp >= (int64_t)n_seq * h_v) return;
  const int n = (int)(grp / h_v), h = (int)(grp % h_v);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int64_t lo = min((int64_t)cu[n], t_total);
  const int64_t hi = min(max((int64_t)cu[n + 1], lo), t_total);
  const int32_t slot = slots[n];
  if (!slot_ok(slot, n_slots)) {  // padding entry: zero outputs (the output pass skips it)
    const int64_t o_ld = (int64_t)h_v * D;
    const int col0 = h * D + 16 * NTW * tile;
    for (int64_t e = tid; e < (hi - lo) * 16 * NTW; e += 64 * MW)
      o[(lo + e / (16 * NTW)) * o_ld + col0 + e % (16 * NTW)] = from_f32<Op>(0.f);
    return;
  }
  const bool init = has_init == nullptr || has_init[n] != 0;
  float* st_ptr = state + ((int64_t)slot * h_v + h) * D * D;
  const int32_t gc0 = first_chunk<C>(cstart, cu, n_seq, t_total, n);

  if (conv_x != nullptr) {
    // Fused-input prefill: the sequence's final conv window, the last W-1
    // rows of (old window ++ x), one channel per thread over the sequence's
    // workgroups.  Every read of the old windows (the prep pass) is done, and
    // the output pass takes its q halo from the units.
    const int wm1 = conv_w - 1;
    const int64_t len = hi - lo;
    const int stride = 64 * MW * h_v * NTILE;
    for (int c = (h * NTILE + tile) * 64 * MW + (int)tid; c < c_ch; c += stride) {
      Op* cs = conv_state + ((int64_t)slot * c_ch + c) * wm1;
      Op prev[kMaxConvW - 1], nw[kMaxConvW - 1];
#pragma unroll
      for (int j = 0; j < kMaxConvW - 1; ++j) prev[j] = j < wm1 && init && len < wm1 ? cs[j] : from_f32<Op>(0.f);
#pragma unroll
      for (int j = 0; j < kMaxConvW - 1; ++j) {
        const int64_t p = len - wm1 + j;  // position in the sequence; < 0 reaches into the old window
        Op v = from_f32<Op>(0.f);
#pragma unroll
        for (int t = 0; t < kMaxConvW - 1; ++t) v = t == wm1 + (int)p ? prev[t] : v;  // (no register index)
        nw[j] = j < wm1 && p >= 0 ? conv_x[(lo + p) * c_ch + c] : v;
      }
#pragma unroll
      for (int j = 0; j < kMaxConvW - 1; ++j)
        if (j < wm1) cs[j] = nw[j];
    }
  }

  f32x4 Sacc[SM][NTW];
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int mt = SM * wave + m, dv = 16 * (NTW * tile + j) + l16;
      if (init) {
        const float4 v = *reinterpret_cast<const float4*>(st_ptr + dv * D + 16 * mt + 4 * g4);
        Sacc[m][j] = f32x4{v.x, v.y, v.z, v.w};
      } else {
        Sacc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

  const uint32_t lp = lane * 8 * sizeof(Op);  // a lane's pair within a pair tile
  const uint32_t lf = lane * 4 * sizeof(Op);  // a lane's fragment within a 16x16 tile
  const int nch = (int)((hi - lo + C - 1) / C);
  // unit of chunk k of this sequence, clamped to the last one: loads past the
  // end re-read it, so every load is unconditional and the wait counts exact
  auto unit_of = [&](int k) { return ws + uniform_i64(((int64_t)(gc0 + min(k, nch - 1)) * h_v + h) * K::UNIT); };
  // K^T lives in the unit of the QK head's first V head (the same chunk)
  const int64_t kt_delta = -(int64_t)(h % kt_group) * K::UNIT;
  Pair<Op> wn[PD][UPW][NPD], kt[PD][SM][NPC];
  FragT ut[PD][UPW][NTW];
  f32x4 fk[PD][UPW];
  float egn[PD];
  // A stage's operands as NPIECE single vector loads: the -W rows, Ut, the
  // K^T rows, f_k of the U rows, e^{G_n}.
  constexpr int NW = UPW * NPD, NU = UPW * NTW, NK = SM * NPC, NPIECE = NW + NU + NK + UPW + 1;
  auto piece = [&](int s, const unsigned char* u, int j) {
    if (j < NW) {
      const int mt = min(wave + MW * (j / NPD), CT - 1);
      wn[s][j / NPD][j % NPD].load(at<Op>(u, K::W_OFF + (uint32_t)(mt * NPD + j % NPD) * PB + lp));
    } else if (j < NW + NU) {
      const int i = (j - NW) / NTW, jt = (j - NW) % NTW;
      const int mt = min(wave + MW * i, CT - 1);
      ut[s][i][jt] = *at<FragT>(u, K::UT_OFF + (uint32_t)(mt * NT + NTW * tile + jt) * PB / 2 + lf);
    } else if (j < NW + NU + NK) {
      const int m = (j - NW - NU) / NPC, sp = (j - NW - NU) % NPC;
      kt[s][m][sp].load(at<Op>(u + kt_delta, K::KT_OFF + (uint32_t)((SM * wave + m) * NPC + sp) * PB + lp));
    } else if (j < NPIECE - 1) {
      const int i = j - NW - NU - NK;
      const int mt = min(wave + MW * i, CT - 1);
      fk[s][i] = *at<f32x4>(u, K::FK_OFF + 4 * (16 * mt + 4 * g4));
    } else {
      egn[s] = *at<float>(u, K::F_OFF);
    }
  };
  const FragT zf = zero_frag<Op>();
  // One chunk from stage s (unit uc).  The NPIECE loads of stage ls (unit
  // ul: the chunk PD - 1 ahead) are threaded one at a time between this
  // chunk's MFMAs and LDS steps.  The CU's vector memory pipeline takes one
  // 64-lane 16-byte load per ~16 clocks, and the waves run in step between
  // barriers: issued in bursts the loads stall every wave together,
  // interleaved they stream while the MFMA and LDS work runs.
  auto step = [&](int s, unsigned char* uc, int ls, const unsigned char* ul) {
    int pc = 0;
    auto next_load = [&]() {
      if (pc < NPIECE) {
        __builtin_amdgcn_sched_barrier(0);
        piece(ls, ul, pc);
        __builtin_amdgcn_sched_barrier(0);
      }
      ++pc;
    };
    // h = S^T at the chunk start: this wave's pairs
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const FragT h0 = frag_from<Op>(Sacc[0][j]), h1 = SM > 1 ? frag_from<Op>(Sacc[SM - 1][j]) : zf;
      next_load();
      store_pair<Op>(at<Op>(uc, K::H_OFF + (uint32_t)(wave * NT + NTW * tile + j) * PB + lp), h0, h1);
      store_pair<Op>(&sH[wave][j][lane * 8], h0, h1);
    }
    next_load();
    __syncthreads();
    // U = Ut - W S^T for this wave's row tiles
    {
      Pair<Op> hp[NPD][NTW];
#pragma unroll
      for (int sp = 0; sp < NPD; ++sp)
#pragma unroll
        for (int j = 0; j < NTW; ++j) hp[sp][j].load(&sH[sp][j][lane * 8]);
      __builtin_amdgcn_sched_barrier(0);  // all of h requested before the first product
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        // (a wave past the last row tile, CT < NPD, computes on the clamped
        // tile it loaded and keeps nothing; its loads stay in step)
        const int mt = wave + MW * i;
        f32x4 acc[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[j][e] = to_f32(ut[s][i][j][e]);
#pragma unroll
        for (int sp = 0; sp < NPD; ++sp)
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            typename Frag<Op>::type b0, b1;
            hp[sp][j].split(b0, b1);
            wn[s][i][sp].mma(acc[j], b0, b1);
            next_load();
          }
        if (CT % MW == 0 || mt < CT) {
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            *at<FragT>(uc, K::UT_OFF + (uint32_t)(mt * NT + NTW * tile + j) * PB / 2 + lf) = frag_from<Op>(acc[j]);
            f32x4 su;
#pragma unroll
            for (int e = 0; e < 4; ++e) su[e] = acc[j][e] * fk[s][i][e];
            *reinterpret_cast<FragT*>(&sU[mt][j][lane * 4]) = frag_from<Op>(su);
          }
        }
      }
      // the decay of S^T does not wait for U
#pragma unroll
      for (int m = 0; m < SM; ++m)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) Sacc[m][j][e] *= egn[s];
    }
    __syncthreads();
    // S^T <- e^{G_n} S^T + K^T diag(f_k) U for this wave's d_k tiles
    {
      FragT uf[CT][NTW];
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int j = 0; j < NTW; ++j) uf[t][j] = *reinterpret_cast<const FragT*>(&sU[t][j][lane * 4]);
#pragma unroll
      for (int sp = 0; sp < NPC; ++sp)
#pragma unroll
        for (int m = 0; m < SM; ++m)
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            kt[s][m][sp].mma(Sacc[m][j], uf[2 * sp][j], 2 * sp + 1 < CT ? uf[2 * sp + 1][j] : zf);
            next_load();
          }
    }
#pragma unroll
    for (int j = 0; j < NPIECE; ++j) next_load();  // any left (small shapes)
  };
  // chunks 0 .. PD-2 into stages 0 .. PD-2 (in the loop's order, so the wait
  // counts at the loop head need no slack); chunk c runs from stage c % PD
  // and loads chunk c + PD - 1 into stage (c - 1) % PD
  if (nch > 0) {
#pragma unroll
    for (int s = 0; s < PD - 1; ++s)
#pragma unroll
      for (int j = 0; j < NPIECE; ++j) piece(s, unit_of(s), j);
  }
  int k = 0;
  for (; k + PD <= nch; k += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) step(s, unit_of(k + s), (s + PD - 1) % PD, unit_of(k + s + PD - 1));
  }
#pragma unroll
  for (int s = 0; s < PD - 1; ++s)  // the last nch % PD chunks (uniform over the workgroup)
    if (k + s < nch) step(s, unit_of(k + s), (s + PD - 1) % PD, unit_of(k + s + PD - 1));

#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int mt = SM * wave + m, dv = 16 * (NTW * tile + j) + l16;
      *reinterpret_cast<float4*>(st_ptr + dv * D + 16 * mt + 4 * g4) =
          make_float4(Sacc[m][j][0], Sacc[m][j][1], Sacc[m][j][2], Sacc[m][j][3]);
    }
}

// ---------------------------------------------------- chain with output
// Four consecutive activations of a row, raw (8 bytes of bf16, 16 of fp32).
template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
  uint2 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void zero() { u = make_uint2(0, 0); }
  __device__ __forceinline__ void to_f32(float* v) const {
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
  }
};
template <> struct Raw4<float> {
  float4 u;
  __device__ __forceinline__ void load(const float* p) { u = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void zero() { u = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void to_f32(float* v) const {
    v[0] = u.x;
    v[1] = u.y;
    v[2] = u.z;
    v[3] = u.w;
  }
};
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  const bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4*>(p) = b;
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Many chains at once: one workgroup per (sequence, V head) holds all of S^T
// and computes each chunk's output itself, so neither S^T at the chunk start
// nor U goes through the workspace and no output pass runs.  Wave w owns the
// chunk's row tile w (its rows of U and of O) and d_k tiles 2w, 2w + 1 of S^T.
// Per chunk:
//   h = bf16(S^T) -> LDS; the chunk's q rows, P, f_q and z are requested; barrier
//   U = Ut - W S^T for row tile w -> LDS twice (diag(f_k) U for the state
//   update, U for the output), and O^T = (h as A) x (q as B): the transposed
//   product, so a lane holds 4 consecutive d_v values of one token; times f_q;
//   barrier
//   S^T <- e^{G_n} S^T + K^T diag(f_k) U; O^T += (U as A) x (P as B), P's high
//   and low parts; the gated RMSNorm over d_v and 8-byte stores.
// The products, their operands (bf16 S^T, bf16 U) and their order are those of
// the chain and output kernels.  q is the prep pass's copy of the chunk's q
// rows, kept with K^T in the unit of the QK head's first V head; the V heads
// of a QK head run on one XCD.
template <typename T, typename Op, int D, int C, int PD>
__global__ __launch_bounds__(kChainThreads<D>) void chunk_chain_out_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const uint8_t* __restrict__ has_init,
    const int32_t* __restrict__ cstart, const int32_t* __restrict__ order, unsigned char* __restrict__ ws,
    float* __restrict__ state, int32_t n_slots, T* __restrict__ o, int64_t t_total, int32_t n_seq, int32_t h_v,
    int32_t kt_group, const T* __restrict__ z, const T* __restrict__ norm_w, float norm_eps, const Op* __restrict__ conv_x,
    Op* __restrict__ conv_state, int32_t c_ch, int32_t conv_w) {
  static_assert(sizeof(T) == sizeof(Op), "outputs in the activation type");
  using K = Cfg<Op, D, C>;
  using FragT = typename Frag<Op>::type;
  constexpr int NT = K::NT, CT = K::CT, NPD = K::NPD, NPC = K::NPC;
  constexpr int MW = NPD;                   // waves
  static_assert(64 * MW == kChainThreads<D>, "one wave per h pair");
  static_assert(CT <= MW, "one chunk row tile per wave");
  static_assert(PD >= 2, "a chunk's loads go to a stage other than its own");
  constexpr int SM = NT >= 2 ? 2 : 1;       // d_k tiles of S^T per wave
  constexpr uint32_t PB = K::PAIR * sizeof(Op);
  __shared__ __attribute__((aligned(16))) Op sH[NPD][NT][64 * 8];  // h, pairs
  __shared__ __attribute__((aligned(16))) Op sU[CT][NT][64 * 4];   // diag(f_k) U, accumulator layout
  __shared__ __attribute__((aligned(16))) Op sUo[CT][NT][64 * 4];  // U
  __shared__ __attribute__((aligned(16))) float sNW[D];             // norm weights
  // chain index: the kt_group V heads of a QK head on consecutive slots of one XCD
  const int xcd = blockIdx.x & 7, qb = blockIdx.x >> 3;
  const int64_t grp = ((int64_t)(qb / kt_group) * 8 + xcd) * kt_group + qb % kt_group;
  if (grp >= (int64_t)n_seq * h_v) return;
  // sequences longest first when the chunk index gives their order
  const int n = order ? order[grp / h_v] : (int)(grp / h_v), h = (int)(grp % h_v);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int64_t lo = min((int64_t)cu[n], t_total);
  const int64_t hi = min(max((int64_t)cu[n + 1], lo), t_total);
  const int32_t slot = slots[n];
  const int64_t o_ld = (int64_t)h_v * D;
  if (!slot_ok(slot, n_slots)) {  // padding entry: zero outputs
    for (int64_t e = tid; e < (hi - lo) * D; e += 64 * MW) o[(lo + e / D) * o_ld + h * D + e % D] = from_f32<T>(0.f);
    return;
  }
  const bool init = has_init == nullptr || has_init[n] != 0;
  float* st_ptr = state + ((int64_t)slot * h_v + h) * D * D;
  const int32_t gc0 = first_chunk<C>(cstart, cu, n_seq, t_total, n);

  if (conv_x != nullptr) {
    // fused-input prefill: the sequence's final conv window, one channel per
    // thread over the sequence's workgroups (the prep pass read the old ones)
    const int wm1 = conv_w - 1;
    const int64_t len = hi - lo;
    const int stride = 64 * MW * h_v;
    for (int c = h * 64 * MW + (int)tid; c < c_ch; c += stride) {
      Op* cs = conv_state + ((int64_t)slot * c_ch + c) * wm1;
      Op prev[kMaxConvW - 1], nw[kMaxConvW - 1];
#pragma unroll
      for (int j = 0; j < kMaxConvW - 1; ++j) prev[j] = j < wm1 && init && len < wm1 ? cs[j] : from_f32<Op>(0.f);
#pragma unroll
      for (int j = 0; j < kMaxConvW - 1; ++j) {
        const int64_t p = len - wm1 + j;
        Op v = from_f32<Op>(0.f);
#pragma unroll
        for (int t = 0; t < kMaxConvW - 1; ++t) v = t == wm1 + (int)p ? prev[t] : v;  // (no register index)
        nw[j] = j < wm1 && p >= 0 ? conv_x[(lo + p) * c_ch + c] : v;
      }
#pragma unroll
      for (int j = 0; j < kMaxConvW - 1; ++j)
        if (j < wm1) cs[j] = nw[j];
    }
  }

  f32x4 Sacc[SM][NT];
#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt = SM * wave + m, dv = 16 * j + l16;
      if (init) {
        const float4 v = *reinterpret_cast<const float4*>(st_ptr + dv * D + 16 * mt + 4 * g4);
        Sacc[m][j] = f32x4{v.x, v.y, v.z, v.w};
      } else {
        Sacc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

  const uint32_t lp = lane * 8 * sizeof(Op);
  const uint32_t lf = lane * 4 * sizeof(Op);
  const int nch = (int)((hi - lo + C - 1) / C);
  auto unit_of = [&](int k) { return ws + uniform_i64(((int64_t)(gc0 + min(k, nch - 1)) * h_v + h) * K::UNIT); };
  const int64_t kt_delta = -(int64_t)(h % kt_group) * K::UNIT;  // the QK head's first V head (K^T, q)
  const int mt = min(wave, CT - 1);  // this wave's chunk row tile (waves past CT keep nothing)
  const bool rows = wave < CT;
  Pair<Op> wn[PD][NPD], kt[PD][SM][NPC];
  FragT ut[PD][NT];
  f32x4 fk[PD];
  float egn[PD];
  constexpr int NW = NPD, NU = NT, NK = SM * NPC, NPIECE = NW + NU + NK + 2;
  auto piece = [&](int s, const unsigned char* u, int j) {
    if (j < NW) {
      wn[s][j].load(at<Op>(u, K::W_OFF + (uint32_t)(mt * NPD + j) * PB + lp));
    } else if (j < NW + NU) {
      ut[s][j - NW] = *at<FragT>(u, K::UT_OFF + (uint32_t)(mt * NT + (j - NW)) * PB / 2 + lf);
    } else if (j < NW + NU + NK) {
      const int m = (j - NW - NU) / NPC, sp = (j - NW - NU) % NPC;
      kt[s][m][sp].load(at<Op>(u + kt_delta, K::KT_OFF + (uint32_t)((SM * wave + m) * NPC + sp) * PB + lp));
    } else if (j < NPIECE - 1) {
      fk[s] = *at<f32x4>(u, K::FK_OFF + 4 * (16 * mt + 4 * g4));
    } else {
      egn[s] = *at<float>(u, K::F_OFF);
    }
  };
  const FragT zf = zero_frag<Op>();
  // the norm weights in LDS (read after the first chunk's barriers): a load
  // of them in the epilogue would wait for the output stores issued before it
  if (z)
    for (int e = (int)tid; e < D; e += 64 * MW) sNW[e] = to_f32(norm_w[e]);
  auto step = [&](int s, unsigned char* uc, int ls, const unsigned char* ul, int k) {
    int pc = 0;
    auto next_load = [&]() {
      if (pc < NPIECE) {
        __builtin_amdgcn_sched_barrier(0);
        piece(ls, ul, pc);
        __builtin_amdgcn_sched_barrier(0);
      }
      ++pc;
    };
    // this chunk's output operands for row tile mt
    const int64_t c0 = lo + (int64_t)k * C;
    const int row = 16 * mt + (int)l16;  // this lane's token within the chunk
    const bool live = rows && c0 + row < hi;
    Pair<Op> qp[NPD], pa[NPC], pl[NPC];
#pragma unroll
    for (int sp = 0; sp < NPD; ++sp) qp[sp].load(at<Op>(uc + kt_delta, K::H_OFF + (uint32_t)(mt * NPD + sp) * PB + lp));
#pragma unroll
    for (int sp = 0; sp < NPC; ++sp)
      if (2 * sp <= mt) {
        pa[sp].load(at<Op>(uc, K::P_OFF + (uint32_t)(mt * NPC + sp) * PB + lp));
        if constexpr (K::P_PARTS == 2) pl[sp].load(at<Op>(uc, K::P_OFF + (uint32_t)((CT + mt) * NPC + sp) * PB + lp));
      }
    const float fq = *at<float>(uc, K::FQ_OFF + 4 * row);
    Raw4<T> zr[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (z && live) zr[j].load(z + (c0 + row) * o_ld + h * D + 16 * j + 4 * g4);
      else zr[j].zero();
    }
    // h = S^T at the chunk start: this wave's pairs
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const FragT h0 = frag_from<Op>(Sacc[0][j]), h1 = SM > 1 ? frag_from<Op>(Sacc[SM - 1][j]) : zf;
      next_load();
      store_pair<Op>(&sH[wave][j][lane * 8], h0, h1);
    }
    next_load();
    __syncthreads();
    // U = Ut - W S^T and O^T = h^T q^T for row tile mt, one d_v tile at a time
    f32x4 Oacc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      f32x4 acc, oac = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = to_f32(ut[s][j][e]);
#pragma unroll
      for (int sp = 0; sp < NPD; ++sp) {
        Pair<Op> hp;
        hp.load(&sH[sp][j][lane * 8]);
        FragT b0, b1, q0, q1;
        hp.split(b0, b1);
        qp[sp].split(q0, q1);
        wn[s][sp].mma(acc, b0, b1);
        mma_k32(oac, b0, b1, q0, q1);
        next_load();
      }
      if (rows) {
        f32x4 su;
#pragma unroll
        for (int e = 0; e < 4; ++e) su[e] = acc[e] * fk[s][e];
        *reinterpret_cast<FragT*>(&sU[mt][j][lane * 4]) = frag_from<Op>(su);
        *reinterpret_cast<FragT*>(&sUo[mt][j][lane * 4]) = frag_from<Op>(acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Oacc[j][e] = oac[e] * fq;  // scale e^{G_t} r_q[t] on Q S^T only
    }
    // the decay of S^T does not wait for U
#pragma unroll
    for (int m = 0; m < SM; ++m)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[m][j][e] *= egn[s];
    __syncthreads();
    // S^T <- e^{G_n} S^T + K^T diag(f_k) U; O^T += U^T P^T
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      FragT uf[CT];
#pragma unroll
      for (int t = 0; t < CT; ++t) uf[t] = *reinterpret_cast<const FragT*>(&sU[t][j][lane * 4]);
#pragma unroll
      for (int sp = 0; sp < NPC; ++sp)
#pragma unroll
        for (int m = 0; m < SM; ++m) {
          kt[s][m][sp].mma(Sacc[m][j], uf[2 * sp], 2 * sp + 1 < CT ? uf[2 * sp + 1] : zf);
          next_load();
        }
      if (rows) {
#pragma unroll
        for (int t = 0; t < CT; ++t) uf[t] = *reinterpret_cast<const FragT*>(&sUo[t][j][lane * 4]);
#pragma unroll
        for (int sp = 0; sp < NPC; ++sp)
          if (2 * sp <= mt) {
            FragT p0, p1;
            const FragT u1 = 2 * sp + 1 < CT ? uf[2 * sp + 1] : zf;
            pa[sp].split(p0, p1);
            mma_k32(Oacc[j], uf[2 * sp], u1, p0, p1);
            if constexpr (K::P_PARTS == 2) {
              pl[sp].split(p0, p1);
              mma_k32(Oacc[j], uf[2 * sp], u1, p0, p1);
            }
          }
      }
    }
#pragma unroll
    for (int j = 0; j < NPIECE; ++j) next_load();  // any left (small shapes)
    // gated RMSNorm over d_v: this lane's 4 x NT values of its token, the rest
    // of the row in the lanes of the other three lane groups
    if (rows) {
      if (z) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = fmaf(Oacc[j][e], Oacc[j][e], ss);
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float rstd = fast_rsq(ss * (1.0f / D) + norm_eps);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          float zz[4], v[4];
          zr[j].to_f32(zz);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = Oacc[j][e] * rstd * sNW[16 * j + 4 * g4 + e] * fast_silu(zz[e]);
          if (live) store4(o + (c0 + row) * o_ld + h * D + 16 * j + 4 * g4, v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          float v[4] = {Oacc[j][0], Oacc[j][1], Oacc[j][2], Oacc[j][3]};
          if (live) store4(o + (c0 + row) * o_ld + h * D + 16 * j + 4 * g4, v);
        }
      }
    }
  };
  if (nch > 0) {
#pragma unroll
    for (int s = 0; s < PD - 1; ++s)
#pragma unroll
      for (int j = 0; j < NPIECE; ++j) piece(s, unit_of(s), j);
  }
  int k = 0;
  for (; k + PD <= nch; k += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) step(s, unit_of(k + s), (s + PD - 1) % PD, unit_of(k + s + PD - 1), k + s);
  }
#pragma unroll
  for (int s = 0; s < PD - 1; ++s)  // the last nch % PD chunks (uniform over the workgroup)
    if (k + s < nch) step(s, unit_of(k + s), (s + PD - 1) % PD, unit_of(k + s + PD - 1), k + s);

#pragma unroll
  for (int m = 0; m < SM; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int mt2 = SM * wave + m, dv = 16 * j + l16;
      *reinterpret_cast<float4*>(st_ptr + dv * D + 16 * mt2 + 4 * g4) =
          make_float4(Sacc[m][j][0], Sacc[m][j][1], Sacc[m][j][2], Sacc[m][j][3]);
    }
}

// ------------------------------------------------------------------ output
// Per (chunk, V head): O = diag(f_q) Q h^T + P U (the scale is in f_q and P); with z,
// out = O / sqrt(mean_dv(O^2) + eps) * w * silu(z).  Wave w computes d_v
// tiles w*DVT .. w*DVT+DVT-1 for all C rows with every operand load issued up
// front; the fp32 tile then goes through LDS so the norm and the z / out
// traffic run row-wise, 8 consecutive elements (16 bytes of bf16) per lane.
template <typename T, typename Op, int D, int C, bool FUSE = false, int W = 4>
__global__ __launch_bounds__(kThreads<D>) __attribute__((amdgpu_waves_per_eu(3))) void chunk_out_kernel(
    const T* __restrict__ qkv, const int32_t* __restrict__ cu, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ cstart, const unsigned char* __restrict__ ws, int32_t n_slots, int32_t n_seq,
    int64_t t_total, int32_t h_k, int32_t h_v, T* __restrict__ o, const T* __restrict__ z,
    const T* __restrict__ norm_w, float norm_eps, ConvIn conv, const uint8_t* __restrict__ has_init) {
  static_assert(sizeof(T) == sizeof(Op), "raw q rows are MFMA operands");
  using K = Cfg<Op, D, C>;
  using FragT = typename Frag<Op>::type;
  constexpr int NT = K::NT, CT = K::CT, NPD = K::NPD, NPC = K::NPC, DVT = K::DVT, LD_O = K::LD_O;
  constexpr int LPR = K::LPR, RPP = K::RPP, RPT = K::RPT;
  constexpr uint32_t PB = K::PAIR * sizeof(Op);
  __shared__ __attribute__((aligned(16))) float sO[K::OUT_BYTES / 4];
  const int gc = blockIdx.x / h_v;
  const int h = blockIdx.x % h_v;
  int n;
  int32_t first;
  locate_chunk<C>(cstart, cu, n_seq, t_total, gc, n, first);
  if (n >= n_seq) return;
  if (!slot_ok(slots[n], n_slots)) return;  // the chain zeroed this sequence's outputs
  const uint32_t tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int64_t seq_lo = min((int64_t)cu[n], t_total);
  const int64_t seq_hi = min(max((int64_t)cu[n + 1], seq_lo), t_total);
  const int64_t c0 = seq_lo + (int64_t)(gc - first) * C;
  const int nvalid = (int)min((int64_t)C, seq_hi - c0);
  const unsigned char* u = ws + ((int64_t)gc * h_v + h) * K::UNIT;
  const uint32_t lp = lane * 8 * sizeof(Op), lf = lane * 4 * sizeof(Op);
  const FragT zf = zero_frag<Op>();

  // ---- all operand loads.  Fused-input: U, f_q and z are requested before
  // the q conv staging so their latency overlaps it, h and P after it (the
  // staging's taps and windows leave no registers for them).  Otherwise the
  // q rows go first, then every operand.
  Pair<Op> hp[NPD][DVT], pa[CT][NPC], pl[CT][NPC];  // (pl: P's low part, bf16 operands only)
  FragT Uf[CT][DVT];
  f32x4 fq[CT];
  Raw8<T> zr[RPT];  // this thread's z pieces of the epilogue rows
  const int64_t o_ld = (int64_t)h_v * D;
  const int e0 = (tid % LPR) * 8;
  auto load_hp = [&]() {
#pragma unroll
    for (int sp = 0; sp < NPD; ++sp)
#pragma unroll
      for (int j = 0; j < DVT; ++j)
        hp[sp][j].load_nt(at<Op>(u, K::H_OFF + (uint32_t)(sp * NT + wave * DVT + j) * PB + lp));
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int sp = 0; sp < NPC; ++sp)
        if (2 * sp <= mt) {
          pa[mt][sp].load_nt(at<Op>(u, K::P_OFF + (uint32_t)(mt * NPC + sp) * PB + lp));
          if constexpr (K::P_PARTS == 2)
            pl[mt][sp].load_nt(at<Op>(u, K::P_OFF + (uint32_t)((CT + mt) * NPC + sp) * PB + lp));
        }
  };
  auto load_uz = [&]() {
#pragma unroll
    for (int mt = 0; mt < CT; ++mt) fq[mt] = *at<f32x4>(u, K::FQ_OFF + 4 * (16 * mt + 4 * g4));
#pragma unroll
    for (int mt = 0; mt < CT; ++mt)
#pragma unroll
      for (int j = 0; j < DVT; ++j)
        Uf[mt][j] = nt_ld(at<FragT>(u, K::UT_OFF + (uint32_t)(mt * NT + wave * DVT + j) * PB / 2 + lf));
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int r = (int)(tid / LPR) + k * RPP;
      if (z && r < nvalid) zr[k].load_nt(z + (c0 + r) * o_ld + h * D + e0);
      else zr[k].zero();
    }
  };

  // q rows of the chunk into LDS, 16-byte pieces: raw from qkv, or conv1d +
  // SiLU of x in the fused-input mode
  Op* sQ = reinterpret_cast<Op*>(sO);
  if constexpr (FUSE) {
    load_uz();
    const int hk = h / (h_v / h_k);
    const int c_ch = 2 * h_k * D + h_v * D;
    // the window before the sequence start: the old q window the prep pass
    // kept in this (first) chunk's unit, indexed like the conv state
    const ConvIn ci{conv.x, conv.w, conv.bias, u + K::HALO_OFF, -(int64_t)hk * D,
                    has_init == nullptr || has_init[n] != 0, seq_lo};
    const int cols[1] = {hk * D}, dst[1] = {0};
    stage_conv<T, Op, D, C, W, 1, 4, K::THREADS>(ci, c_ch, cols, c0, nvalid, sQ, dst, K::LD_Q, (int)tid);
    load_hp();
  } else {
    const int hk = h / (h_v / h_k);
    const int c_ch = 2 * h_k * D + h_v * D;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int r = (int)(tid / LPR) + k * RPP;
      if (r < C) {
        Raw8<T> q;
        if (r < nvalid) q.load(qkv + (c0 + r) * c_ch + (int64_t)hk * D + e0);
        else q.zero();
        raw_store<Op>(*reinterpret_cast<const Raw8<Op>*>(&q), sQ + r * K::LD_Q + e0);
      }
    }
    load_hp();
    load_uz();
  }
  __syncthreads();

  // ---- O = diag(f_q) Q h^T + P U
  f32x4 Oacc[CT][DVT];
#pragma unroll
  for (int mt = 0; mt < CT; ++mt)
#pragma unroll
    for (int j = 0; j < DVT; ++j) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const Op* qrow = sQ + (16 * mt + l16) * K::LD_Q + 4 * g4;
#pragma unroll
      for (int sp = 0; sp < NPD; ++sp) {
        FragT b0, b1;
        hp[sp][j].split(b0, b1);
        if (32 * sp + 16 < D) mma_k32(acc, lds_frag<Op>(qrow + 32 * sp), lds_frag<Op>(qrow + 32 * sp + 16), b0, b1);
        else mma_k16(acc, lds_frag<Op>(qrow + 32 * sp), b0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= fq[mt][i];  // scale e^{G_t} r_q[t] on Q S^T only
#pragma unroll
      for (int sp = 0; sp < NPC; ++sp)
        if (2 * sp <= mt) {
          pa[mt][sp].mma(acc, Uf[2 * sp][j], 2 * sp + 1 < CT ? Uf[2 * sp + 1][j] : zf);
          if constexpr (K::P_PARTS == 2) pl[mt][sp].mma(acc, Uf[2 * sp][j], 2 * sp + 1 < CT ? Uf[2 * sp + 1][j] : zf);
        }
      Oacc[mt][j] = acc;
    }
  __syncthreads();  // q is read; the O tile goes over it
#pragma unroll
  for (int mt = 0; mt < CT; ++mt)
#pragma unroll
    for (int j = 0; j < DVT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sO[(16 * mt + 4 * g4 + i) * LD_O + 16 * (wave * DVT + j) + l16] = Oacc[mt][j][i];
  __syncthreads();

  // ---- row-wise: gated RMSNorm and 16-byte stores
  float w[8];
  if (z) load8(norm_w + e0, w);
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int r = (int)(tid / LPR) + k * RPP;
    if (r >= C) break;  // uniform over the LPR lanes of a row
    float v[8];
    // (lanes 8..15 of a row take their second half first: the 16 lanes' first
    // reads then cover 64 distinct banks)
    const bool hi_first = (tid & 8) != 0;
    const float4 first = *reinterpret_cast<const float4*>(sO + r * LD_O + e0 + (hi_first ? 4 : 0));
    const float4 second = *reinterpret_cast<const float4*>(sO + r * LD_O + e0 + (hi_first ? 0 : 4));
    const float4 lo4 = hi_first ? second : first, hi4 = hi_first ? first : second;
    v[0] = lo4.x; v[1] = lo4.y; v[2] = lo4.z; v[3] = lo4.w;
    v[4] = hi4.x; v[5] = hi4.y; v[6] = hi4.z; v[7] = hi4.w;
    const bool live = r < nvalid;
    const int64_t off = (c0 + r) * o_ld + h * D + e0;
    if (z) {
      float zz[8];
      zr[k].to_f32(zz);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
      ss = group_sum<LPR>(ss);
      const float rstd = fast_rsq(ss * (1.0f / D) + norm_eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] * rstd * w[e] * fast_silu(zz[e]);
    }
    if (live) store8_nt(o + off, v);
  }
}

// (conv_x non-null: the fused-input prefill, whose chain also stores the
// final conv windows)
template <typename Op, int D, int C, int NTW, int PD>
hipError_t launch_chain(const ChunkArgs& a, int64_t groups, const int32_t* cstart, unsigned char* units,
                        const Op* conv_x, hipStream_t st) {
  constexpr int TW = Cfg<Op, D, C>::NT >= NTW ? NTW : Cfg<Op, D, C>::NT;
  hipLaunchKernelGGL((chunk_state_kernel<Op, D, C, TW, PD>), dim3((unsigned)(groups * (Cfg<Op, D, C>::NT / TW))),
                     dim3(kChainThreads<D>), 0, st, a.cu_seqlens, a.slots, a.has_init, cstart, units, a.state,
                     a.n_slots, (Op*)a.o, a.t_total, a.n_seq, a.s.h_v, a.s.h_v / a.s.h_k, conv_x,
                     (Op*)const_cast<void*>(a.conv_state), a.s.c_ch(), a.s.conv_w);
  return hipGetLastError();
}

// The chain that computes the output itself: one workgroup per chain, the
// kt_group V heads of a QK head on one XCD.
template <typename T, typename Op, int D, int C, int PD>
hipError_t launch_chain_out(const ChunkArgs& a, const int32_t* cstart, unsigned char* units, const Op* conv_x,
                            hipStream_t st) {
  const int g = a.s.h_v / a.s.h_k;
  const int64_t chains = (int64_t)a.n_seq * a.s.h_v;
  const int64_t blocks = (chains + 8 * g - 1) / (8 * g) * 8 * g;
  const int32_t* order = cstart ? cstart + a.n_seq + 1 : nullptr;
  hipLaunchKernelGGL((chunk_chain_out_kernel<T, Op, D, C, PD>), dim3((unsigned)blocks), dim3(kChainThreads<D>), 0, st,
                     a.cu_seqlens, a.slots, a.has_init, cstart, order, units, a.state, a.n_slots, (T*)a.o, a.t_total,
                     a.n_seq, a.s.h_v, g, (const T*)a.z, (const T*)a.norm_w, a.norm_eps, conv_x,
                     (Op*)const_cast<void*>(a.conv_state), a.s.c_ch(), a.s.conv_w);
  return hipGetLastError();
}

// A launch-table shape: NTW d_v tiles per chain workgroup, or (NTW = 8, all of
// d_v at the layer's head dim) the chain that computes the output itself when
// every chunk row tile has its own wave; else the widest split chain.
// (bf16 only: the fp32 mode's operands do not fit its registers)
template <typename Op, int D, int C>
constexpr bool chain_out_fits(int ntw) {
  return ntw >= 8 && sizeof(Op) == 2 && Cfg<Op, D, C>::CT <= Cfg<Op, D, C>::NPD;
}
template <typename T, typename Op, int D, int C, int NTW, int PD>
hipError_t launch_shape(const ChunkArgs& a, int64_t groups, const int32_t* cstart, unsigned char* units,
                        const Op* conv_x, hipStream_t st) {
  if constexpr (chain_out_fits<Op, D, C>(NTW)) return launch_chain_out<T, Op, D, C, PD>(a, cstart, units, conv_x, st);
  else return launch_chain<Op, D, C, (NTW >= 8 ? 4 : NTW), PD>(a, groups, cstart, units, conv_x, st);
}

// workspace: [chunk index: cstart (n_seq + 1), order (n_seq)][units]
inline size_t idx_bytes(int32_t n_seq) { return ((2 * (size_t)n_seq + 1) * 4 + 255) / 256 * 256; }

template <typename T, typename Op, int D, int C>
size_t ws_bytes(int32_t n_seq, int64_t t_total, int32_t h_v) {
  using K = Cfg<Op, D, C>;
  const int64_t max_chunks = t_total / C + n_seq;
  return idx_bytes(n_seq) + (size_t)max_chunks * h_v * K::UNIT;
}

// One split-path call: chunk index (more than kScanSeqs sequences), prep,
// chain, output; FUSE computes q, k, v (conv1d + SiLU of a.x, width W) and
// g, beta (from a.a_in, a.b_in) in the prep and output kernels, and stores
// the final conv windows in the chain kernel.
template <typename T, typename Op, int D, int C, bool FUSE = false, int W = 4>
hipError_t run(const ChunkArgs& a, hipStream_t st) {
  using K = Cfg<Op, D, C>;
  static_assert(sizeof(T) == sizeof(Op), "the chain writes O in the activation type");
  static_assert(W <= kMaxConvW, "conv window");
  if (a.n_seq == 0) return hipSuccess;
  int32_t* cstart = a.n_seq > kScanSeqs ? reinterpret_cast<int32_t*>(a.workspace) : nullptr;
  unsigned char* units = reinterpret_cast<unsigned char*>(a.workspace) + idx_bytes(a.n_seq);
  if (cstart) {
    hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.n_seq, a.t_total, (int32_t)C,
                       cstart, cstart + a.n_seq + 1);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const int64_t max_chunks = a.t_total / C + a.n_seq;
  // the chain's launch shape from the measured table (launch_table.hpp): one
  // d_v tile per workgroup is the most parallel chain, more tiles per
  // workgroup share each -W and K^T load, which bounds many chains at once;
  // all of d_v in one workgroup also computes the output (no output pass)
  const ChainShape shape = chain_shape((int64_t)a.n_seq * a.s.h_v, a.t_total / a.n_seq);
  const bool chain_out = chain_out_fits<Op, D, C>(shape.ntw);
  if (max_chunks > 0) {
    // two V heads per QK head: one prep workgroup per QK head shares the q/k
    // loads (or convolutions) and the raw Gram products between them
    const ConvIn ci{a.x, a.conv_w, a.conv_b, a.conv_state, 0, false, 0};
    const GateIn gi{a.a_in, a.b_in, a.A_log, a.dt_bias};
    constexpr bool pair_fits = PrepLDS<Op, D, C, FUSE, 2>::BYTES <= 160 * 1024;
    constexpr int G2 = pair_fits ? 2 : 1;  // (fp32 at d = 128 and C = 64, which no entry point takes)
    if (pair_fits && a.s.h_v == 2 * a.s.h_k)
      hipLaunchKernelGGL((chunk_prep_kernel<T, Op, D, C, FUSE, W, G2>), dim3((unsigned)(max_chunks * a.s.h_k)),
                         dim3(K::THREADS), 0, st, (const T*)a.qkv, a.g, a.beta, a.cu_seqlens, a.slots, cstart,
                         a.n_slots, a.n_seq, a.t_total, a.s.h_k, a.s.h_v, a.scale, units, ci, gi, a.has_init,
                         (int32_t)chain_out);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<T, Op, D, C, FUSE, W, 1>), dim3((unsigned)(max_chunks * a.s.h_v)),
                         dim3(K::THREADS), 0, st, (const T*)a.qkv, a.g, a.beta, a.cu_seqlens, a.slots, cstart,
                         a.n_slots, a.n_seq, a.t_total, a.s.h_k, a.s.h_v, a.scale, units, ci, gi, a.has_init,
                         (int32_t)chain_out);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const int64_t groups = ((int64_t)a.n_seq * a.s.h_v + 7) / 8 * 8;
  const Op* cx = FUSE ? reinterpret_cast<const Op*>(a.x) : nullptr;
  hipError_t ce = hipErrorInvalidValue;
#define GDN_CHAIN_CASE(NTW_, PD_)                   \
  if (shape.ntw == NTW_ && shape.pd == PD_)          \
    ce = launch_shape<T, Op, D, C, NTW_, PD_>(a, groups, cstart, units, cx, st);
  GDN_CHAIN_SHAPES(GDN_CHAIN_CASE)
#undef GDN_CHAIN_CASE
  if (ce != hipSuccess) return ce;
  if (max_chunks > 0 && !chain_out)
    hipLaunchKernelGGL((chunk_out_kernel<T, Op, D, C, FUSE, W>), dim3((unsigned)(max_chunks * a.s.h_v)),
                       dim3(K::THREADS), 0, st, (const T*)a.qkv, a.cu_seqlens, a.slots, cstart, units, a.n_slots,
                       a.n_seq, a.t_total, a.s.h_k, a.s.h_v, (T*)a.o, (const T*)a.z, (const T*)a.norm_w,
                       a.norm_eps, ConvIn{a.x, a.conv_w, a.conv_b, a.conv_state, 0, false, 0}, a.has_init);
  return hipGetLastError();
}

}  // namespace split
}  // namespace gdn

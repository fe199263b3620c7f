// Fused recurrent GDN step for decode (t_step = 1) and MTP draft tokens
// (t_step > 1): gating, q/k L2 norm, the token-wise gated delta rule and the
// gated-RMSNorm epilogue in one kernel.
//
// The fused recurrent GDN kernel of LightLLM PR #1184 "[model] support
// Qwen3next" (Highlights, "Advanced Triton Kernel Optimizations") and the
// recurrent linear-attention operation of LightLLM #1097 (Highlights,
// "Specialized Triton Kernels"); per-draft-position states follow the MTP
// buffers of PR #1184 ("Enhanced Multi-Token Prediction").  Per token, with
// the state S in R^{d_v x d_k} and row i of S written s_i:
//   S <- e^g S;  u_i = beta (v_i - s_i.k);  s_i <- s_i + u_i k;  o_i = scale s_i.q
// and since rows are independent, o_i = scale (e^g (s_i.q) + u_i (k.q)) needs
// only the two dot products of the decayed old row.
//
// HBM design: the step is bound by the fp32 state (64 KiB per head at d=128,
// read once and written once).  One 256-thread workgroup owns one (request,
// V head) state; 16 lanes (one DPP row) hold one state row, each lane D/16
// consecutive-in-16-byte-groups columns, so every state load/store instruction
// moves 256-byte contiguous row segments.  All D*D/256 values per thread are
// loaded up front (D/16 rows x D/16 columns) so a workgroup has its whole
// state in flight before the first reduction.  The MTP step is its own
// kernel (recurrent_mtp_kernel): it writes one state per draft position and
// requests each next token's inputs ahead of those stores.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;

template <int D>
struct RowLayout {
  static constexpr int F = D / 16;               // columns per lane
  static constexpr int VW = F < 4 ? F : 4;       // floats per vector access
  static constexpr int NG = F / VW;              // vector groups per lane
  static constexpr int PASSES = D / 16;          // rows per thread (16 rows per pass)
  // first column of vector group j for column lane c
  __device__ static int col(int j, int c) { return j * 16 * VW + VW * c; }
};

// In-place decode reads and writes each state once, so those accesses are
// nontemporal: on gfx950 these streams reach the HBM rate that plain accesses
// to scattered slots do not.  The MTP step (per-position states written token
// after token) measures faster with plain accesses throughout.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <int VW, bool NT = true>
__device__ __forceinline__ void ld_f32(const float* p, float* v) {
  if constexpr (!NT) {
    if constexpr (VW == 4) {
      const float4 a = *reinterpret_cast<const float4*>(p);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else if constexpr (VW == 2) {
      const float2 a = *reinterpret_cast<const float2*>(p);
      v[0] = a.x; v[1] = a.y;
    } else {
      v[0] = *p;
    }
  } else if constexpr (VW == 4) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  } else if constexpr (VW == 2) {
    const f32x2_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(p));
    v[0] = a[0]; v[1] = a[1];
  } else {
    v[0] = __builtin_nontemporal_load(p);
  }
}
template <int VW, bool NT = true>
__device__ __forceinline__ void st_f32(float* p, const float* v) {
  if constexpr (!NT) {
    if constexpr (VW == 4) *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else if constexpr (VW == 2) *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    else *p = v[0];
  } else if constexpr (VW == 4) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
  } else if constexpr (VW == 2) {
    __builtin_nontemporal_store(f32x2_t{v[0], v[1]}, reinterpret_cast<f32x2_t*>(p));
  } else {
    __builtin_nontemporal_store(v[0], p);
  }
}
// VW consecutive floats from LDS.
template <int VW>
__device__ __forceinline__ void ld_lds_f32(const float* p, float* v) {
  if constexpr (VW == 4) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  } else if constexpr (VW == 2) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    v[0] = a.x; v[1] = a.y;
  } else {
    v[0] = *p;
  }
}

// One token's inputs as loaded (raw activations, converted at use): q and k
// of the QK head as vectors, this thread's v rows, its z rows (column lane 0
// only) and the per-position state slot.
template <typename T, int D>
struct TokenIn {
  using L = RowLayout<D>;
  typedef T vec_t __attribute__((ext_vector_type(L::VW)));
  vec_t k[L::NG], q[L::NG];
  T v[L::PASSES], z[L::PASSES];
  T a, b;
  int32_t dst;

  __device__ __forceinline__ void load(const T* __restrict__ qkv, const T* __restrict__ a_in,
                                       const T* __restrict__ b_in, const int32_t* __restrict__ out_slots,
                                       int64_t row, int c_ch, int hk, int h, int h_k, int h_v, int r16, int c) {
    const T* q_ptr = qkv + row * c_ch + hk * D;
    const T* k_ptr = qkv + row * c_ch + (h_k + hk) * D;
    const T* v_ptr = qkv + row * c_ch + 2 * h_k * D + h * D;
#pragma unroll
    for (int j = 0; j < L::NG; ++j) {
      k[j] = *reinterpret_cast<const vec_t*>(k_ptr + L::col(j, c));
      q[j] = *reinterpret_cast<const vec_t*>(q_ptr + L::col(j, c));
    }
#pragma unroll
    for (int p = 0; p < L::PASSES; ++p) v[p] = v_ptr[p * 16 + r16];
    a = a_in[row * h_v + h];
    b = b_in[row * h_v + h];
    dst = out_slots ? out_slots[row] : -1;
  }
  __device__ __forceinline__ void load_z(const T* __restrict__ z_in, int64_t row, int h, int h_v, int r16, int c) {
    const T* z_ptr = z_in + (row * h_v + h) * D;
#pragma unroll
    for (int p = 0; p < L::PASSES; ++p) z[p] = z_in && c == 0 ? z_ptr[p * 16 + r16] : from_f32<T>(0.0f);
  }
};

// The step for one (request, V head).  In place (MTP false): the final state
// goes back to slots[i].  MTP: the state after token t goes to out_slots[i][t],
// and token t+1's inputs are requested before token t's output and 64 KiB
// state stores: loads and stores share one counter that drains in issue order,
// so inputs loaded after the stores would wait for every store to complete.
template <typename T, int D, bool MTP>
__device__ __forceinline__ void recurrent_step(
    const T* __restrict__ qkv, const T* __restrict__ a_in, const T* __restrict__ b_in,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, float* __restrict__ state, int32_t n_slots,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ out_slots, T* __restrict__ o,
    const T* __restrict__ z, const T* __restrict__ norm_w, float norm_eps, float scale, int32_t t_step,
    int32_t h_k, int32_t h_v, float* red) {
  using L = RowLayout<D>;
  constexpr int F = L::F, VW = L::VW, NG = L::NG, PASSES = L::PASSES;

  const int i = blockIdx.x / h_v;
  const int h = blockIdx.x % h_v;
  const int hk = h / (h_v / h_k);
  const int tid = threadIdx.x;
  const int r16 = tid >> 4;   // row within a pass
  const int c = tid & 15;     // column lane
  const int c_ch = 2 * h_k * D + h_v * D;
  const int32_t slot = slots[i];

  if (!slot_ok(slot, n_slots)) {  // padding request: zero outputs
    for (int t = 0; t < t_step; ++t)
      for (int r = tid; r < D; r += kThreads) o[(((int64_t)i * t_step + t) * h_v + h) * D + r] = from_f32<T>(0.0f);
    return;
  }

  // ---- whole state into registers
  float s[PASSES][F];
  const float* src = state + ((int64_t)slot * h_v + h) * D * D;
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
#pragma unroll
    for (int j = 0; j < NG; ++j) ld_f32<VW, !MTP>(src + (p * 16 + r16) * D + L::col(j, c), &s[p][j * VW]);

  const float neg_A = -expf(A_log[h]);
  const float dtb = dt_bias[h];
  TokenIn<T, D> in;
  if (MTP) {
    in.load(qkv, a_in, b_in, out_slots, (int64_t)i * t_step, c_ch, hk, h, h_k, h_v, r16, c);
    in.load_z(z, (int64_t)i * t_step, h, h_v, r16, c);
  }

  for (int t = 0; t < t_step; ++t) {
    const int64_t row = (int64_t)i * t_step + t;
    if (!MTP) in.load(qkv, a_in, b_in, out_slots, row, c_ch, hk, h, h_k, h_v, r16, c);
    float kv[F], qv[F];
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        kv[j * VW + e] = to_f32(in.k[j][e]);
        qv[j * VW + e] = to_f32(in.q[j][e]);
      }

    // q, k L2 norm over the head (eps 1e-6 inside the root) and k.q
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < F; ++e) { sk = fmaf(kv[e], kv[e], sk); sq = fmaf(qv[e], qv[e], sq); }
    sk = group_sum<16>(sk);
    sq = group_sum<16>(sq);
    const float rk = fast_rsq(sk + 1e-6f), rq = fast_rsq(sq + 1e-6f);
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < F; ++e) { kv[e] *= rk; qv[e] *= rq; kq = fmaf(kv[e], qv[e], kq); }
    kq = group_sum<16>(kq);

    // gating
    const float g = neg_A * softplusf_(to_f32(in.a) + dtb);
    const float beta = sigmoidf_(to_f32(in.b));
    const float eg = expf(g);

    float orow[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      float dk = 0.f, dq = 0.f;
#pragma unroll
      for (int e = 0; e < F; ++e) { dk = fmaf(s[p][e], kv[e], dk); dq = fmaf(s[p][e], qv[e], dq); }
      dk = group_sum<16>(dk);
      dq = group_sum<16>(dq);
      const float u = beta * (to_f32(in.v[p]) - eg * dk);
      orow[p] = scale * (eg * dq + u * kq);
#pragma unroll
      for (int e = 0; e < F; ++e) s[p][e] = fmaf(eg, s[p][e], u * kv[e]);
    }
    const int32_t pos_slot = in.dst;
    float zrow[PASSES];
    if (MTP) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) zrow[p] = to_f32(in.z[p]);
      if (t + 1 < t_step) {
        in.load(qkv, a_in, b_in, out_slots, row + 1, c_ch, hk, h, h_k, h_v, r16, c);
        in.load_z(z, row + 1, h, h_v, r16, c);
      }
    }

    T* o_ptr = o + (row * h_v + h) * D;
    if (z) {
      // gated RMSNorm over d_v: every lane of a row group holds that row's o
      float ss = 0.f;
      if (c == 0) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) ss = fmaf(orow[p], orow[p], ss);
      }
      ss = wave_sum(ss);
      if ((tid & 63) == 0) red[tid >> 6] = ss;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
      __syncthreads();
      const float rstd = fast_rsq(tot * (1.0f / D) + norm_eps);
      if (!MTP) {
        in.load_z(z, row, h, h_v, r16, c);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) zrow[p] = to_f32(in.z[p]);
      }
      if (c == 0) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          const int r = p * 16 + r16;
          o_ptr[r] = from_f32<T>(orow[p] * rstd * to_f32(norm_w[r]) * fast_silu(zrow[p]));
        }
      }
    } else if (c == 0) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) o_ptr[p * 16 + r16] = from_f32<T>(orow[p]);
    }

    if (MTP && slot_ok(pos_slot, n_slots)) {
      float* dp = state + ((int64_t)pos_slot * h_v + h) * D * D;
#pragma unroll
      for (int p = 0; p < PASSES; ++p)
#pragma unroll
        for (int j = 0; j < NG; ++j) st_f32<VW, false>(dp + (p * 16 + r16) * D + L::col(j, c), &s[p][j * VW]);
    }
  }

  if (!MTP) {
    float* dp = state + ((int64_t)slot * h_v + h) * D * D;
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int j = 0; j < NG; ++j) st_f32<VW, true>(dp + (p * 16 + r16) * D + L::col(j, c), &s[p][j * VW]);
  }
}

// ---------------------------------------------------------------- decode
// The whole decode / MTP step in one kernel (gdn_decode): conv window update
// + SiLU, gating, q/k L2 norm, the recurrence and the gated-RMSNorm epilogue.
// One workgroup per (request, QK head) with 256 threads per V head of that QK
// head (G = h_v / h_k of them).  Every conv channel the workgroup reads -- q
// and k of the QK head, v of its G V heads -- is owned by one thread, which
// reads its slot window, computes the conv outputs of its channel for a block
// of tokens into LDS (in fp32: the conv output never reaches memory and is
// never rounded to the activation type), and writes the channel's new window
// itself; no other thread of any workgroup touches that channel, so the
// in-place window update needs no ordering between workgroups.  Each group of
// 256 threads then runs the token steps of its V head exactly as
// recurrent_step does, taking q, k, v from LDS.
template <int D, int G>
struct FusedLayout {
  static constexpr int THREADS = 256 * G;
  static constexpr int NCH = (2 + G) * D;          // conv channels per workgroup
  static constexpr int TB = 4;                     // tokens per LDS block
  static constexpr int CPT = (NCH + THREADS - 1) / THREADS;  // channels per thread
};

// One token step of V head h (256 threads: 16 row groups x 16 column lanes)
// with q, k, v of the token read from LDS: gating, q/k L2 norm, the state
// rows' update and the output, with the gated RMSNorm over d_v when z is given.
template <typename T, int D>
__device__ __forceinline__ void fused_token(float (&s)[D / 16][D / 16], const float* __restrict__ yq,
                                            const float* __restrict__ yk, const float* __restrict__ yv, float a_t, float b_t,
                                            float neg_A, float dtb, float scale, const T* __restrict__ z_row,
                                            const T* __restrict__ norm_w, float norm_eps, T* __restrict__ o_row,
                                            float* red, int red_base, int tid, int r16, int c) {
  using L = RowLayout<D>;
  constexpr int F = L::F, VW = L::VW, NG = L::NG, PASSES = L::PASSES;
  float kv[F], qv[F];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    ld_lds_f32<VW>(yq + L::col(j, c), &qv[j * VW]);
    ld_lds_f32<VW>(yk + L::col(j, c), &kv[j * VW]);
  }
  float sk = 0.f, sq = 0.f;
#pragma unroll
  for (int e = 0; e < F; ++e) { sk = fmaf(kv[e], kv[e], sk); sq = fmaf(qv[e], qv[e], sq); }
  sk = group_sum<16>(sk);
  sq = group_sum<16>(sq);
  const float rk = fast_rsq(sk + 1e-6f), rq = fast_rsq(sq + 1e-6f);
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < F; ++e) { kv[e] *= rk; qv[e] *= rq; kq = fmaf(kv[e], qv[e], kq); }
  kq = group_sum<16>(kq);
  const float g = neg_A * softplusf_(a_t + dtb);
  const float beta = sigmoidf_(b_t);
  const float eg = expf(g);

  float orow[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    float dk = 0.f, dq = 0.f;
#pragma unroll
    for (int e = 0; e < F; ++e) { dk = fmaf(s[p][e], kv[e], dk); dq = fmaf(s[p][e], qv[e], dq); }
    dk = group_sum<16>(dk);
    dq = group_sum<16>(dq);
    const float u = beta * (yv[p * 16 + r16] - eg * dk);
    orow[p] = scale * (eg * dq + u * kq);
#pragma unroll
    for (int e = 0; e < F; ++e) s[p][e] = fmaf(eg, s[p][e], u * kv[e]);
  }

  if (z_row) {
    float ss = 0.f;
    if (c == 0) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) ss = fmaf(orow[p], orow[p], ss);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) tot += red[red_base + w];
    __syncthreads();
    const float rstd = fast_rsq(tot * (1.0f / D) + norm_eps);
    if (c == 0) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int r = p * 16 + r16;
        o_row[r] = from_f32<T>(orow[p] * rstd * to_f32(norm_w[r]) * fast_silu(to_f32(z_row[r])));
      }
    }
  } else if (c == 0) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) o_row[p * 16 + r16] = from_f32<T>(orow[p]);
  }
}

// ONE: all t_step tokens fit one LDS block (t_step <= TB), so the block loop,
// and the conv registers' lifetime across it, disappear; TOK1: exactly one
// token (decode), with no token loop at all.
template <typename T, int D, int G, int W, bool MTP, bool ONE, bool TOK1 = false>
__global__ __launch_bounds__(256 * G) __attribute__((amdgpu_waves_per_eu(ONE && (MTP || TOK1) ? 4 : 1))) void decode_fused_kernel(
    const T* __restrict__ x, const T* __restrict__ conv_w, const T* __restrict__ conv_b, T* __restrict__ conv_state,
    const T* __restrict__ a_in, const T* __restrict__ b_in, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, float* __restrict__ state, int32_t n_slots, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ out_slots, T* __restrict__ o, const T* __restrict__ z, const T* __restrict__ norm_w,
    float norm_eps, float scale, int32_t t_step, int32_t h_k, int32_t h_v) {
  using L = RowLayout<D>;
  using FL = FusedLayout<D, G>;
  constexpr int VW = L::VW, NG = L::NG, PASSES = L::PASSES, TB = FL::TB, NCH = FL::NCH;
  __shared__ __attribute__((aligned(16))) float ys[TB][NCH];   // conv outputs: q | k | v of the G heads
  __shared__ __attribute__((aligned(16))) T zs[TB][G][D];       // z rows of the block's tokens
  __shared__ float gab[TB][G][2];                               // a, b of the block's tokens
  __shared__ float red[G * 4];

  const int i = blockIdx.x / h_k;
  const int hk = blockIdx.x % h_k;
  const int tid = threadIdx.x;
  const int half = tid >> 8;             // which V head of the QK head
  const int htid = tid & 255;
  const int h = hk * G + half;
  const int r16 = htid >> 4, c = htid & 15;
  const int c_ch = 2 * h_k * D + h_v * D;
  const int32_t slot = slots[i];

  if (!slot_ok(slot, n_slots)) {  // padding request: zero outputs, no pool entry touched
    for (int t = 0; t < t_step; ++t)
      for (int r = htid; r < D; r += 256) o[(((int64_t)i * t_step + t) * h_v + h) * D + r] = from_f32<T>(0.0f);
    return;
  }

  // ---- the state of V head h into registers first, so its loads are in
  // flight while the conv runs
  float s[PASSES][L::F];
  const float* src = state + ((int64_t)slot * h_v + h) * D * D;
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
#pragma unroll
    for (int j = 0; j < NG; ++j) ld_f32<VW, !MTP>(src + (p * 16 + r16) * D + L::col(j, c), &s[p][j * VW]);

  const float neg_A = -expf(A_log[h]);
  const float dtb = dt_bias[h];

  // conv + SiLU of tokens [t0, t0 + nt) into LDS, channel by channel (bias,
  // then the window oldest first, fp32 FMA: the order of the conv kernels);
  // per-position windows (MTP) and the final in-place window are stored as
  // soon as they are known
  auto conv_block = [&](float (&win)[FL::CPT][W - 1], const float (&wt)[FL::CPT][W], const float (&bias)[FL::CPT],
                        const int (&ch)[FL::CPT], int t0, int nt) {
    // the block's a, b and z rows into LDS too, so no token step loads from
    // memory after a state store (loads and stores drain in issue order)
    for (int e = tid; e < nt * G; e += FL::THREADS) {
      const int64_t ab = ((int64_t)i * t_step + t0 + e / G) * h_v + hk * G + e % G;
      gab[e / G][e % G][0] = to_f32(a_in[ab]);
      gab[e / G][e % G][1] = to_f32(b_in[ab]);
    }
    if (z)
      for (int e = tid; e < nt * G * D; e += FL::THREADS) {
        const int tt = e / (G * D), g = (e / D) % G, r = e % D;
        zs[tt][g][r] = z[(((int64_t)i * t_step + t0 + tt) * h_v + hk * G + g) * D + r];
      }
#pragma unroll
    for (int k = 0; k < FL::CPT; ++k) {
      const int lc = tid + k * FL::THREADS;
      if (lc < NCH) {
        // the block's inputs of this channel, all requested before the first
        // is used (one memory latency, not one per token)
        T xin[FL::TB];
#pragma unroll
        for (int tt = 0; tt < FL::TB; ++tt)
          if (tt < nt) xin[tt] = x[((int64_t)i * t_step + t0 + tt) * c_ch + ch[k]];
#pragma unroll
        for (int tt = 0; tt < FL::TB; ++tt) {
          if (tt >= nt) break;
          const int64_t row = (int64_t)i * t_step + t0 + tt;
          const T xv = xin[tt];
          float acc = bias[k];
#pragma unroll
          for (int j = 0; j < W - 1; ++j) acc = fmaf(wt[k][j], win[k][j], acc);
          acc = fmaf(wt[k][W - 1], to_f32(xv), acc);
          ys[tt][lc] = fast_silu(acc);
#pragma unroll
          for (int j = 0; j < W - 2; ++j) win[k][j] = win[k][j + 1];
          win[k][W - 2] = to_f32(xv);
          if (MTP) {
            const int32_t d = out_slots[row];
            if (slot_ok(d, n_slots)) {
              T* cd = conv_state + ((int64_t)d * c_ch + ch[k]) * (W - 1);
#pragma unroll
              for (int j = 0; j < W - 1; ++j) cd[j] = from_f32<T>(win[k][j]);
            }
          }
        }
        if (!MTP && t0 + nt == t_step) {
          T* cs = conv_state + ((int64_t)slot * c_ch + ch[k]) * (W - 1);
#pragma unroll
          for (int j = 0; j < W - 1; ++j) cs[j] = from_f32<T>(win[k][j]);
        }
      }
    }
  };
  // the token steps of a block, reading the block's conv outputs from LDS
  auto token_block = [&](int t0, int nt) {
    for (int tt = 0; tt < nt; ++tt) {
      const int64_t row = (int64_t)i * t_step + t0 + tt;
      fused_token<T, D>(s, &ys[tt][0], &ys[tt][D], &ys[tt][2 * D + half * D], gab[tt][half][0], gab[tt][half][1],
                        neg_A, dtb, scale, z ? &zs[tt][half][0] : nullptr, norm_w, norm_eps,
                        o + (row * h_v + h) * D, red, half * 4, tid, r16, c);
      if (MTP) {
        const int32_t d = out_slots[row];
        if (slot_ok(d, n_slots)) {
          float* dp = state + ((int64_t)d * h_v + h) * D * D;
#pragma unroll
          for (int p = 0; p < PASSES; ++p)
#pragma unroll
            for (int j = 0; j < NG; ++j) st_f32<VW, false>(dp + (p * 16 + r16) * D + L::col(j, c), &s[p][j * VW]);
        }
      } else if (t0 + tt == t_step - 1) {  // in place: the final state back to the home slot
        float* dp = state + ((int64_t)slot * h_v + h) * D * D;
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
#pragma unroll
          for (int j = 0; j < NG; ++j) st_f32<VW, true>(dp + (p * 16 + r16) * D + L::col(j, c), &s[p][j * VW]);
      }
    }
  };

  {
    // this thread's conv channels: global channel, taps, bias, window
    int ch[FL::CPT];
    float wt[FL::CPT][W], bias[FL::CPT], win[FL::CPT][W - 1];
#pragma unroll
    for (int k = 0; k < FL::CPT; ++k) {
      const int lc = tid + k * FL::THREADS;  // local channel: q (D), k (D), v of the G heads (G D)
      ch[k] = lc < D ? hk * D + lc : lc < 2 * D ? h_k * D + hk * D + (lc - D) : 2 * h_k * D + hk * G * D + (lc - 2 * D);
      if (lc < NCH) {
#pragma unroll
        for (int j = 0; j < W; ++j) wt[k][j] = to_f32(conv_w[(int64_t)ch[k] * W + j]);
        bias[k] = conv_b ? to_f32(conv_b[ch[k]]) : 0.0f;
        const T* cs = conv_state + ((int64_t)slot * c_ch + ch[k]) * (W - 1);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) win[k][j] = to_f32(cs[j]);
      }
    }
    if constexpr (ONE) {
      conv_block(win, wt, bias, ch, 0, TOK1 ? 1 : t_step);
      __syncthreads();
    } else {
      for (int t0 = 0; t0 < t_step; t0 += TB) {
        const int nt = min(TB, t_step - t0);
        conv_block(win, wt, bias, ch, t0, nt);
        __syncthreads();
        token_block(t0, nt);
        __syncthreads();  // the block's conv outputs are read before the next block overwrites them
      }
    }
  }
  if constexpr (ONE) token_block(0, TOK1 ? 1 : t_step);
}

template <typename T, int D, int G, int W, bool MTP, bool ONE, bool TOK1 = false>
hipError_t decode_launch1(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_fused_kernel<T, D, G, W, MTP, ONE, TOK1>), dim3((unsigned)((int64_t)a.n_seq * a.s.h_k)),
                     dim3(256 * G), 0, st, (const T*)a.x, (const T*)a.conv_w, (const T*)a.conv_b, (T*)a.conv_state,
                     (const T*)a.a, (const T*)a.b, a.A_log, a.dt_bias, a.state, a.n_slots, a.slots, a.out_slots,
                     (T*)a.o, (const T*)a.z, (const T*)a.norm_w, a.norm_eps, a.scale, a.t_step, a.s.h_k, a.s.h_v);
  return hipGetLastError();
}

template <typename T, int D, int G, int W>
hipError_t decode_launch(const DecodeArgs& a, hipStream_t st) {
  const bool one = a.t_step <= FusedLayout<D, G>::TB;
  if (a.out_slots)
    return one ? decode_launch1<T, D, G, W, true, true>(a, st) : decode_launch1<T, D, G, W, true, false>(a, st);
  if (a.t_step == 1) return decode_launch1<T, D, G, W, false, true, true>(a, st);
  return one ? decode_launch1<T, D, G, W, false, true>(a, st) : decode_launch1<T, D, G, W, false, false>(a, st);
}

template <typename T, int D, int G>
hipError_t decode_by_width(const DecodeArgs& a, hipStream_t st) {
  switch (a.s.conv_w) {
    case 2: return decode_launch<T, D, G, 2>(a, st);
    case 3: return decode_launch<T, D, G, 3>(a, st);
    case 4: return decode_launch<T, D, G, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t decode_by_group(const DecodeArgs& a, hipStream_t st) {
  switch (a.s.h_v / a.s.h_k) {
    case 1: return decode_by_width<T, D, 1>(a, st);
    case 2: return decode_by_width<T, D, 2>(a, st);
  }
  return hipErrorInvalidValue;
}

#define GDN_RECURRENT_ARGS                                                                                         \
  const T *__restrict__ qkv, const T *__restrict__ a_in, const T *__restrict__ b_in,                               \
      const float *__restrict__ A_log, const float *__restrict__ dt_bias, float *__restrict__ state,              \
      int32_t n_slots, const int32_t *__restrict__ slots, const int32_t *__restrict__ out_slots,                    \
      T *__restrict__ o, const T *__restrict__ z, const T *__restrict__ norm_w, float norm_eps, float scale,       \
      int32_t t_step, int32_t h_k, int32_t h_v

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(GDN_RECURRENT_ARGS) {
  __shared__ float red[kThreads / 64];
  recurrent_step<T, D, false>(qkv, a_in, b_in, A_log, dt_bias, state, n_slots, slots, out_slots, o, z, norm_w,
                              norm_eps, scale, t_step, h_k, h_v, red);
}

// (the prefetched inputs take it to two workgroups per CU; held to three,
// as in place, it spills and runs 10 % slower)
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void recurrent_mtp_kernel(
    GDN_RECURRENT_ARGS) {
  __shared__ float red[kThreads / 64];
  recurrent_step<T, D, true>(qkv, a_in, b_in, A_log, dt_bias, state, n_slots, slots, out_slots, o, z, norm_w,
                             norm_eps, scale, t_step, h_k, h_v, red);
}
#undef GDN_RECURRENT_ARGS

template <typename T, int D>
hipError_t impl(const RecurrentArgs& a, hipStream_t st) {
  if (a.n_seq == 0 || a.t_step == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)a.n_seq * a.s.h_v));
  if (a.out_slots)
    hipLaunchKernelGGL((recurrent_mtp_kernel<T, D>), grid, dim3(kThreads), 0, st, (const T*)a.qkv, (const T*)a.a,
                       (const T*)a.b, a.A_log, a.dt_bias, a.state, a.n_slots, a.slots, a.out_slots, (T*)a.o,
                       (const T*)a.z, (const T*)a.norm_w, a.norm_eps, a.scale, a.t_step, a.s.h_k, a.s.h_v);
  else
    hipLaunchKernelGGL((recurrent_kernel<T, D>), grid, dim3(kThreads), 0, st, (const T*)a.qkv, (const T*)a.a,
                       (const T*)a.b, a.A_log, a.dt_bias, a.state, a.n_slots, a.slots, a.out_slots, (T*)a.o,
                       (const T*)a.z, (const T*)a.norm_w, a.norm_eps, a.scale, a.t_step, a.s.h_k, a.s.h_v);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(const Shape& s) {
  const int g = s.h_v / s.h_k;
  return g == 1 || g == 2;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.n_seq == 0 || a.t_step == 0) return hipSuccess;
  switch (a.s.d) {
    case 16: return a.bf16 ? decode_by_group<bf16, 16>(a, st) : decode_by_group<float, 16>(a, st);
    case 32: return a.bf16 ? decode_by_group<bf16, 32>(a, st) : decode_by_group<float, 32>(a, st);
    case 64: return a.bf16 ? decode_by_group<bf16, 64>(a, st) : decode_by_group<float, 64>(a, st);
    case 128: return a.bf16 ? decode_by_group<bf16, 128>(a, st) : decode_by_group<float, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t st) {
  switch (a.s.d) {
    case 16: return a.bf16 ? impl<bf16, 16>(a, st) : impl<float, 16>(a, st);
    case 32: return a.bf16 ? impl<bf16, 32>(a, st) : impl<float, 32>(a, st);
    case 64: return a.bf16 ? impl<bf16, 64>(a, st) : impl<float, 64>(a, st);
    case 128: return a.bf16 ? impl<bf16, 128>(a, st) : impl<float, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

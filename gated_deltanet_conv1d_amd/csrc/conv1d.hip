// Causal depthwise conv1d + SiLU over the packed q|k|v channels.
//
// The operation LightLLM PR #1184 "[model] support Qwen3next" (Highlights,
// "Advanced Triton Kernel Optimizations": causal 1D convolutions) and LightLLM
// #1097 (Highlights, "Specialized Triton Kernels": causal 1D convolution) add
// for the GDN layer.  Per channel c and sequence position t:
//   y[t, c] = silu(bias[c] + sum_{j<W} w[c, j] * xe[t - (W-1) + j, c]),
// with xe = (slot's conv state, oldest first) ++ (the sequence's inputs).
//
// Layout choice for HBM: a thread owns 8 consecutive channels (one 16-byte
// bf16 vector) and walks a run of tokens, keeping the W-1 previous inputs in
// registers, so every x row is read once per tile (plus a W-1 row halo) with
// fully coalesced 16-byte accesses across the 8192-channel row.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;  // channels per thread
constexpr int kTile = 16;  // tokens per block on the fast path

template <typename T, int W>
struct Taps {
  float w[W][kVec];
  float b[kVec];
  // the kVec channels' taps are kVec * W consecutive weights: W vector loads
  __device__ void load(const T* __restrict__ wt, const T* __restrict__ bias, int c0) {
    float f[W * kVec];
#pragma unroll
    for (int j = 0; j < W; ++j) load8(wt + (int64_t)c0 * W + kVec * j, f + kVec * j);
#pragma unroll
    for (int i = 0; i < kVec; ++i)
#pragma unroll
      for (int j = 0; j < W; ++j) w[j][i] = f[i * W + j];
    if (bias) {
      load8(bias + c0, b);
    } else {
#pragma unroll
      for (int i = 0; i < kVec; ++i) b[i] = 0.0f;
    }
  }
  // out = silu(b + sum_j w[j] * win[j]) where win[W-1] is the current token.
  __device__ void apply(const float (&win)[W][kVec], float* out) const {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      float acc = b[i];
#pragma unroll
      for (int j = 0; j < W; ++j) acc = fmaf(w[j][i], win[j][i], acc);
      out[i] = fast_silu(acc);
    }
  }
};

// A thread's kVec channels of one slot's conv state are kVec * (W-1)
// consecutive values (channel-major, oldest first): W-1 vector accesses.
template <typename T, int W>
__device__ __forceinline__ void load_window(const T* __restrict__ st, float (&win)[W][kVec]) {
  float f[(W - 1) * kVec];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) load8(st + kVec * j, f + kVec * j);
#pragma unroll
  for (int i = 0; i < kVec; ++i)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) win[j][i] = f[i * (W - 1) + j];
}
template <typename T, int W>
__device__ __forceinline__ void store_window(T* __restrict__ st, const float (&win)[W][kVec]) {
  float f[(W - 1) * kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) f[i * (W - 1) + j] = win[j][i];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) store8(st + kVec * j, f + kVec * j);
}

__device__ __forceinline__ int32_t find_seq(const int32_t* __restrict__ cu, int32_t n_seq, int64_t t) {
  // largest i in [0, n_seq) with cu[i] <= t
  int32_t lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One block: kThreads * kVec channels x `tile` tokens.
template <typename T, int W>
__global__ __launch_bounds__(kThreads) void conv1d_fwd_kernel(
    const T* __restrict__ x, const T* __restrict__ wt, const T* __restrict__ bias,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const uint8_t* __restrict__ has_init,
    const T* __restrict__ conv_state, int32_t n_slots, T* __restrict__ y, int32_t n_seq, int64_t t_total,
    int32_t c_ch, int32_t n_cblk, int32_t tile) {
  const int64_t blk = blockIdx.x;
  const int cblk = (int)(blk % n_cblk);
  const int64_t t0 = (blk / n_cblk) * tile;
  const int c0 = (cblk * kThreads + (int)threadIdx.x) * kVec;
  if (c0 >= c_ch || t0 >= t_total) return;
  const int64_t t1 = min(t0 + (int64_t)tile, t_total);

  Taps<T, W> taps;
  taps.load(wt, bias, c0);

  int32_t n = find_seq(cu, n_seq, t0);
  // Fast path: a full tile inside one sequence, past its first W-1 tokens.
  // All TILE + W - 1 row loads are issued before any use, so they overlap
  // instead of costing one memory latency per token.
  if (tile == kTile) {
    const int64_t lo = min((int64_t)cu[n], t_total);
    const int64_t hi = min(max((int64_t)cu[n + 1], lo), t_total);
    if (t0 - (W - 1) >= lo && t0 + kTile <= hi && slot_ok(slots[n], n_slots)) {
      float rows[kTile + W - 1][kVec];
#pragma unroll
      for (int k = 0; k < kTile + W - 1; ++k) load8(x + (t0 - (W - 1) + k) * c_ch + c0, rows[k]);
#pragma unroll
      for (int k = 0; k < kTile; ++k) {
        float out[kVec];
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
          float acc = taps.b[i];
#pragma unroll
          for (int j = 0; j < W; ++j) acc = fmaf(taps.w[j][i], rows[k + j][i], acc);
          out[i] = fast_silu(acc);
        }
        store8(y + (t0 + k) * c_ch + c0, out);
      }
      return;
    }
  }
  int64_t t = t0;
  while (t < t1 && n < n_seq) {
    const int64_t lo = min((int64_t)cu[n], t_total);
    const int64_t hi = min(max((int64_t)cu[n + 1], lo), t_total);
    if (t >= hi) { ++n; continue; }
    const int64_t te = min(hi, t1);
    const int32_t slot = slots[n];
    if (!slot_ok(slot, n_slots)) {  // padding entry: zero rows
      float zero[kVec] = {};
      for (; t < te; ++t) store8(y + t * c_ch + c0, zero);
      ++n;
      continue;
    }
    const bool init = has_init == nullptr || has_init[n] != 0;
    // window rows 0..W-2 hold positions t-(W-1) .. t-1; row W-1 the current token
    float win[W][kVec];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int64_t pos = t - (W - 1) + j;
      if (pos >= lo) {
        load8(x + pos * c_ch + c0, win[j]);
      } else {
        const int64_t back = lo - pos;  // 1 .. W-1 steps before the sequence start
#pragma unroll
        for (int i = 0; i < kVec; ++i)
          win[j][i] = init ? to_f32(conv_state[((int64_t)slot * c_ch + c0 + i) * (W - 1) + (W - 1 - back)]) : 0.0f;
      }
    }
    for (; t < te; ++t) {
      load8(x + t * c_ch + c0, win[W - 1]);
      float out[kVec];
      taps.apply(win, out);
      store8(y + t * c_ch + c0, out);
#pragma unroll
      for (int j = 0; j < W - 1; ++j)
#pragma unroll
        for (int i = 0; i < kVec; ++i) win[j][i] = win[j + 1][i];
    }
    ++n;
  }
}

// After the conv: store the last W-1 entries of xe per sequence.  Runs as its
// own launch so that every read of the old state in the conv has finished.
template <typename T, int W>
__global__ __launch_bounds__(kThreads) void conv1d_store_state_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ cu, const int32_t* __restrict__ slots,
    const uint8_t* __restrict__ has_init, T* __restrict__ conv_state, int32_t n_slots, int64_t t_total,
    int32_t c_ch, int32_t n_cblk) {
  const int n = blockIdx.x / n_cblk;
  const int c0 = ((blockIdx.x % n_cblk) * kThreads + (int)threadIdx.x) * kVec;
  if (c0 >= c_ch) return;
  const int32_t slot = slots[n];
  if (!slot_ok(slot, n_slots)) return;
  const bool init = has_init == nullptr || has_init[n] != 0;
  const int64_t lo = min((int64_t)cu[n], t_total);
  const int64_t len = min(max((int64_t)cu[n + 1], lo), t_total) - lo;
  T* st = conv_state + ((int64_t)slot * c_ch + c0) * (W - 1);
  // the old window matters only when the sequence is shorter than W - 1
  float prev[W][kVec], nw[W][kVec];
  if (init && len < W - 1) {
    load_window<T, W>(st, prev);
  } else {
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
#pragma unroll
      for (int i = 0; i < kVec; ++i) prev[j][i] = 0.0f;
  }
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int64_t p = len - (W - 1) + j;  // position in the sequence; < 0 reaches into the old state
    if (p >= 0) {
      load8(x + (lo + p) * c_ch + c0, nw[j]);
    } else {  // old window entry (W - 1) + p, selected without a runtime register index
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        float v = 0.0f;
#pragma unroll
        for (int t = 0; t < W - 1; ++t) v = t == (W - 1) + (int)p ? prev[t][i] : v;
        nw[j][i] = v;
      }
    }
  }
  store_window<T, W>(st, nw);
}

// Decode / MTP: one block per (request, channel block); the window lives in
// registers across the request's t_step tokens.
template <typename T, int W>
__global__ __launch_bounds__(kThreads) void conv1d_update_kernel(
    const T* __restrict__ x, const T* __restrict__ wt, const T* __restrict__ bias, T* __restrict__ conv_state,
    int32_t n_slots, const int32_t* __restrict__ slots, const int32_t* __restrict__ out_slots,
    T* __restrict__ y, int32_t t_step, int32_t c_ch, int32_t n_cblk) {
  const int i = blockIdx.x / n_cblk;
  const int c0 = ((blockIdx.x % n_cblk) * kThreads + (int)threadIdx.x) * kVec;
  if (c0 >= c_ch) return;
  const int32_t slot = slots[i];
  const int64_t row0 = (int64_t)i * t_step;
  if (!slot_ok(slot, n_slots)) {
    float zero[kVec] = {};
    for (int p = 0; p < t_step; ++p) store8(y + (row0 + p) * c_ch + c0, zero);
    return;
  }
  Taps<T, W> taps;
  taps.load(wt, bias, c0);
  float win[W][kVec];
  load_window<T, W>(conv_state + ((int64_t)slot * c_ch + c0) * (W - 1), win);
  for (int p = 0; p < t_step; ++p) {
    load8(x + (row0 + p) * c_ch + c0, win[W - 1]);
    float out[kVec];
    taps.apply(win, out);
    store8(y + (row0 + p) * c_ch + c0, out);
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
#pragma unroll
      for (int ii = 0; ii < kVec; ++ii) win[j][ii] = win[j + 1][ii];
    if (out_slots) {
      const int32_t d = out_slots[row0 + p];
      if (slot_ok(d, n_slots)) store_window<T, W>(conv_state + ((int64_t)d * c_ch + c0) * (W - 1), win);
    }
  }
  if (!out_slots) store_window<T, W>(conv_state + ((int64_t)slot * c_ch + c0) * (W - 1), win);
}

template <typename T, int W>
hipError_t fwd_impl(const ConvFwdArgs& a, hipStream_t st) {
  const int c_ch = a.s.c_ch();
  const int n_cblk = (c_ch / kVec + kThreads - 1) / kThreads;
  if (a.t_total > 0 && a.n_seq > 0) {
    // aim for >= ~2048 blocks on 256 CUs; halo overhead is (W-1)/tile
    // fixed 16-token tiles (the fast path's size): >= 1024 blocks from 4096
    // tokens up, halo overhead (W-1)/16
    const int64_t tile = kTile;
    const int64_t n_tiles = (a.t_total + tile - 1) / tile;
    hipLaunchKernelGGL((conv1d_fwd_kernel<T, W>), dim3((unsigned)(n_tiles * n_cblk)), dim3(kThreads), 0, st,
                       (const T*)a.x, (const T*)a.w, (const T*)a.bias, a.cu_seqlens, a.slots, a.has_init,
                       (const T*)a.conv_state, a.n_slots, (T*)a.y, a.n_seq, a.t_total, c_ch, n_cblk, (int32_t)tile);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (a.n_seq > 0) {
    hipLaunchKernelGGL((conv1d_store_state_kernel<T, W>), dim3((unsigned)(a.n_seq * n_cblk)), dim3(kThreads), 0,
                       st, (const T*)a.x, a.cu_seqlens, a.slots, a.has_init, (T*)a.conv_state, a.n_slots,
                       a.t_total, c_ch, n_cblk);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int W>
hipError_t update_impl(const ConvUpdateArgs& a, hipStream_t st) {
  const int c_ch = a.s.c_ch();
  const int n_cblk = (c_ch / kVec + kThreads - 1) / kThreads;
  if (a.n_seq == 0 || a.t_step == 0) return hipSuccess;
  hipLaunchKernelGGL((conv1d_update_kernel<T, W>), dim3((unsigned)(a.n_seq * n_cblk)), dim3(kThreads), 0, st,
                     (const T*)a.x, (const T*)a.w, (const T*)a.bias, (T*)a.conv_state, a.n_slots, a.slots,
                     a.out_slots, (T*)a.y, a.t_step, c_ch, n_cblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, hipStream_t st) {
  switch (a.s.conv_w * 2 + (a.bf16 ? 1 : 0)) {
    case 2 * 2 + 1: return fwd_impl<bf16, 2>(a, st);
    case 3 * 2 + 1: return fwd_impl<bf16, 3>(a, st);
    case 4 * 2 + 1: return fwd_impl<bf16, 4>(a, st);
    case 2 * 2: return fwd_impl<float, 2>(a, st);
    case 3 * 2: return fwd_impl<float, 3>(a, st);
    case 4 * 2: return fwd_impl<float, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv1d_update(const ConvUpdateArgs& a, hipStream_t st) {
  switch (a.s.conv_w * 2 + (a.bf16 ? 1 : 0)) {
    case 2 * 2 + 1: return update_impl<bf16, 2>(a, st);
    case 3 * 2 + 1: return update_impl<bf16, 3>(a, st);
    case 4 * 2 + 1: return update_impl<bf16, 4>(a, st);
    case 2 * 2: return update_impl<float, 2>(a, st);
    case 3 * 2: return update_impl<float, 3>(a, st);
    case 4 * 2: return update_impl<float, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

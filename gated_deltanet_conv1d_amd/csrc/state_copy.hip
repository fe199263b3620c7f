// Slot-indexed state copy for the MTP commit: pool[dst[i]] <- pool[src[i]],
// bitwise, for the fp32 recurrent-state pool and the conv-state pool.  This
// is the buffer copy of LightLLM PR #1184 "[model] support Qwen3next" (review
// comment on the copy docstring: source and destination indices as 1-D
// arrays), done here as one HBM-bound kernel of 16-byte vector moves.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kIter = 4;                                     // 16-byte vectors per thread per piece
constexpr int64_t kPiece = (int64_t)kThreads * kIter * 16;  // bytes per block

// grid: n pairs x (state pieces + conv pieces)
__global__ __launch_bounds__(kThreads) void state_copy_kernel(
    uint8_t* __restrict__ state, uint8_t* __restrict__ conv, int64_t state_bytes, int64_t conv_bytes,
    int32_t n_slots, const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int32_t state_pieces,
    int32_t pieces) {
  const int pair = blockIdx.x / pieces;
  const int piece = blockIdx.x % pieces;
  const int32_t s = src[pair], d = dst[pair];
  if (!slot_ok(s, n_slots) || !slot_ok(d, n_slots) || s == d) return;
  const uint8_t* from;
  uint8_t* to;
  int64_t off, bytes;
  if (piece < state_pieces) {
    from = state + (int64_t)s * state_bytes;
    to = state + (int64_t)d * state_bytes;
    off = (int64_t)piece * kPiece;
    bytes = state_bytes;
  } else {
    if (!conv) return;
    from = conv + (int64_t)s * conv_bytes;
    to = conv + (int64_t)d * conv_bytes;
    off = (int64_t)(piece - state_pieces) * kPiece;
    bytes = conv_bytes;
  }
  // nontemporal: every byte is read once and written once; on gfx950 this
  // copy of scattered 2 MiB slots runs ~1.4x faster than with plain accesses
  u32x4 v[kIter];
#pragma unroll
  for (int k = 0; k < kIter; ++k) {
    const int64_t o = off + ((int64_t)k * kThreads + threadIdx.x) * 16;
    if (o < bytes) v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(from + o));
  }
#pragma unroll
  for (int k = 0; k < kIter; ++k) {
    const int64_t o = off + ((int64_t)k * kThreads + threadIdx.x) * 16;
    if (o < bytes) __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(to + o));
  }
}

// Slot-table check: entry i of the list slots ++ out_slots gets flags[i] =
// 1 if it is neither -1 nor a slot in [0, n_slots) (padding by another
// value), | 2 if it is a slot in [0, n_slots) equal to an earlier entry of
// the list.  One thread per entry scans the entries before it (a debugging
// aid: quadratic in the list length, which is a few thousand at most).
__global__ __launch_bounds__(kThreads) void slot_check_kernel(int32_t n_slots, const int32_t* __restrict__ slots,
                                                              int32_t n, const int32_t* __restrict__ out_slots,
                                                              int32_t n_out, int32_t* __restrict__ flags) {
  const int64_t total = (int64_t)n + n_out;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int32_t v = i < n ? slots[i] : out_slots[i - n];
    int32_t f = (v < -1 || v >= n_slots) ? 1 : 0;
    if (v >= 0 && v < n_slots)
      for (int64_t j = 0; j < i; ++j)
        if ((j < n ? slots[j] : out_slots[j - n]) == v) {
          f |= 2;
          break;
        }
    flags[i] = f;
  }
}

}  // namespace

hipError_t launch_slot_check(const SlotCheckArgs& a, hipStream_t st) {
  const int64_t total = (int64_t)a.n + a.n_out;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(slot_check_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(kThreads), 0, st,
                     a.n_slots, a.slots, a.n, a.out_slots, a.n_out, a.flags);
  return hipGetLastError();
}

hipError_t launch_state_copy(const StateCopyArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  const int64_t state_bytes = (int64_t)a.s.h_v * a.s.d * a.s.d * 4;
  const int64_t conv_bytes = (int64_t)a.s.c_ch() * (a.s.conv_w - 1) * (a.bf16 ? 2 : 4);
  const int32_t sp = (int32_t)((state_bytes + kPiece - 1) / kPiece);
  const int32_t cp = a.conv_state ? (int32_t)((conv_bytes + kPiece - 1) / kPiece) : 0;
  const int32_t pieces = sp + cp;
  hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((int64_t)a.n * pieces)), dim3(kThreads), 0, st,
                     (uint8_t*)a.state, (uint8_t*)a.conv_state, state_bytes, conv_bytes, a.n_slots, a.src, a.dst,
                     sp, pieces);
  return hipGetLastError();
}

}  // namespace gdn

// Host-side launchers, one per kernel family.  Each lives in the .hip file of
// its kernels; gdn_api.cpp validates arguments and then calls these.
// Arguments are already validated: sizes supported, pointers non-null where required.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct Shape {
  int h_k, h_v, d, conv_w;  // d = d_k = d_v
  int c_ch() const { return 2 * h_k * d + h_v * d; }
};

struct ConvFwdArgs {
  Shape s;
  bool bf16;
  int32_t n_seq;
  int64_t t_total;
  const void* x;
  const void* w;
  const void* bias;
  const int32_t* cu_seqlens;
  const int32_t* slots;
  const uint8_t* has_init;
  void* conv_state;
  int32_t n_slots;
  void* y;
};
hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, hipStream_t st);

struct ConvUpdateArgs {
  Shape s;
  bool bf16;
  int32_t n_seq, t_step;
  const void* x;
  const void* w;
  const void* bias;
  void* conv_state;
  int32_t n_slots;
  const int32_t* slots;
  const int32_t* out_slots;
  void* y;
};
hipError_t launch_conv1d_update(const ConvUpdateArgs& a, hipStream_t st);

struct GatingArgs {
  bool bf16;
  int64_t n_tokens;
  int32_t h_v;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  float* g;
  float* beta;
};
hipError_t launch_gating(const GatingArgs& a, hipStream_t st);

struct StateCopyArgs {
  Shape s;
  bool bf16;
  float* state;
  void* conv_state;
  int32_t n_slots;
  const int32_t* src;
  const int32_t* dst;
  int32_t n;
};
hipError_t launch_state_copy(const StateCopyArgs& a, hipStream_t st);

struct SlotCheckArgs {
  int32_t n_slots;
  const int32_t* slots;
  int32_t n;
  const int32_t* out_slots;
  int32_t n_out;
  int32_t* flags;
};
hipError_t launch_slot_check(const SlotCheckArgs& a, hipStream_t st);

struct RecurrentArgs {
  Shape s;
  bool bf16;
  int32_t n_seq, t_step;
  float scale;
  const void* qkv;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  float* state;
  int32_t n_slots;
  const int32_t* slots;
  const int32_t* out_slots;
  void* o;
  const void* z;
  const void* norm_w;
  float norm_eps;
};
hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t st);

// The whole decode / MTP step in one launch: conv window update + SiLU and
// the fused recurrent step, for h_v / h_k in {1, 2}.
struct DecodeArgs {
  Shape s;
  bool bf16;
  int32_t n_seq, t_step;
  float scale;
  const void* x;
  const void* conv_w;
  const void* conv_b;
  void* conv_state;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  float* state;
  int32_t n_slots;
  const int32_t* slots;
  const int32_t* out_slots;
  void* o;
  const void* z;
  const void* norm_w;
  float norm_eps;
};
bool decode_supported(const Shape& s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

struct ChunkArgs {
  Shape s;
  bool bf16;
  int32_t n_seq;
  int64_t t_total;
  int32_t chunk;
  float scale;
  const void* qkv;
  const float* g;
  const float* beta;
  const int32_t* cu_seqlens;
  const int32_t* slots;
  const uint8_t* has_init;
  float* state;
  int32_t n_slots;
  void* o;
  const void* z;
  const void* norm_w;
  float norm_eps;
  void* workspace;
  size_t ws_bytes;
  // Fused-input mode (x != nullptr): q, k, v are conv1d + SiLU of x, computed
  // in the chunk kernels (qkv unused), and g, beta come from a, b (g, beta
  // unused).  conv_state is read for the window before each sequence and then
  // updated in place with the final windows.
  const void* x = nullptr;
  const void* conv_w = nullptr;
  const void* conv_b = nullptr;
  const void* conv_state = nullptr;
  const void* a_in = nullptr;
  const void* b_in = nullptr;
  const float* A_log = nullptr;
  const float* dt_bias = nullptr;
};
// True when the chunk kernels have an instantiation for (d, chunk, dtype).
bool chunk_supported(int d, int chunk, bool bf16);
// The chunked form runs as a chunk-parallel preparation pass, a per-(sequence,
// V head, d_v tile) state pass and a chunk-parallel output pass, which talk
// through a caller-owned workspace of this many bytes.
size_t chunk_split_workspace_size(const Shape& s, bool bf16, int32_t n_seq, int64_t t_total, int32_t chunk);
hipError_t launch_chunk_split(const ChunkArgs& a, hipStream_t st);
// The fused-input prefill on the split path (a.x != nullptr), final conv
// windows included.
hipError_t launch_prefill_fused(const ChunkArgs& a, hipStream_t st);

// Gemma-form RMSNorm of the layer input (block.hip).
struct GemmaNormArgs {
  bool bf16;
  int64_t rows;
  int hidden;  // multiple of 8
  const void* x;
  const void* w;
  float eps;
  void* out;
};
hipError_t launch_gemma_norm(const GemmaNormArgs& a, hipStream_t st);

// Y[m, n] = sum_k X[m, k] W[n, k] (+ residual), bf16 in and out, fp32
// accumulation (block.hip).  Weight rows [0, n_w0) come from w0, [n_w0, n)
// from w1.  Output column n goes to the segment s with seg[s].begin <= n <
// seg[s+1].begin, at seg[s].ptr[m * seg[s].ld + n - seg[s].begin].
struct ProjSeg {
  int64_t begin;
  void* ptr;
  int64_t ld;
};
struct ProjArgs {
  int64_t m;
  int n, k;  // k a multiple of 8
  const void* x;
  int64_t ldx;
  const void* w0;
  int n_w0;
  const void* w1;
  int nseg;  // 1..4
  ProjSeg seg[4];
  const void* residual;  // [m][ld_res] bf16 or NULL; only with one segment
  int64_t ld_res;
};
hipError_t launch_proj(const ProjArgs& a, hipStream_t st);

}  // namespace gdn

// C ABI of the GDN hot path: argument validation and kernel dispatch.
// The calls, shapes and conventions are documented in include/gdn.h.
// Nothing here allocates, synchronises, or reads device memory.
#include "../../include/gdn.h"

#include <hip/hip_runtime.h>

#include "gdn_launch.hpp"

namespace {

using gdn::Shape;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int check_act(int32_t act) { return (act == GDN_BF16 || act == GDN_F32) ? GDN_OK : GDN_ERR_DTYPE; }

// Row counts above this are rejected: the workspace bytes (rows / chunk x h_v
// x ~100 KB) and every element offset stay far inside 64 bits below it.
constexpr int64_t kMaxRows = (int64_t)1 << 40;
inline bool rows_ok(int64_t rows) { return rows >= 0 && rows <= kMaxRows; }

// Validate a gdn_dims and turn it into the kernels' Shape.
int check_dims(const gdn_dims* d, Shape* s) {
  if (!d) return GDN_ERR_NULL;
  if (d->h_k <= 0 || d->h_v <= 0 || d->d_k <= 0 || d->d_v <= 0 || d->conv_w <= 0) return GDN_ERR_SHAPE;
  if (d->h_v % d->h_k != 0) return GDN_ERR_SHAPE;
  if (d->d_k != d->d_v) return GDN_ERR_UNSUPPORTED;
  if (d->d_k != 16 && d->d_k != 32 && d->d_k != 64 && d->d_k != 128) return GDN_ERR_UNSUPPORTED;
  if (d->conv_w < 2 || d->conv_w > 4) return GDN_ERR_UNSUPPORTED;
  if ((int64_t)2 * d->h_k * d->d_k + (int64_t)d->h_v * d->d_v > (1 << 24)) return GDN_ERR_UNSUPPORTED;
  *s = Shape{d->h_k, d->h_v, d->d_k, d->conv_w};
  return GDN_OK;
}

// All pointers in the list must be non-null.
template <typename... P>
int need(P... p) {
  const void* ptrs[] = {static_cast<const void*>(p)...};
  for (const void* q : ptrs)
    if (!q) return GDN_ERR_NULL;
  return GDN_OK;
}

// All non-null pointers in the list must be 16-byte aligned.
template <typename... P>
int align_ok(P... p) {
  const void* ptrs[] = {static_cast<const void*>(p)...};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return GDN_ERR_ALIGN;
  return GDN_OK;
}

inline int from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

#define GDN_TRY(expr)              \
  do {                             \
    int rc_ = (expr);              \
    if (rc_ != GDN_OK) return rc_; \
  } while (0)

}  // namespace

extern "C" {

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: invalid or inconsistent size";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown activation dtype";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: size not supported by this library";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: a kernel launch failed";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer not 16-byte aligned";
    case GDN_ERR_TOO_LARGE: return "GDN_ERR_TOO_LARGE: sizes exceed the static scratch of gdn_prefill_noalloc";
  }
  return "unknown gdn_status";
}

const char* gdn_version(void) { return "0.1.0"; }

int gdn_conv1d_fwd(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, const void* x, const void* w,
                   const void* bias, const int32_t* cu_seqlens, const int32_t* slots, const uint8_t* has_init,
                   void* conv_state, int32_t n_slots, void* y, void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (n_seq < 0 || !rows_ok(t_total) || n_slots < 0) return GDN_ERR_SHAPE;
  if (n_seq == 0 && t_total > 0) return GDN_ERR_SHAPE;
  if (n_seq == 0) return GDN_OK;
  GDN_TRY(need(w, cu_seqlens, slots, conv_state));
  if (t_total > 0) GDN_TRY(need(x, y));
  if (x && x == y) return GDN_ERR_SHAPE;
  GDN_TRY(align_ok(x, w, bias, conv_state, y));
  gdn::ConvFwdArgs a{s, act == GDN_BF16, n_seq, t_total, x, w, bias, cu_seqlens, slots, has_init,
                     conv_state, n_slots, y};
  return from_hip(gdn::launch_conv1d_fwd(a, (hipStream_t)stream));
}

int gdn_conv1d_update(const gdn_dims* dims, int32_t act, int32_t n_seq, int32_t t_step, const void* x, const void* w,
                      const void* bias, void* conv_state, int32_t n_slots, const int32_t* slots,
                      const int32_t* out_slots, void* y, void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (n_seq < 0 || t_step < 0 || n_slots < 0) return GDN_ERR_SHAPE;
  if (n_seq == 0 || t_step == 0) return GDN_OK;
  GDN_TRY(need(x, w, conv_state, slots, y));
  if (x == y) return GDN_ERR_SHAPE;
  GDN_TRY(align_ok(x, w, bias, conv_state, y));
  gdn::ConvUpdateArgs a{s, act == GDN_BF16, n_seq, t_step, x, w, bias, conv_state, n_slots, slots, out_slots, y};
  return from_hip(gdn::launch_conv1d_update(a, (hipStream_t)stream));
}

int gdn_gating(int32_t act, int64_t n_tokens, int32_t h_v, const void* a, const void* b, const float* A_log,
               const float* dt_bias, float* g, float* beta, void* stream) {
  GDN_TRY(check_act(act));
  if (!rows_ok(n_tokens) || h_v <= 0) return GDN_ERR_SHAPE;
  if (n_tokens == 0) return GDN_OK;
  GDN_TRY(need(a, b, A_log, dt_bias, g, beta));
  gdn::GatingArgs args{act == GDN_BF16, n_tokens, h_v, a, b, A_log, dt_bias, g, beta};
  return from_hip(gdn::launch_gating(args, (hipStream_t)stream));
}

size_t gdn_chunk_prefill_workspace_size(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total,
                                        int32_t chunk) {
  Shape s;
  if (check_dims(dims, &s) != GDN_OK || check_act(act) != GDN_OK || n_seq < 0 || !rows_ok(t_total)) return 0;
  return gdn::chunk_split_workspace_size(s, act == GDN_BF16, n_seq, t_total, chunk);
}

int gdn_chunk_prefill(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, int32_t chunk, float scale,
                      const void* qkv, const float* g, const float* beta, const int32_t* cu_seqlens,
                      const int32_t* slots, const uint8_t* has_init, float* state, int32_t n_slots, void* o,
                      const void* z, const void* norm_w, float norm_eps, void* workspace, size_t ws_bytes,
                      void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (n_seq < 0 || !rows_ok(t_total) || n_slots < 0) return GDN_ERR_SHAPE;
  if (n_seq == 0 && t_total > 0) return GDN_ERR_SHAPE;
  if (!gdn::chunk_supported(s.d, chunk, act == GDN_BF16)) return GDN_ERR_UNSUPPORTED;
  if (n_seq == 0) return GDN_OK;
  GDN_TRY(need(cu_seqlens, slots, state));
  if (t_total > 0) GDN_TRY(need(qkv, g, beta, o));
  if (z && !norm_w) return GDN_ERR_NULL;
  if (!(norm_eps >= 0.0f)) return GDN_ERR_SHAPE;
  GDN_TRY(align_ok(qkv, state, o, z, workspace));
  const size_t need_ws = gdn::chunk_split_workspace_size(s, act == GDN_BF16, n_seq, t_total, chunk);
  if (!workspace || ws_bytes < need_ws) return GDN_ERR_WORKSPACE;
  gdn::ChunkArgs a{s,     act == GDN_BF16, n_seq,  t_total, chunk,  scale,    qkv,      g,         beta,    cu_seqlens,
                   slots, has_init,        state,  n_slots, o,      z,        norm_w,   norm_eps,  workspace, ws_bytes};
  return from_hip(gdn::launch_chunk_split(a, (hipStream_t)stream));
}

size_t gdn_prefill_workspace_size(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, int32_t chunk) {
  Shape s;
  if (check_dims(dims, &s) != GDN_OK || check_act(act) != GDN_OK || n_seq < 0 || !rows_ok(t_total)) return 0;
  return gdn::chunk_split_workspace_size(s, act == GDN_BF16, n_seq, t_total, chunk);
}

int gdn_prefill(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, int32_t chunk, float scale,
                const void* x, const void* conv_w, const void* conv_b, const void* a, const void* b,
                const float* A_log, const float* dt_bias, const int32_t* cu_seqlens, const int32_t* slots,
                const uint8_t* has_init, void* conv_state, float* state, int32_t n_slots, void* o, const void* z,
                const void* norm_w, float norm_eps, void* workspace, size_t ws_bytes, void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (n_seq < 0 || !rows_ok(t_total) || n_slots < 0) return GDN_ERR_SHAPE;
  if (n_seq == 0 && t_total > 0) return GDN_ERR_SHAPE;
  if (!gdn::chunk_supported(s.d, chunk, act == GDN_BF16)) return GDN_ERR_UNSUPPORTED;
  if (n_seq == 0) return GDN_OK;
  GDN_TRY(need(cu_seqlens, slots, state, conv_state, conv_w));
  if (t_total > 0) GDN_TRY(need(x, a, b, A_log, dt_bias, o));
  if (z && !norm_w) return GDN_ERR_NULL;
  if (!(norm_eps >= 0.0f)) return GDN_ERR_SHAPE;
  GDN_TRY(align_ok(x, conv_w, conv_b, conv_state, state, o, z, workspace));
  const size_t need_ws = gdn::chunk_split_workspace_size(s, act == GDN_BF16, n_seq, t_total, chunk);
  if (!workspace || ws_bytes < need_ws) return GDN_ERR_WORKSPACE;
  gdn::ChunkArgs args{s,     act == GDN_BF16, n_seq,  t_total, chunk,  scale,    nullptr,  nullptr,   nullptr,
                      cu_seqlens, slots, has_init, state,  n_slots, o,      z,        norm_w,   norm_eps,
                      workspace, ws_bytes};
  args.x = x;
  args.conv_w = conv_w;
  args.conv_b = conv_b;
  args.conv_state = conv_state;
  args.a_in = a;
  args.b_in = b;
  args.A_log = A_log;
  args.dt_bias = dt_bias;
  return from_hip(gdn::launch_prefill_fused(args, (hipStream_t)stream));
}

int gdn_recurrent_decode(const gdn_dims* dims, int32_t act, int32_t n_seq, int32_t t_step, float scale,
                         const void* qkv, const void* a, const void* b, const float* A_log, const float* dt_bias,
                         float* state, int32_t n_slots, const int32_t* slots, const int32_t* out_slots, void* o,
                         const void* z, const void* norm_w, float norm_eps, void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (n_seq < 0 || t_step < 0 || n_slots < 0) return GDN_ERR_SHAPE;
  if (n_seq == 0 || t_step == 0) return GDN_OK;
  GDN_TRY(need(qkv, a, b, A_log, dt_bias, state, slots, o));
  if (z && !norm_w) return GDN_ERR_NULL;
  if (!(norm_eps >= 0.0f)) return GDN_ERR_SHAPE;
  GDN_TRY(align_ok(qkv, state, o, z));
  gdn::RecurrentArgs args{s,     act == GDN_BF16, n_seq,   t_step, scale,     qkv, a,      b,       A_log,
                          dt_bias, state,         n_slots, slots,  out_slots, o,   z,      norm_w, norm_eps};
  return from_hip(gdn::launch_recurrent(args, (hipStream_t)stream));
}

int gdn_decode(const gdn_dims* dims, int32_t act, int32_t n_seq, int32_t t_step, float scale, const void* x,
               const void* conv_w, const void* conv_b, const void* a, const void* b, const float* A_log,
               const float* dt_bias, void* conv_state, float* state, int32_t n_slots, const int32_t* slots,
               const int32_t* out_slots, void* o, const void* z, const void* norm_w, float norm_eps, void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (n_seq < 0 || t_step < 0 || n_slots < 0) return GDN_ERR_SHAPE;
  if (!gdn::decode_supported(s)) return GDN_ERR_UNSUPPORTED;
  if (n_seq == 0 || t_step == 0) return GDN_OK;
  GDN_TRY(need(x, conv_w, a, b, A_log, dt_bias, conv_state, state, slots, o));
  if (z && !norm_w) return GDN_ERR_NULL;
  if (!(norm_eps >= 0.0f)) return GDN_ERR_SHAPE;
  GDN_TRY(align_ok(x, conv_w, conv_b, conv_state, state, o, z));
  gdn::DecodeArgs args{s,       act == GDN_BF16, n_seq, t_step, scale, x,         conv_w, conv_b, conv_state, a, b,
                       A_log,   dt_bias,         state, n_slots, slots, out_slots, o,      z,      norm_w,     norm_eps};
  return from_hip(gdn::launch_decode(args, (hipStream_t)stream));
}

int gdn_rmsnorm_gemma(int32_t act, int64_t rows, int32_t hidden, const void* x, const void* w, float eps, void* out,
                      void* stream) {
  GDN_TRY(check_act(act));
  if (!rows_ok(rows) || hidden <= 0 || hidden % 8 != 0 || !(eps >= 0.0f)) return GDN_ERR_SHAPE;
  if (rows == 0) return GDN_OK;
  GDN_TRY(need(x, w, out));
  GDN_TRY(align_ok(x, w, out));
  gdn::GemmaNormArgs a{act == GDN_BF16, rows, hidden, x, w, eps, out};
  return from_hip(gdn::launch_gemma_norm(a, (hipStream_t)stream));
}

int gdn_in_proj(const gdn_dims* dims, int32_t act, int64_t t_total, int32_t hidden, const void* xn,
                const void* w_qkvz, const void* w_ba, void* qkv, void* z, void* b, void* a, void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (act != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (!rows_ok(t_total) || hidden <= 0 || hidden % 8 != 0) return GDN_ERR_SHAPE;
  if (t_total == 0) return GDN_OK;
  GDN_TRY(need(xn, w_qkvz, w_ba, qkv, z, b, a));
  GDN_TRY(align_ok(xn, w_qkvz, w_ba, qkv, z, b, a));
  const int c_ch = s.c_ch(), vd = s.h_v * s.d;
  gdn::ProjArgs p{};
  p.m = t_total;
  p.n = c_ch + vd + 2 * s.h_v;
  p.k = hidden;
  p.x = xn;
  p.ldx = hidden;
  p.w0 = w_qkvz;
  p.n_w0 = c_ch + vd;
  p.w1 = w_ba;
  p.nseg = 4;
  p.seg[0] = {0, qkv, c_ch};
  p.seg[1] = {c_ch, z, vd};
  p.seg[2] = {c_ch + vd, b, s.h_v};
  p.seg[3] = {c_ch + vd + s.h_v, a, s.h_v};
  return from_hip(gdn::launch_proj(p, (hipStream_t)stream));
}

int gdn_out_proj(const gdn_dims* dims, int32_t act, int64_t t_total, int32_t hidden, const void* o,
                 const void* w_out, const void* residual, void* y, void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (act != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (!rows_ok(t_total) || hidden <= 0 || hidden % 8 != 0) return GDN_ERR_SHAPE;
  if (t_total == 0) return GDN_OK;
  GDN_TRY(need(o, w_out, y));
  GDN_TRY(align_ok(o, w_out, residual, y));
  gdn::ProjArgs p{};
  p.m = t_total;
  p.n = hidden;
  p.k = s.h_v * s.d;
  p.x = o;
  p.ldx = p.k;
  p.w0 = w_out;
  p.n_w0 = hidden;
  p.w1 = nullptr;
  p.nseg = 1;
  p.seg[0] = {0, y, hidden};
  p.residual = residual;
  p.ld_res = hidden;
  return from_hip(gdn::launch_proj(p, (hipStream_t)stream));
}

int gdn_state_copy(const gdn_dims* dims, int32_t act, float* state, void* conv_state, int32_t n_slots,
                   const int32_t* src, const int32_t* dst, int32_t n, void* stream) {
  Shape s;
  GDN_TRY(check_dims(dims, &s));
  GDN_TRY(check_act(act));
  if (n < 0 || n_slots < 0) return GDN_ERR_SHAPE;
  if (n == 0) return GDN_OK;
  GDN_TRY(need(state, src, dst));
  GDN_TRY(align_ok(state, conv_state));
  gdn::StateCopyArgs a{s, act == GDN_BF16, state, conv_state, n_slots, src, dst, n};
  return from_hip(gdn::launch_state_copy(a, (hipStream_t)stream));
}

int gdn_check_slots(int32_t n_slots, const int32_t* slots, int32_t n, const int32_t* out_slots, int32_t n_out,
                    int32_t* flags, void* stream) {
  if (n_slots < 0 || n < 0 || n_out < 0) return GDN_ERR_SHAPE;
  if (n + (int64_t)n_out == 0) return GDN_OK;
  GDN_TRY(need(flags));
  if (n > 0) GDN_TRY(need(slots));
  if (n_out > 0) GDN_TRY(need(out_slots));
  gdn::SlotCheckArgs a{n_slots, slots, n, out_slots, n_out, flags};
  return from_hip(gdn::launch_slot_check(a, (hipStream_t)stream));
}

}  // extern "C"

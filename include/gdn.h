/*
 * gdn.h -- C ABI of the Gated DeltaNet (GDN) layer hot path for MI355X (gfx950).
 *
 * The layer: a causal depthwise conv1d + SiLU over the packed q|k|v channels,
 * fused gating, L2-normalised q/k, the gated delta rule evaluated chunk-wise
 * for prefill and token-wise for decode and MTP draft tokens, a gated-RMSNorm
 * epilogue, and slot-indexed state copies.  The operations are the ones
 * LightLLM PR #1184 "[model] support Qwen3next" lists under Highlights
 * ("Advanced Triton Kernel Optimizations": causal 1D convolutions, fused
 * recurrent GDN, fused gating; "Enhanced Multi-Token Prediction": state copying
 * for linear-attention states) and LightLLM #1097 "[model] Support Qwen3next"
 * lists under Highlights ("Specialized Triton Kernels": causal conv1d, fused GDN
 * gating, gated RMSNorm, chunked and recurrent linear-attention operations).
 * The head layout (16 QK heads, 32 V heads, head dim 128) is the one lmdeploy
 * issue #3961 "[Feature] Qwen3-Next-80B-A3B Support" gives under "New
 * attention kernels".  The recurrence is the published gated delta rule of
 * Gated Delta Networks (Yang, Kautz, Hatamizadeh, ICLR 2025), row form:
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t,      S in R^{d_v x d_k}.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees, synchronises, or reads device memory from the host.
 *    All work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns before it finishes.  Calls are graph-capturable.
 *  - Arrays are dense and row-major in the stated shapes.  Activations use
 *    `act` (GDN_BF16 or GDN_F32); recurrent states are always fp32; index
 *    arrays are int32; flags are uint8.  Pointers must be 16-byte aligned.
 *  - Packed channel order of a conv row: [q heads | k heads | v heads], each
 *    head's d entries contiguous; c_ch = 2*h_k*d_k + h_v*d_v.  V head h reads
 *    QK head h / (h_v / h_k).
 *  - Recurrent state pool: float [n_slots][h_v][d_v][d_k] (S, row i = d_v index).
 *    Conv state pool: act [n_slots][c_ch][conv_w-1], oldest input first.
 *  - Slot -1, or any slot outside [0, n_slots), marks a padding entry: its
 *    output rows are written as zeros and no pool entry is read or written.
 *  - Preconditions that cannot be checked without a host sync, undefined if
 *    violated: cu_seqlens non-decreasing with cu_seqlens[0] = 0 and
 *    cu_seqlens[n_seq] = t_total; no slot used twice in one call (in either
 *    role); copy sources disjoint from copy destinations.
 *  - Returns GDN_OK or a negative gdn_status.  Argument errors are reported
 *    before anything is enqueued; GDN_ERR_HIP means a launch failed.
 *  - Supported sizes: d_k == d_v in {16, 32, 64, 128}; h_v a multiple of h_k;
 *    conv_w in {2, 3, 4}; chunk in {16, 32, 64}.  Row counts (t_total, rows)
 *    above 2^40 are rejected with GDN_ERR_SHAPE (no device holds such a batch;
 *    below it every size computed from them, workspace bytes included, is
 *    exact in 64 bits), and the workspace-size queries return 0 for them.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,        /* a required pointer is NULL                       */
  GDN_ERR_SHAPE = -2,       /* a size is negative, zero where not allowed, or inconsistent */
  GDN_ERR_DTYPE = -3,       /* unknown activation dtype                         */
  GDN_ERR_UNSUPPORTED = -4, /* a valid but unsupported size (head dim, chunk, conv width) */
  GDN_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required       */
  GDN_ERR_HIP = -6,         /* a kernel launch failed                           */
  GDN_ERR_ALIGN = -7,       /* a pointer is not 16-byte aligned                 */
  GDN_ERR_TOO_LARGE = -8    /* the sizes need more than gdn_prefill_noalloc's static scratch */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* Layer shape: h_k QK heads, h_v V heads, head dims, conv width (taps). */
typedef struct {
  int32_t h_k, h_v, d_k, d_v, conv_w;
} gdn_dims;

/* Human-readable name of a gdn_status value (static string). */
const char* gdn_status_string(int status);

/* Library version as "major.minor.patch" (static string). */
const char* gdn_version(void);

/*
 * gdn_conv1d_fwd -- causal depthwise conv1d + SiLU over a packed varlen batch
 * (prefill).  For sequence i (rows cu_seqlens[i] .. cu_seqlens[i+1]-1):
 *   y[t, c] = silu(bias[c] + sum_{j<W} w[c, j] * xe[t - (W-1) + j, c])
 * where xe is the slot's conv state (or zeros when has_init[i] == 0) followed
 * by the sequence's inputs; w[c, W-1] multiplies the current token.  The last
 * W-1 entries of xe are then stored to conv_state[slots[i]] (a sequence
 * shorter than W-1 keeps the tail of the old state).
 *   x          act [t_total][c_ch]         inputs
 *   w          act [c_ch][conv_w]          taps
 *   bias       act [c_ch] or NULL
 *   cu_seqlens int32 [n_seq + 1]
 *   slots      int32 [n_seq]
 *   has_init   uint8 [n_seq] or NULL (= all 1)
 *   conv_state act [n_slots][c_ch][conv_w-1], read and updated in place
 *   y          act [t_total][c_ch]         output (may not alias x)
 * Enqueues two kernels: the conv, then the state store.
 */
int gdn_conv1d_fwd(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, const void* x,
                   const void* w, const void* bias, const int32_t* cu_seqlens, const int32_t* slots,
                   const uint8_t* has_init, void* conv_state, int32_t n_slots, void* y, void* stream);

/*
 * gdn_conv1d_update -- the same conv for decode / MTP: n_seq requests with
 * t_step new tokens each, request-major (each request's t_step rows are
 * consecutive, the MTP row layout of LightLLM PR #1159 "Qwen3 mtp dense").
 * Each request continues from conv_state[slots[i]].  out_slots NULL: the final
 * window is stored back to slots[i].  Otherwise the window after token p is
 * stored to out_slots[i*t_step + p] (skipped where -1) and slots[i] is only read.
 *   x  act [n_seq][t_step][c_ch];  y act [n_seq][t_step][c_ch]
 */
int gdn_conv1d_update(const gdn_dims* dims, int32_t act, int32_t n_seq, int32_t t_step, const void* x,
                      const void* w, const void* bias, void* conv_state, int32_t n_slots,
                      const int32_t* slots, const int32_t* out_slots, void* y, void* stream);

/*
 * gdn_gating -- fused GDN gating, elementwise over n_tokens * h_v:
 *   g    = -exp(A_log[h]) * softplus(a + dt_bias[h])     (log-decay, <= 0)
 *   beta = sigmoid(b)
 *   a, b act [n_tokens][h_v];  A_log, dt_bias float [h_v];  g, beta float [n_tokens][h_v]
 */
int gdn_gating(int32_t act, int64_t n_tokens, int32_t h_v, const void* a, const void* b, const float* A_log,
               const float* dt_bias, float* g, float* beta, void* stream);

/* Bytes of device workspace gdn_chunk_prefill needs for these sizes. */
size_t gdn_chunk_prefill_workspace_size(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total,
                                        int32_t chunk);

/*
 * gdn_chunk_prefill -- gated delta rule over a packed varlen batch, evaluated
 * chunk by chunk in the WY/UT form (the "chunked" operation of LightLLM #1097).
 * Per sequence i and V head h, starting from state[slots[i]][h] (zeros when
 * has_init[i] == 0), q and k are L2-normalised per head (eps 1e-6 inside the
 * square root) and the recurrence above runs over the sequence's tokens; the
 * final state is stored back to the slot.  When z is non-NULL the gated-RMSNorm
 * epilogue is applied per (token, V head) over d_v:
 *   out = o / sqrt(mean(o^2) + norm_eps) * norm_w * silu(z)
 * otherwise out = o.
 *   qkv        act [t_total][c_ch]         conv output (q|k|v packed)
 *   g, beta    float [t_total][h_v]        from gdn_gating
 *   state      float [n_slots][h_v][d_v][d_k]
 *   o          act [t_total][h_v][d_v]     output
 *   z          act [t_total][h_v][d_v] or NULL;  norm_w act [d_v] (needed with z)
 *   workspace  device scratch of at least gdn_chunk_prefill_workspace_size() bytes
 *              (a pure function of the sizes; never NULL when n_seq > 0)
 * The result does not depend on `chunk` in exact arithmetic.
 */
int gdn_chunk_prefill(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, int32_t chunk,
                      float scale, const void* qkv, const float* g, const float* beta, const int32_t* cu_seqlens,
                      const int32_t* slots, const uint8_t* has_init, float* state, int32_t n_slots, void* o,
                      const void* z, const void* norm_w, float norm_eps, void* workspace, size_t ws_bytes,
                      void* stream);

/*
 * gdn_prefill -- the whole prefill path in one call: conv1d + SiLU (as
 * gdn_conv1d_fwd), gating (as gdn_gating) and the chunked rule with its
 * epilogue (as gdn_chunk_prefill), with the conv output and the gates
 * computed inside the chunk kernels instead of round-tripping through device
 * memory (the fusion of the causal convolution into the chunked GDN operation
 * that LightLLM #1097 lists among its specialized kernels).  Results equal
 * those three calls in sequence; conv_state and state are updated in place
 * the same way.
 *   x        act [t_total][c_ch]   conv input;  conv_w act [c_ch][conv_w];  conv_b act [c_ch] or NULL
 *   a, b     act [t_total][h_v];   A_log, dt_bias float [h_v]
 *   conv_state act [n_slots][c_ch][conv_w-1];  state float [n_slots][h_v][d_v][d_k]
 *   o, z, norm_w, norm_eps, scale, chunk: as in gdn_chunk_prefill
 *   workspace  at least gdn_prefill_workspace_size() bytes (never NULL when t_total > 0)
 * Supported as gdn_chunk_prefill (d, chunk, dtype) with conv_w in {2, 3, 4};
 * always runs the chunk-parallel path.
 */
size_t gdn_prefill_workspace_size(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, int32_t chunk);
int gdn_prefill(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, int32_t chunk, float scale,
                const void* x, const void* conv_w, const void* conv_b, const void* a, const void* b,
                const float* A_log, const float* dt_bias, const int32_t* cu_seqlens, const int32_t* slots,
                const uint8_t* has_init, void* conv_state, float* state, int32_t n_slots, void* o, const void* z,
                const void* norm_w, float norm_eps, void* workspace, size_t ws_bytes, void* stream);

/*
 * gdn_prefill_noalloc -- gdn_prefill for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results as gdn_prefill without the
 * workspace: the library keeps one static scratch array of
 * gdn_prefill_noalloc_limit() bytes (256 MiB) per device, held from the
 * library's first use on that device until the process ends, and allocates
 * nothing.  Sizes whose gdn_prefill_workspace_size() exceeds the limit return
 * GDN_ERR_TOO_LARGE before anything is enqueued (a 4096-token prefill at 32 V
 * heads, d = 128, chunk 64 fits with up to 20 sequences).  The call runs on
 * the current device, which must be the stream's.  Every call on a device
 * shares that device's scratch: calls that overlap on one device (different
 * streams, no ordering between them) race.
 */
size_t gdn_prefill_noalloc_limit(void);
int gdn_prefill_noalloc(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, int32_t chunk,
                        float scale, const void* x, const void* conv_w, const void* conv_b, const void* a,
                        const void* b, const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                        const int32_t* slots, const uint8_t* has_init, void* conv_state, float* state,
                        int32_t n_slots, void* o, const void* z, const void* norm_w, float norm_eps, void* stream);

/*
 * gdn_recurrent_decode -- the fused recurrent step for decode (t_step = 1)
 * and MTP draft tokens (t_step > 1): gating, q/k L2 norm, the token-wise
 * recurrence and the gated-RMSNorm epilogue in one pass that reads each
 * recurrent state once.  Request-major inputs as in gdn_conv1d_update.
 *   qkv   act [n_seq][t_step][c_ch]  (conv output)
 *   a, b  act [n_seq][t_step][h_v];  A_log, dt_bias float [h_v]
 *   state float pool; each request starts from state[slots[i]]
 *   out_slots NULL: final state stored back to slots[i] (in place).
 *             else int32 [n_seq][t_step]: the state after draft token p is
 *             stored to out_slots[i][p] (skipped where -1); slots[i] is only read.
 *   o     act [n_seq][t_step][h_v][d_v];  z, norm_w as in gdn_chunk_prefill.
 */
int gdn_recurrent_decode(const gdn_dims* dims, int32_t act, int32_t n_seq, int32_t t_step, float scale,
                         const void* qkv, const void* a, const void* b, const float* A_log, const float* dt_bias,
                         float* state, int32_t n_slots, const int32_t* slots, const int32_t* out_slots, void* o,
                         const void* z, const void* norm_w, float norm_eps, void* stream);

/*
 * gdn_decode -- the whole decode / MTP draft step in one call: the conv window
 * update + SiLU (as gdn_conv1d_update) and the fused recurrent step with its
 * epilogue (as gdn_recurrent_decode), with the conv output kept in fp32 inside
 * the kernel instead of round-tripping through device memory in the
 * activation type (the fusion of the causal convolution and the fused
 * recurrent GDN step that LightLLM PR #1184 lists under Highlights, "Advanced
 * Triton Kernel Optimizations").  Because the conv output is not rounded, the
 * results are not bit-equal to the two separate calls; both follow the same
 * definitions.  conv_state and state are updated as those calls update them:
 * in place (out_slots NULL), or per draft position into out_slots with the
 * home slots only read.
 *   x      act [n_seq][t_step][c_ch]   conv input;  conv_w act [c_ch][conv_w];  conv_b act [c_ch] or NULL
 *   a, b   act [n_seq][t_step][h_v];   A_log, dt_bias float [h_v]
 *   conv_state act [n_slots][c_ch][conv_w-1];  state float [n_slots][h_v][d_v][d_k]
 *   slots, out_slots, o, z, norm_w, norm_eps, scale: as in gdn_recurrent_decode
 * Supported for h_v / h_k in {1, 2} (GDN_ERR_UNSUPPORTED otherwise).
 */
int gdn_decode(const gdn_dims* dims, int32_t act, int32_t n_seq, int32_t t_step, float scale, const void* x,
               const void* conv_w, const void* conv_b, const void* a, const void* b, const float* A_log,
               const float* dt_bias, void* conv_state, float* state, int32_t n_slots, const int32_t* slots,
               const int32_t* out_slots, void* o, const void* z, const void* norm_w, float norm_eps, void* stream);

/*
 * The layer around the core.  LightLLM #1097 "[model] Support Qwen3next" lists
 * a Gemma RMSNorm kernel next to the GDN kernels ("Specialized Triton
 * Kernels"); the layer's projections are in_proj_qkvz, in_proj_ba and
 * out_proj.  The layouts are readings: weights in [out_features][in_features]
 * order; in_proj_qkvz's outputs are the packed q|k|v conv input followed by z,
 * in_proj_ba's are b followed by a.  These three calls take bf16 only
 * (GDN_ERR_UNSUPPORTED for GDN_F32 in the projections); hidden is a positive
 * multiple of 8.
 *
 * gdn_rmsnorm_gemma -- the Gemma form of RMSNorm over the hidden size:
 *   out[t, :] = x[t, :] / sqrt(mean_j x[t, j]^2 + eps) * (1 + w)
 *   x, out  act [rows][hidden]   (out may not alias x)
 *   w       act [hidden]
 */
int gdn_rmsnorm_gemma(int32_t act, int64_t rows, int32_t hidden, const void* x, const void* w, float eps, void* out,
                      void* stream);

/*
 * gdn_in_proj -- the input projections of the normalised layer input xn, on
 * MFMA (bf16 operands, fp32 accumulation, each output rounded once):
 *   P = xn w_qkvz^T:  qkv = P[:, :c_ch]  (the conv input of gdn_prefill /
 *                     gdn_decode),  z = P[:, c_ch:]
 *   R = xn w_ba^T:    b = R[:, :h_v],  a = R[:, h_v:]
 *   xn     bf16 [t_total][hidden]
 *   w_qkvz bf16 [c_ch + h_v*d_v][hidden]
 *   w_ba   bf16 [2*h_v][hidden]
 *   qkv    bf16 [t_total][c_ch];  z bf16 [t_total][h_v][d_v];  b, a bf16 [t_total][h_v]
 * One kernel.  No output may alias an input.
 */
int gdn_in_proj(const gdn_dims* dims, int32_t act, int64_t t_total, int32_t hidden, const void* xn,
                const void* w_qkvz, const void* w_ba, void* qkv, void* z, void* b, void* a, void* stream);

/*
 * gdn_out_proj -- y = o w_out^T (+ residual), bf16 operands, fp32 accumulation,
 * the residual added before the one rounding:
 *   o        bf16 [t_total][h_v*d_v]   (the gated-RMSNorm output of the core)
 *   w_out    bf16 [hidden][h_v*d_v]
 *   residual bf16 [t_total][hidden] or NULL
 *   y        bf16 [t_total][hidden]    (may equal residual; may not alias o)
 */
int gdn_out_proj(const gdn_dims* dims, int32_t act, int64_t t_total, int32_t hidden, const void* o,
                 const void* w_out, const void* residual, void* y, void* stream);

/*
 * gdn_state_copy -- bitwise pool[dst[i]] <- pool[src[i]] for i < n, for the
 * recurrent state pool and (when conv_state is non-NULL) the conv state pool.
 * This is the MTP commit copy of LightLLM PR #1184 (copy buffers from source
 * indices to destination indices, both given as 1-D index arrays).  A pair
 * with -1 (or an out-of-range slot) on either side, or src == dst, is skipped.
 *   src, dst int32 [n]
 */
int gdn_state_copy(const gdn_dims* dims, int32_t act, float* state, void* conv_state, int32_t n_slots,
                   const int32_t* src, const int32_t* dst, int32_t n, void* stream);

/*
 * gdn_check_slots -- a debugging check of a call's slot tables, on the device
 * (the calls above cannot check them without a host sync: an entry used twice
 * races, see the conventions).  Over the list L = slots[0..n) followed by
 * out_slots[0..n_out), writes for each entry i
 *   flags[i] = (L[i] < -1 || L[i] >= n_slots ? 1 : 0)        padding other than -1
 *            | (0 <= L[i] < n_slots and L[i] == L[j] for some j < i ? 2 : 0)
 * so an all-zero flags array means every entry is -1 or a distinct in-range
 * slot.  For gdn_prefill / gdn_decode pass the call's slots and out_slots;
 * for gdn_state_copy pass dst, then src if sources must also be distinct.
 * O((n + n_out)^2) work on one stream; intended for tests and debugging.
 *   slots int32 [n];  out_slots int32 [n_out] (NULL when n_out == 0)
 *   flags int32 [n + n_out]   (device, written)
 */
int gdn_check_slots(int32_t n_slots, const int32_t* slots, int32_t n, const int32_t* out_slots, int32_t n_out,
                    int32_t* flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

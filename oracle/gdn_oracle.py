"""fp64 CPU oracle for the Gated DeltaNet (GDN) layer's data-parallel hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never uses it, and this
module imports nothing from the product path.

It is plain and slow on purpose: numpy in float64, a Python loop over tokens
with each step vectorised over heads, no chunking, blocking or fusion.  Inputs
arrive as exact activation values (bf16 or fp32 numbers held in float arrays)
and are upcast to float64; nothing is rounded on the way.

Sources.  The pages name the operations but never write their formulas:
  * LightLLM PR #1184 "[model] support Qwen3next", Highlights ("Advanced Triton
    Kernel Optimizations"): causal 1D convolutions, fused recurrent GDN and
    fused gating for the Gated Delta Networks (GDN) linear-attention layer;
    "Enhanced Multi-Token Prediction (MTP)": state copying for linear
    attention states during decode; "Refactored Memory Management": a
    MambaCacheManager holding per-request linear-attention states.
  * LightLLM #1097 "[model] Support Qwen3next", Highlights ("Specialized Triton
    Kernels"): causal 1D convolution, fused GDN gating, gated RMSNorm, and
    chunked and recurrent Flash Linear Attention operations.
  * lmdeploy issue #3961 "[Feature] Qwen3-Next-80B-A3B Support", "New attention
    kernels": Gated DeltaNet with 16 QK heads, 32 V heads, head_dim 128.
The recurrence itself is the published gated delta rule of Gated Delta
Networks (Yang, Kautz and Hatamizadeh, ICLR 2025), written here in the row
form S in R^{d_v x d_k}:

    S_t = exp(g_t) * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = scale * S_t q_t,

with q_t, k_t L2-normalised per head, g_t = -exp(A_log) * softplus(a_t + dt_bias)
and beta_t = sigmoid(b_t).  Readings taken where the pages are silent (conv
tap orientation, packed channel order, V->QK head map, epsilons, gated-RMSNorm
order, slot conventions) are stated at each function.
"""
from __future__ import annotations

import numpy as np

# Epsilon inside the square root of the q/k L2 normalisation (a reading: the
# pages give none; at d=128 it is immaterial since sum(q^2) is O(d)).
L2NORM_EPS = 1e-6


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------------ scalars
def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow for either sign."""
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(x):
    """x * sigmoid(x)."""
    x = _f64(x)
    return x * sigmoid(x)


def softplus(x):
    """log(1 + e^x) in the exact stable form max(x, 0) + log1p(e^-|x|)."""
    x = _f64(x)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


# ------------------------------------------------------------ causal conv1d
def causal_conv1d_silu(x, w, bias=None, state0=None):
    """Depthwise causal conv over time followed by SiLU, for one sequence.

    Operation named in LightLLM PR #1184, Highlights ("Advanced Triton Kernel
    Optimizations", causal 1D convolutions) and LightLLM #1097 ("Specialized
    Triton Kernels").

    x      [T, C]      inputs of one sequence
    w      [C, W]      taps; w[:, W-1] multiplies the current token (reading:
                       cross-correlation with W-1 steps of left history)
    bias   [C] or None
    state0 [C, W-1]    the W-1 inputs before this sequence, oldest first
                       (None = zeros, i.e. no history)

    y[t, c] = silu(bias[c] + sum_j w[c, j] * xe[t - (W-1) + j, c]) where xe is
    state0 followed by x.  Returns (y [T, C], new state [C, W-1]) where the new
    state is the last W-1 entries of xe (so a sequence shorter than W-1 keeps
    the tail of the old state).
    """
    x = _f64(x)
    w = _f64(w)
    T, C = x.shape
    W = w.shape[1]
    if state0 is None:
        state0 = np.zeros((C, W - 1))
    xe = np.concatenate([_f64(state0).T, x], axis=0)          # [W-1+T, C]
    pre = np.zeros((T, C))
    for j in range(W):
        pre += w[:, j] * xe[j:j + T]
    if bias is not None:
        pre += _f64(bias)
    y = silu(pre)
    new_state = xe[xe.shape[0] - (W - 1):].T.copy()
    return y, new_state


# ------------------------------------------------------------------ gating
def gating(a, b, A_log, dt_bias):
    """Fused GDN gating (LightLLM PR #1184 Highlights, "fused gating";
    LightLLM #1097 "Specialized Triton Kernels", fused GDN gating).

    g = -exp(A_log[h]) * softplus(a + dt_bias[h])   (log-decay, <= 0)
    beta = sigmoid(b)
    a, b: [..., H_v]; A_log, dt_bias: [H_v].
    """
    g = -np.exp(_f64(A_log)) * softplus(_f64(a) + _f64(dt_bias))
    beta = sigmoid(b)
    return g, beta


# ---------------------------------------------------------------- l2 norm
def l2norm(x, eps=L2NORM_EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis (per head)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def split_qkv(y, h_k, h_v, d_k, d_v):
    """Split packed conv output rows into q, k, v heads.

    Reading of "packed q/k/v channels": channels are [q heads | k heads | v
    heads], each head's d entries contiguous.
    """
    y = _f64(y)
    T = y.shape[0]
    q = y[:, : h_k * d_k].reshape(T, h_k, d_k)
    k = y[:, h_k * d_k: 2 * h_k * d_k].reshape(T, h_k, d_k)
    v = y[:, 2 * h_k * d_k: 2 * h_k * d_k + h_v * d_v].reshape(T, h_v, d_v)
    return q, k, v


def qk_head(h, h_k, h_v):
    """V head h reads QK head h // (h_v / h_k): consecutive V heads share one
    QK head (reading of lmdeploy #3961's 16 QK / 32 V heads)."""
    return h // (h_v // h_k)


# ------------------------------------------------------ gated delta rule
def delta_step(S, k, v, q, g, beta, scale):
    """One token of the gated delta rule for a stack of heads.

    S [H, d_v, d_k], k/q [H, d_k], v [H, d_v], g/beta [H].
    S <- exp(g) S;  u = beta (v - S k);  S <- S + u k^T;  o = scale S q.
    This is exp(g) S (I - beta k k^T) + beta v k^T expanded.
    Returns (S, o).
    """
    S = S * np.exp(g)[:, None, None]
    u = beta[:, None] * (v - np.matmul(S, k[:, :, None])[:, :, 0])
    S = S + u[:, :, None] * k[:, None, :]
    o = scale * np.matmul(S, q[:, :, None])[:, :, 0]
    return S, o


def gated_delta_rule(q, k, v, g, beta, S0=None, scale=1.0, heads=None, keep_states=False):
    """Token-by-token gated delta rule for one sequence.

    The recurrent form of the layer (LightLLM PR #1184 Highlights, fused
    recurrent GDN; LightLLM #1097, recurrent FLA operations).

    q, k  [T, H_k, d_k]  already L2-normalised
    v     [T, H_v, d_v]
    g, beta [T, H_v]
    S0    [H_v, d_v, d_k] or None (zeros)
    heads optional list of V heads to evaluate (others are skipped)
    Returns o [T, n_heads, d_v], S_T [n_heads, d_v, d_k] and, if keep_states,
    the list of states after each token.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, H_k, d_k = k.shape
    H_v, d_v = v.shape[1], v.shape[2]
    hs = list(range(H_v)) if heads is None else list(heads)
    hk = [qk_head(h, H_k, H_v) for h in hs]
    S = np.zeros((len(hs), d_v, d_k)) if S0 is None else _f64(S0)[hs].copy()
    o = np.zeros((T, len(hs), d_v))
    states = []
    for t in range(T):
        S, o[t] = delta_step(S, k[t, hk], v[t, hs], q[t, hk], g[t, hs], beta[t, hs], scale)
        if keep_states:
            states.append(S.copy())
    return o, S, states


# ----------------------------------------------------------- gated RMSNorm
def gated_rmsnorm(o, z, w, eps):
    """Gated RMSNorm epilogue (LightLLM #1097, "Specialized Triton Kernels").

    Reading: normalise each (token, V head) row of o over d_v, multiply by the
    plain weight w (not Gemma's 1+w, which the page lists separately), then by
    silu(z):  out = o / sqrt(mean(o^2) + eps) * w * silu(z).
    """
    o = _f64(o)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return (o / rms) * _f64(w) * silu(z)


# ------------------------------------------------------- whole-layer steps
def layer_sequence(x, a, b, z, conv_w, conv_b, A_log, dt_bias, norm_w, conv_state0, ssm_state0,
                   dims, scale=1.0, norm_eps=1e-6, heads=None, keep_states=False, perturb=None,
                   perturb_qk=None):
    """One sequence through the hot path, in the pages' kernel order:
    causal conv1d + SiLU -> split q/k/v -> L2 norm -> gating -> gated delta
    rule -> gated RMSNorm.

    dims = (h_k, h_v, d_k, d_v).  conv_state0 / ssm_state0 may be None (no
    history).  z None skips the epilogue (out = o).  With keep_states the
    states after every token are returned too (conv windows and recurrent
    states), which is what the MTP draft step stores per position.

    perturb, perturb_qk: optional functions applied to the conv output and
    to the normalised q and k respectively (e.g. rounding to bf16).  The
    pages run the conv and the linear-attention operation as separate kernels
    (LightLLM #1097, "Specialized Triton Kernels"), so the conv output exists
    as an activation tensor between them; evaluating the layer again with
    such tensors held at activation precision measures how far one rounding
    moves a result (its conditioning).  None (the default) is the exact
    evaluation.
    """
    h_k, h_v, d_k, d_v = dims
    y, conv_T = causal_conv1d_silu(x, conv_w, conv_b, conv_state0)
    if perturb is not None:
        y = perturb(y)
    q, k, v = split_qkv(y, h_k, h_v, d_k, d_v)
    q, k = l2norm(q), l2norm(k)
    if perturb_qk is not None:
        q, k = perturb_qk(q), perturb_qk(k)
    g, beta = gating(a, b, A_log, dt_bias)
    o, S_T, states = gated_delta_rule(q, k, v, g, beta, ssm_state0, scale, heads, keep_states)
    hs = list(range(h_v)) if heads is None else list(heads)
    out = o if z is None else gated_rmsnorm(o, _f64(z)[:, hs], norm_w, norm_eps)
    res = dict(y=y, g=g, beta=beta, o=o, out=out, ssm=S_T, conv=conv_T)
    if keep_states:
        res["ssm_states"] = states
        res["conv_states"] = [causal_conv1d_silu(x[: p + 1], conv_w, conv_b, conv_state0)[1]
                              for p in range(len(x))]
    return res


# ------------------------------------------------- the layer around the core
# LightLLM #1097 ("Specialized Triton Kernels") lists a Gemma RMSNorm kernel
# beside the GDN kernels, and the layer's input projections are named
# in_proj_qkvz and in_proj_ba; the pages give neither formulas nor layouts.
# Readings:
#   * the layer input is normalised over the hidden size by the Gemma form of
#     RMSNorm, whose weight enters as (1 + w): x / sqrt(mean(x^2) + eps) * (1 + w);
#   * in_proj_qkvz maps it to the packed q | k | v conv input followed by z
#     (h_v * d_v columns, V head major), in_proj_ba to b followed by a (h_v
#     columns each), the order of the projections' names;
#   * out_proj maps the gated-RMSNorm output, flattened over (V head, d_v), to
#     the hidden size; with residual the layer input is added to it;
#   * every weight has the [out_features, in_features] layout of a linear layer.

def gemma_rmsnorm(x, w, eps=1e-6):
    """Gemma-style RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * (1 + w)."""
    x = _f64(x)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return (x / rms) * (1.0 + _f64(w))


def linear(x, w):
    """x @ w^T for a weight in [out_features, in_features] layout."""
    return _f64(x) @ _f64(w).T


def block_sequence(X, weights, conv_w, conv_b, A_log, dt_bias, norm_w, conv_state0, ssm_state0, dims,
                   scale=1.0, norm_eps=1e-6, block_eps=1e-6, residual=True, keep_states=False, perturb=None):
    """One sequence through the whole layer: Gemma RMSNorm -> in_proj_qkvz and
    in_proj_ba -> the core (layer_sequence) -> out_proj (+ the input).

    X [T, hidden]; weights: dict with norm_w [hidden], w_qkvz [c_ch + h_v d_v,
    hidden], w_ba [2 h_v, hidden], w_out [hidden, h_v d_v].  perturb, when
    given, is applied to every activation tensor the layer hands from one
    kernel to the next (the normalised input, both projections, the conv
    output inside the core and the core's output), as in layer_sequence.
    """
    h_k, h_v, d_k, d_v = dims
    c_ch = 2 * h_k * d_k + h_v * d_v
    X = _f64(X)
    T = X.shape[0]
    pert = perturb if perturb is not None else (lambda t: t)
    xn = pert(gemma_rmsnorm(X, weights["norm_w"], block_eps))
    p = pert(linear(xn, weights["w_qkvz"]))
    q = pert(linear(xn, weights["w_ba"]))
    x, z = p[:, :c_ch], p[:, c_ch:].reshape(T, h_v, d_v)
    b, a = q[:, :h_v], q[:, h_v:]
    r = layer_sequence(x, a, b, z, conv_w, conv_b, A_log, dt_bias, norm_w, conv_state0, ssm_state0, dims,
                       scale, norm_eps, keep_states=keep_states, perturb=perturb)
    o = pert(r["out"].reshape(T, h_v * d_v))
    y = linear(o, weights["w_out"])
    if residual:
        y = y + X
    return dict(r, xn=xn, x=x, z=z, a=a, b=b, core_out=o, block_out=y)


def prefill_batch(x, a, b, z, cu_seqlens, slots, has_init, conv_pool, ssm_pool, params, dims,
                  scale=1.0, norm_eps=1e-6):
    """Packed varlen prefill over whole pools (small cases only).

    x [t_total, c_ch], a/b [t_total, h_v], z [t_total, h_v, d_v] or None.
    Sequence i spans rows cu_seqlens[i]:cu_seqlens[i+1] and owns slot
    slots[i] of conv_pool [n_slots, c_ch, W-1] and ssm_pool [n_slots, h_v, d_v,
    d_k] (the slot-pool layout of the MambaCacheManager in LightLLM PR #1184).
    has_init[i] = 0 starts from zero history.  An empty sequence stores its
    initial state unchanged (zeros when has_init is 0).  slot -1 marks a
    padding entry: its rows are written as zeros and no pool entry is read or
    written.
    Returns (out, conv_pool', ssm_pool') with new pool copies.
    """
    conv_pool = _f64(conv_pool).copy()
    ssm_pool = _f64(ssm_pool).copy()
    h_k, h_v, d_k, d_v = dims
    out = np.zeros((x.shape[0], h_v, d_v))
    for i in range(len(slots)):
        lo, hi = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        s = int(slots[i])
        if s < 0:
            continue
        init = has_init is None or bool(has_init[i])
        r = layer_sequence(x[lo:hi], a[lo:hi], b[lo:hi], None if z is None else z[lo:hi],
                           params["conv_w"], params.get("conv_b"), params["A_log"], params["dt_bias"],
                           params["norm_w"], conv_pool[s] if init else None,
                           ssm_pool[s] if init else None, dims, scale, norm_eps)
        out[lo:hi] = r["out"]
        conv_pool[s] = r["conv"]
        ssm_pool[s] = r["ssm"]
    return out, conv_pool, ssm_pool


def decode_batch(x, a, b, z, slots, out_slots, conv_pool, ssm_pool, params, dims,
                 scale=1.0, norm_eps=1e-6):
    """Decode / MTP draft step over pools (small cases only).

    Inputs are request-major [n, t_step, ...]: each request contributes
    t_step consecutive rows, the layout LightLLM PR #1159 ("Qwen3 mtp dense",
    review of flashattention_infer_struct.py) uses for mtp_step+1 rows per
    request.  Each request continues from its home slot.  out_slots None:
    the final states go back to the home slot.  Otherwise the states after
    draft token p go to out_slots[i][p] (skipped where -1) and the home slot
    is left untouched.  slot -1 marks a padding request (zero outputs).
    """
    conv_pool = _f64(conv_pool).copy()
    ssm_pool = _f64(ssm_pool).copy()
    h_k, h_v, d_k, d_v = dims
    n, t_step = x.shape[0], x.shape[1]
    out = np.zeros((n, t_step, h_v, d_v))
    conv0 = conv_pool.copy()
    ssm0 = ssm_pool.copy()
    for i in range(n):
        s = int(slots[i])
        if s < 0:
            continue
        r = layer_sequence(x[i], a[i], b[i], None if z is None else z[i], params["conv_w"],
                           params.get("conv_b"), params["A_log"], params["dt_bias"], params["norm_w"],
                           conv0[s], ssm0[s], dims, scale, norm_eps, keep_states=out_slots is not None)
        out[i] = r["out"]
        if out_slots is None:
            conv_pool[s] = r["conv"]
            ssm_pool[s] = r["ssm"]
        else:
            for p in range(t_step):
                d = int(out_slots[i][p])
                if d >= 0:
                    conv_pool[d] = r["conv_states"][p]
                    ssm_pool[d] = r["ssm_states"][p]
    return out, conv_pool, ssm_pool


def state_copy(pool, src, dst):
    """pool[dst[i]] <- pool[src[i]] for each pair; -1 on either side skips.

    The MTP commit copy of LightLLM PR #1184 (review comment on the buffer
    copy docstring: copy buffers from source indices to destination indices,
    both given as 1-D index tensors).  Returns a new array.
    """
    out = np.array(pool, copy=True)
    for s, d in zip(src, dst):
        if s >= 0 and d >= 0:
            out[d] = pool[s]
    return out

"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: exact
rational arithmetic, an independent chunked evaluation, closed forms, or a
library routine (torch CPU fp64).  ``test_planted_mistakes_are_caught`` plants
plausible bugs in the oracle and checks that the pins fail on each.
"""
from __future__ import annotations

import inspect
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import gdn_oracle as O
from tests.alt_forms import chunked_form, product_form_exact

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rel_err(x, r):
    x, r = np.asarray(x, np.float64), np.asarray(r, np.float64)
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300))


# ----------------------------------------------------------------- pins
# Rational unit vectors in R^3 (numerators of Pythagorean quadruples).
_UNIT3 = [(1, 2, 2, 3), (2, 1, -2, 3), (2, 3, 6, 7), (3, 4, 0, 5), (0, 3, 4, 5), (2, -2, 1, 3), (6, 2, -3, 7)]


def pin_exact_product_form(T=6, H_k=2, H_v=4):
    """Oracle recurrence vs the exact product form (d_k=3 != d_v=2, GQA 2:1)."""
    dk, dv = 3, 2
    rng = np.random.default_rng(11)
    K = [[[Fraction(u[i], u[3]) for i in range(3)] for u in
          (_UNIT3[(t * 3 + hk * 5) % 7] for t in range(T))] for hk in range(H_k)]
    Q = [[[Fraction(int(rng.integers(-4, 5)), 4) for _ in range(dk)] for _ in range(T)] for _ in range(H_k)]
    V = [[[Fraction(int(rng.integers(-6, 7)), 3) for _ in range(dv)] for _ in range(T)] for _ in range(H_v)]
    alpha = [[Fraction(int(rng.integers(5, 10)), 10) for _ in range(T)] for _ in range(H_v)]
    beta = [[Fraction(int(rng.integers(1, 5)), 4) for _ in range(T)] for _ in range(H_v)]
    S0 = [[[Fraction(int(rng.integers(-3, 4)), 2) for _ in range(dk)] for _ in range(dv)] for _ in range(H_v)]
    scale = Fraction(1, 2)
    # float copies for the oracle
    kf = np.array([[[float(x) for x in K[hk][t]] for hk in range(H_k)] for t in range(T)])
    qf = np.array([[[float(x) for x in Q[hk][t]] for hk in range(H_k)] for t in range(T)])
    vf = np.array([[[float(x) for x in V[h][t]] for h in range(H_v)] for t in range(T)])
    gf = np.array([[math.log(alpha[h][t]) for h in range(H_v)] for t in range(T)])
    bf = np.array([[float(beta[h][t]) for h in range(H_v)] for t in range(T)])
    S0f = np.array([[[float(x) for x in row] for row in S0[h]] for h in range(H_v)])
    o, S_T, _ = O.gated_delta_rule(qf, kf, vf, gf, bf, S0f, scale=float(scale))
    err = 0.0
    for h in range(H_v):
        hk = h // (H_v // H_k)
        o_ex, S_ex = product_form_exact(alpha[h], beta[h], K[hk], V[h], Q[hk], S0[h])
        o_ex = np.array([[float(x * scale) for x in row] for row in o_ex])
        S_ex = np.array([[float(x) for x in row] for row in S_ex])
        err = max(err, rel_err(o[:, h], o_ex), rel_err(S_T[h], S_ex))
    return err


def _rand_seq(rng, T, H_k, H_v, dk, dv, slow=False):
    q = O.l2norm(rng.standard_normal((T, H_k, dk)))
    k = O.l2norm(rng.standard_normal((T, H_k, dk)))
    v = rng.standard_normal((T, H_v, dv))
    if slow:
        g = -rng.uniform(0.0, 0.1, (T, H_v))
    else:
        g, _ = O.gating(rng.standard_normal((T, H_v)), np.zeros((T, H_v)),
                        rng.uniform(0, math.log(16), H_v), rng.uniform(-1, 1, H_v))
    beta = O.sigmoid(rng.standard_normal((T, H_v)))
    S0 = 0.3 * rng.standard_normal((H_v, dv, dk))
    return q, k, v, g, beta, S0


def pin_chunked_equals_recurrent(T=50, chunk=16, dk=16, dv=12, slow=True):
    """Oracle token loop vs the chunked WY/UT form (ragged last chunk, S0 != 0)."""
    rng = np.random.default_rng(5)
    H_k, H_v = 1, 2
    q, k, v, g, beta, S0 = _rand_seq(rng, T, H_k, H_v, dk, dv, slow)
    o, S_T, _ = O.gated_delta_rule(q, k, v, g, beta, S0, scale=0.7)
    err = 0.0
    for h in range(H_v):
        oc, Sc = chunked_form(q[:, 0], k[:, 0], v[:, h], g[:, h], beta[:, h], S0[h], chunk, scale=0.7)
        err = max(err, rel_err(o[:, h], oc), rel_err(S_T[h], Sc))
    return err


def pin_beta_zero_decay():
    """beta = 0: S_T = exp(sum g) S0 and o_t = exp(G_t) S0 q_t."""
    rng = np.random.default_rng(6)
    T, dk, dv = 40, 8, 5
    q, k, v, _, _, S0 = _rand_seq(rng, T, 1, 1, dk, dv)
    g = -rng.uniform(0, 0.05, (T, 1))
    o, S_T, _ = O.gated_delta_rule(q, k, v, g, np.zeros((T, 1)), S0)
    G = np.cumsum(g[:, 0])
    o_ref = np.exp(G)[:, None] * (q[:, 0] @ S0[0].T)
    return max(rel_err(S_T[0], math.exp(G[-1]) * S0[0]), rel_err(o[:, 0], o_ref))


def pin_orthonormal_retrieval():
    """g = 0, beta = 1, orthonormal keys, S0 = 0: S_T k_j = v_j, and querying
    with k_j returns v_j for every key already written."""
    rng = np.random.default_rng(7)
    T, dk, dv = 10, 12, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :T].T                                           # [T, dk] orthonormal rows
    v = rng.standard_normal((T, 1, dv))
    q = np.empty((T, 1, dk))
    q[:, 0] = keys[rng.integers(0, np.arange(1, T + 1))]          # query a key written so far
    o, S_T, _ = O.gated_delta_rule(q, keys[:, None], v, np.zeros((T, 1)), np.ones((T, 1)))
    err = rel_err(S_T[0] @ keys.T, v[:, 0].T)
    for t in range(T):
        j = int(np.argmax(np.abs(keys @ q[t, 0])))
        err = max(err, rel_err(o[t, 0], v[j, 0]))
    return err


def pin_write_invariant():
    """beta = 1, any g and S0: after token t, S_t k_t = v_t (unit k_t)."""
    rng = np.random.default_rng(8)
    T, dk, dv = 20, 8, 6
    q, k, v, g, _, S0 = _rand_seq(rng, T, 1, 1, dk, dv)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    _, _, states = O.gated_delta_rule(q, k, v, g, np.ones((T, 1)), S0, keep_states=True)
    return max(rel_err(states[t][0] @ k[t, 0], v[t, 0]) for t in range(T))


def pin_conv_vs_torch():
    """Oracle conv1d + SiLU vs torch's grouped conv1d (fp64) over state ++ x."""
    rng = np.random.default_rng(9)
    T, C, W = 13, 10, 4
    x, w, b = rng.standard_normal((T, C)), rng.standard_normal((C, W)), rng.standard_normal(C)
    st = rng.standard_normal((C, W - 1))
    y, new_state = O.causal_conv1d_silu(x, w, b, st)
    xe = torch.from_numpy(np.concatenate([st.T, x], 0).T[None])      # [1, C, W-1+T]
    ref = F.silu(F.conv1d(xe, torch.from_numpy(w)[:, None, :], torch.from_numpy(b), groups=C))[0].T.numpy()
    err = rel_err(y, ref)
    full = np.concatenate([st.T, x], 0)
    return max(err, rel_err(new_state, full[-(W - 1):].T))


def pin_gating_vs_torch():
    rng = np.random.default_rng(10)
    a, b = 4 * rng.standard_normal((50, 6)), 4 * rng.standard_normal((50, 6))
    A_log, dtb = rng.uniform(0, math.log(16), 6), rng.uniform(-1, 1, 6)
    g, beta = O.gating(a, b, A_log, dtb)
    t = torch.from_numpy
    g_ref = (-torch.exp(t(A_log)) * F.softplus(t(a) + t(dtb), threshold=50.0)).numpy()
    return max(rel_err(g, g_ref), rel_err(beta, torch.sigmoid(t(b)).numpy()))


def pin_rmsnorm_vs_torch():
    rng = np.random.default_rng(12)
    o, z, w = rng.standard_normal((7, 3, 16)), rng.standard_normal((7, 3, 16)), rng.uniform(0.5, 1.5, 16)
    out = O.gated_rmsnorm(o, z, w, 1e-6)
    t = torch.from_numpy
    ref = (F.rms_norm(t(o), (16,), weight=t(w), eps=1e-6) * F.silu(t(z))).numpy()
    return rel_err(out, ref)


def pin_l2norm():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((9, 2, 16)) * 3
    y = O.l2norm(x, eps=1e-6)
    n = np.linalg.norm(x, axis=-1)
    err = rel_err(np.linalg.norm(y, axis=-1), n / np.sqrt(n * n + 1e-6))
    cos = np.sum(x * y, -1) / (n * np.linalg.norm(y, axis=-1))
    return max(err, float(np.max(np.abs(cos - 1))))


def _silu(x):
    return x / (1.0 + math.exp(-x))


def pin_layer_worked_example():
    """The whole layer on a hand-worked case: T = 2 tokens, 1 QK head, 2 V heads,
    d = 2, conv width 2, through layer_sequence, prefill_batch and the MTP
    form of decode_batch.  Every expected value below is derived by hand from
    the chosen inputs (worked in the comments), not by running the oracle's
    code, so the pin checks the oracle's wiring: which of a, b feeds g and
    beta, the [q | k | v] split and the V->QK head map, z's head slicing, the
    per-position conv and state snapshots, and where the drivers store them.

    Channels: q (0, 1), k (2, 3), v of V head 0 (4, 5), v of V head 1 (6, 7).
    Taps (1, 2) on every channel: w[c, 1] multiplies the current token, so the
    pre-activation is p[t] = x[t-1] + 2 x[t], with x[-1] the old conv window.
    """
    x_prev = np.array([2, 3, 0, -2, 1, 0, -1, 0.5])
    x = np.array([[-1, -1, 1, 1, 1, -1, 0.5, 0.25],
                  [1, 0.5, -0.5, 0.5, -1, 2, 1, -1]])
    # p[0] = x_prev + 2 x[0] = [0, 1, 2, 0, 3, -2, 0, 1]
    # p[1] = x[0] + 2 x[1]   = [1, 0, 0, 2, -1, 3, 5/2, -7/4]
    p = np.array([[0, 1, 2, 0, 3, -2, 0, 1], [1, 0, 0, 2, -1, 3, 2.5, -1.75]])
    y = np.vectorize(_silu)(p)
    # q0 = (0, silu 1), q1 = (silu 1, 0); k0 = (silu 2, 0), k1 = (0, silu 2):
    # normalised with eps = 1e-6 they are c1 e2, c1 e1, c2 e1, c2 e2
    c1 = _silu(1.0) / math.sqrt(_silu(1.0) ** 2 + 1e-6)
    c2 = _silu(2.0) / math.sqrt(_silu(2.0) ** 2 + 1e-6)
    v = [[(y[0, 4], y[0, 5]), (y[0, 6], y[0, 7])], [(y[1, 4], y[1, 5]), (y[1, 6], y[1, 7])]]   # v[t][h]
    # gates: A_log = (0, ln 2), dt_bias = (0, 1/2); softplus(ln m) = ln(1 + m)
    #   head 0: a + dt_bias = 0, ln 3       -> e^g = 1/2, 1/4     (A = 1)
    #   head 1: a + dt_bias = ln 3, 0       -> e^g = 1/16, 1/4    (A = 2)
    #   beta = sigmoid(b): b = (ln 3, 0), (-ln 3, ln 7) -> 3/4, 1/2 and 1/4, 7/8
    a = np.array([[0.0, math.log(3) - 0.5], [math.log(3), -0.5]])
    b = np.array([[math.log(3), 0.0], [-math.log(3), math.log(7)]])
    A_log, dt_bias = np.array([0.0, math.log(2)]), np.array([0.0, 0.5])
    eg = np.array([[0.5, 1 / 16], [0.25, 0.25]])
    beta = np.array([[0.75, 0.5], [0.25, 0.875]])
    S0 = np.array([[[1, -1], [2, 0.5]], [[-0.5, 1], [1, -2]]])
    scale = 0.5
    # With k0 = c2 e1 the first token only rewrites column 1 of S, with
    # k1 = c2 e2 the second only column 2 (u = beta (v - e^g S k), S <- e^g S + u k^T):
    #   S1[:, 0] = e0 (1 - b0 c2^2) S0[:, 0] + b0 c2 v0,   S1[:, 1] = e0 S0[:, 1]
    #   S2[:, 0] = e1 S1[:, 0],   S2[:, 1] = e1 (1 - b1 c2^2) S1[:, 1] + b1 c2 v1
    # and q0 = c1 e2, q1 = c1 e1 read o0 = scale c1 S1[:, 1], o1 = scale c1 S2[:, 0].
    S1, S2, o = np.zeros((2, 2, 2)), np.zeros((2, 2, 2)), np.zeros((2, 2, 2))
    for h in range(2):
        e0, e1, b0, b1 = eg[0, h], eg[1, h], beta[0, h], beta[1, h]
        S1[h][:, 0] = e0 * (1 - b0 * c2 * c2) * S0[h][:, 0] + b0 * c2 * np.array(v[0][h])
        S1[h][:, 1] = e0 * S0[h][:, 1]
        S2[h][:, 0] = e1 * S1[h][:, 0]
        S2[h][:, 1] = e1 * (1 - b1 * c2 * c2) * S1[h][:, 1] + b1 * c2 * np.array(v[1][h])
        o[0, h] = scale * c1 * S1[h][:, 1]
        o[1, h] = scale * c1 * S2[h][:, 0]
    # epilogue per (token, V head): o / sqrt(mean o^2 + 1e-6) * w * silu(z)
    z = np.array([[[1, -1], [2, 0]], [[0, 3], [-1, 1]]], dtype=np.float64)
    norm_w = np.array([1.0, 0.5])
    out = np.zeros((2, 2, 2))
    for t in range(2):
        for h in range(2):
            r = math.sqrt((o[t, h, 0] ** 2 + o[t, h, 1] ** 2) / 2 + 1e-6)
            out[t, h] = [o[t, h, e] / r * norm_w[e] * _silu(z[t, h, e]) for e in range(2)]

    dims = (1, 2, 2, 2)
    taps = np.tile([1.0, 2.0], (8, 1))
    prm = dict(conv_w=taps, conv_b=None, A_log=A_log, dt_bias=dt_bias, norm_w=norm_w)
    err = 0.0

    def d(got, ref):
        return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))

    r = O.layer_sequence(x, a, b, z, taps, None, A_log, dt_bias, norm_w, x_prev[:, None], S0, dims, scale,
                         1e-6, keep_states=True)
    err = max(err, d(r["y"], y), d(np.exp(r["g"]), eg), d(r["beta"], beta), d(r["o"], o), d(r["out"], out),
              d(r["ssm"], S2), d(r["ssm_states"][0], S1), d(r["ssm_states"][1], S2))
    # conv windows (width 2 keeps one input): after token 0 it holds x[0], after token 1 x[1]
    err = max(err, d(r["conv"], x[1][:, None]), d(r["conv_states"][0], x[0][:, None]),
              d(r["conv_states"][1], x[1][:, None]))
    # one V head alone reads its own z, gates and v
    r1 = O.layer_sequence(x, a, b, z, taps, None, A_log, dt_bias, norm_w, x_prev[:, None], S0, dims, scale,
                          1e-6, heads=[1])
    err = max(err, d(r1["out"][:, 0], out[:, 1]), d(r1["ssm"][0], S2[1]))
    # prefill driver: the sequence in slot 2, then a padding entry; slots 0, 1 untouched
    conv_pool = np.stack([np.full((8, 1), 7.0), np.full((8, 1), 8.0), x_prev[:, None]])
    ssm_pool = np.stack([np.full((2, 2, 2), 7.0), np.full((2, 2, 2), 8.0), S0])
    xs, as_, bs, zs = (np.concatenate([u, u[:1]]) for u in (x, a, b, z))
    got, cp, sp = O.prefill_batch(xs, as_, bs, zs, [0, 2, 3], [2, -1], [1, 1], conv_pool, ssm_pool, prm, dims,
                                  scale)
    err = max(err, d(got[:2], out), d(got[2], 0.0), d(cp[2], x[1][:, None]), d(sp[2], S2),
              d(cp[:2], conv_pool[:2]), d(sp[:2], ssm_pool[:2]))
    # MTP draft step from home slot 0: the state after token p goes to out_slots[0][p]
    got, cp, sp = O.decode_batch(x[None], a[None], b[None], z[None], [0], [[3, 1]],
                                 np.stack([x_prev[:, None], conv_pool[0], conv_pool[1], conv_pool[1]]),
                                 np.stack([S0, ssm_pool[0], ssm_pool[1], ssm_pool[1]]), prm, dims, scale)
    err = max(err, d(got[0], out), d(cp[3], x[0][:, None]), d(sp[3], S1), d(cp[1], x[1][:, None]),
              d(sp[1], S2), d(cp[0], x_prev[:, None]), d(sp[0], S0), d(cp[2], conv_pool[1]))
    return err


def pin_gemma_rmsnorm_closed_form():
    """A constant row c 1 normalises to c / sqrt(c^2 + eps) (1 + w); a one-hot
    row s e_j to s / sqrt(s^2 / n + eps) (1 + w_j) at j and zero elsewhere; a
    weight of -1 zeroes its column."""
    n, eps = 6, 1e-6
    w = np.array([0.25, -0.5, 0.0, 1.0, -1.0, 0.125])
    err = 0.0
    for c in (3.0, -0.5):
        got = O.gemma_rmsnorm(np.full((1, n), c), w, eps)[0]
        err = max(err, float(np.abs(got - c / math.sqrt(c * c + eps) * (1.0 + w)).max()))
    s, j = 2.0, 3
    x = np.zeros((2, n))
    x[0, j] = s
    x[1] = np.arange(1.0, n + 1.0)
    exp0 = np.zeros(n)
    exp0[j] = s / math.sqrt(s * s / n + eps) * (1.0 + w[j])
    ms = sum(v * v for v in range(1, n + 1)) / n     # 91 / 6
    exp1 = np.array([(v + 1) / math.sqrt(ms + eps) * (1.0 + w[v]) for v in range(n)])
    got = O.gemma_rmsnorm(x, w, eps)
    return max(err, float(np.abs(got[0] - exp0).max()), float(np.abs(got[1] - exp1).max()), abs(got[1, 4]))


def pin_linear_brute_force():
    """x @ w^T against explicit sums on small integers (exact in fp64), with a
    non-square weight so that a transposed operand cannot pass."""
    rng = np.random.default_rng(40)
    x = rng.integers(-3, 4, (3, 5)).astype(np.float64)
    w = rng.integers(-3, 4, (4, 5)).astype(np.float64)
    ref = np.array([[sum(x[t, k] * w[n, k] for k in range(5)) for n in range(4)] for t in range(3)])
    return float(np.abs(O.linear(x, w) - ref).max())


def pin_block_identity_weights():
    """With selecting projections the layer reduces to the core on its
    normalised input.  hidden = c_ch + h_v d_v + 2 h_v; in_proj_qkvz takes the
    first c_ch + h_v d_v columns of the normalised input (conv input, then z),
    in_proj_ba the last 2 h_v (b, then a); out_proj writes the core output to
    the first h_v d_v columns and zero elsewhere; the input is added."""
    rng = np.random.default_rng(41)
    h_k, h_v, d_k, d_v = dims = (1, 2, 4, 4)
    c_ch, vd = 2 * h_k * d_k + h_v * d_v, h_v * d_v
    H, T = c_ch + vd + 2 * h_v, 7
    eye = np.eye(H)
    wts = dict(norm_w=rng.uniform(-0.5, 0.5, H), w_qkvz=eye[: c_ch + vd], w_ba=eye[c_ch + vd:],
               w_out=np.eye(H, vd))
    X = rng.standard_normal((T, H))
    conv_w, A_log, dt_bias = 0.5 * rng.standard_normal((c_ch, 4)), rng.uniform(0, 2.7, h_v), rng.uniform(-1, 1, h_v)
    norm_w, conv0, ssm0 = rng.uniform(0.5, 1.5, d_v), rng.standard_normal((c_ch, 3)), 0.1 * rng.standard_normal(
        (h_v, d_v, d_k))
    got = O.block_sequence(X, wts, conv_w, None, A_log, dt_bias, norm_w, conv0, ssm0, dims, 1.0, 1e-6, 1e-6)
    xn = O.gemma_rmsnorm(X, wts["norm_w"], 1e-6)
    core = O.layer_sequence(xn[:, :c_ch], xn[:, c_ch + vd + h_v:], xn[:, c_ch + vd: c_ch + vd + h_v],
                            xn[:, c_ch: c_ch + vd].reshape(T, h_v, d_v), conv_w, None, A_log, dt_bias, norm_w,
                            conv0, ssm0, dims, 1.0, 1e-6)
    exp = X.copy()
    exp[:, :vd] += core["out"].reshape(T, vd)
    return max(float(np.abs(got["block_out"] - exp).max()), float(np.abs(got["ssm"] - core["ssm"]).max()))


PINS = {
    "exact_product_form": (pin_exact_product_form, 1e-12),
    "chunked_equals_recurrent": (pin_chunked_equals_recurrent, 1e-11),
    "beta_zero_decay": (pin_beta_zero_decay, 1e-12),
    "orthonormal_retrieval": (pin_orthonormal_retrieval, 1e-12),
    "write_invariant": (pin_write_invariant, 1e-12),
    "conv_vs_torch": (pin_conv_vs_torch, 1e-13),
    "gating_vs_torch": (pin_gating_vs_torch, 1e-13),
    "rmsnorm_vs_torch": (pin_rmsnorm_vs_torch, 1e-13),
    "l2norm": (pin_l2norm, 1e-13),
    "layer_worked_example": (pin_layer_worked_example, 1e-12),
    "gemma_rmsnorm_closed_form": (pin_gemma_rmsnorm_closed_form, 1e-13),
    "linear_brute_force": (pin_linear_brute_force, 1e-300),   # exact: small integers
    "block_identity_weights": (pin_block_identity_weights, 1e-12),
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    assert fn() < tol


# ------------------------------------------------------- more closed forms
def test_chunked_form_many_shapes():
    for T, chunk, dk, dv, slow in [(64, 16, 16, 16, False), (64, 64, 8, 8, True), (1, 16, 4, 4, True),
                                   (97, 32, 16, 8, True), (130, 64, 12, 12, False)]:
        assert pin_chunked_equals_recurrent(T, chunk, dk, dv, slow) < 1e-10


def test_conv_identity_and_shift_taps():
    rng = np.random.default_rng(1)
    T, C, W = 9, 5, 4
    x, st = rng.standard_normal((T, C)), rng.standard_normal((C, W - 1))
    for j in range(W):
        w = np.zeros((C, W))
        w[:, j] = 1.0
        y, _ = O.causal_conv1d_silu(x, w, None, st)
        xe = np.concatenate([st.T, x], 0)
        shift = W - 1 - j                                   # tap j reads the input `shift` steps back
        ref = xe[W - 1 - shift: W - 1 - shift + T]
        assert np.allclose(y, ref * (1 / (1 + np.exp(-ref))), rtol=1e-14, atol=1e-14)


def test_conv_short_sequence_keeps_state_tail():
    rng = np.random.default_rng(2)
    C, W = 4, 4
    st = rng.standard_normal((C, W - 1))
    for T in (0, 1, 2, 3, 5):
        x = rng.standard_normal((T, C))
        _, ns = O.causal_conv1d_silu(x, rng.standard_normal((C, W)), None, st)
        assert np.array_equal(ns, np.concatenate([st.T, x], 0)[-(W - 1):].T)


def test_gating_special_values():
    g, beta = O.gating(np.zeros(3), np.zeros(3), np.zeros(3), np.zeros(3))
    assert np.allclose(np.exp(g), 0.5, rtol=0, atol=1e-15)        # -softplus(0) = -ln 2
    assert np.all(beta == 0.5)
    assert O.softplus(np.array([0.0]))[0] == pytest.approx(math.log(2), abs=1e-16)
    g, _ = O.gating(np.array([800.0, -800.0]), np.zeros(2), np.zeros(2), np.zeros(2))
    assert g[0] == -800.0 and -1e-300 < g[1] <= 0.0                # no overflow either way


def test_rmsnorm_constant_vector():
    c, eps = 0.37, 1e-6
    o = np.full((1, 1, 8), c)
    out = O.gated_rmsnorm(o, np.full((1, 1, 8), 40.0), np.ones(8), eps)   # silu(40) = 40 to 1e-16
    assert np.allclose(out, c / math.sqrt(c * c + eps) * 40.0, rtol=1e-14)


# --------------------------------------------------------- batch drivers
DIMS = (2, 4, 8, 8)          # h_k, h_v, d_k, d_v
C_CH = 2 * 2 * 8 + 4 * 8


def _params(rng):
    return dict(conv_w=0.5 * rng.standard_normal((C_CH, 4)), conv_b=None,
                A_log=rng.uniform(0, math.log(16), 4), dt_bias=rng.uniform(-1, 1, 4),
                norm_w=rng.uniform(0.5, 1.5, 8))


def _batch(rng, T):
    return (rng.standard_normal((T, C_CH)), rng.standard_normal((T, 4)), rng.standard_normal((T, 4)),
            rng.standard_normal((T, 4, 8)))


def _pools(rng, n_slots):
    return rng.standard_normal((n_slots, C_CH, 3)), 0.1 * rng.standard_normal((n_slots, 4, 8, 8))


def test_split_prefill_equals_single_pass():
    rng = np.random.default_rng(20)
    p = _params(rng)
    x, a, b, z = _batch(rng, 23)
    conv, ssm = _pools(rng, 3)
    one, c1, s1 = O.prefill_batch(x, a, b, z, [0, 23], [1], [1], conv, ssm, p, DIMS)
    o1, c2, s2 = O.prefill_batch(x[:10], a[:10], b[:10], z[:10], [0, 10], [1], [1], conv, ssm, p, DIMS)
    o2, c2, s2 = O.prefill_batch(x[10:], a[10:], b[10:], z[10:], [0, 13], [1], [1], c2, s2, p, DIMS)
    assert rel_err(np.concatenate([o1, o2]), one) < 1e-13
    assert rel_err(s2, s1) < 1e-13 and np.array_equal(c2, c1)


def test_decode_steps_equal_prefill():
    rng = np.random.default_rng(21)
    p = _params(rng)
    x, a, b, z = _batch(rng, 6)
    conv, ssm = _pools(rng, 2)
    ref, c_ref, s_ref = O.prefill_batch(x, a, b, z, [0, 6], [1], [1], conv, ssm, p, DIMS)
    c, s = conv, ssm
    outs = []
    for t in range(6):
        o, c, s = O.decode_batch(x[None, t:t + 1], a[None, t:t + 1], b[None, t:t + 1], z[None, t:t + 1],
                                 [1], None, c, s, p, DIMS)
        outs.append(o[0, 0])
    assert rel_err(np.stack(outs), ref) < 1e-13
    assert rel_err(s, s_ref) < 1e-13 and np.array_equal(c, c_ref)


def test_mtp_snapshots_equal_plain_steps():
    rng = np.random.default_rng(22)
    p = _params(rng)
    n, ts = 2, 3
    x, a, b = rng.standard_normal((n, ts, C_CH)), rng.standard_normal((n, ts, 4)), rng.standard_normal((n, ts, 4))
    conv, ssm = _pools(rng, n * (ts + 1))
    home = np.array([5, 1])
    outs = np.array([[0, 2, 7], [3, 4, 6]])
    o, c, s = O.decode_batch(x, a, b, None, home, outs, conv, ssm, p, DIMS)
    assert np.array_equal(c[home], conv[home]) and np.array_equal(s[home], ssm[home])
    for i in range(n):
        for q in range(ts):
            _, c_ref, s_ref = O.decode_batch(x[i:i + 1, :q + 1], a[i:i + 1, :q + 1], b[i:i + 1, :q + 1], None,
                                             home[i:i + 1], None, conv, ssm, p, DIMS)
            assert rel_err(s[outs[i, q]], s_ref[home[i]]) < 1e-13
            assert np.array_equal(c[outs[i, q]], c_ref[home[i]])


def test_permutation_invariance_and_padding():
    rng = np.random.default_rng(23)
    p = _params(rng)
    lens = [5, 0, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x, a, b, z = _batch(rng, cu[-1])
    conv, ssm = _pools(rng, 6)
    slots, init = np.array([4, 0, 2, 5]), np.array([1, 0, 0, 1])
    out, c, s = O.prefill_batch(x, a, b, z, cu, slots, init, conv, ssm, p, DIMS)
    # empty sequence with has_init=0 stores zero history; untouched slots unchanged
    assert np.all(c[0] == 0) and np.all(s[0] == 0)
    for u in (1, 3):
        assert np.array_equal(c[u], conv[u]) and np.array_equal(s[u], ssm[u])
    # reorder sequences and relabel slots
    perm = [2, 0, 3, 1]
    relabel = np.array([3, 5, 0, 1, 2, 4])
    segs = [slice(cu[i], cu[i + 1]) for i in perm]
    cat = lambda arr: np.concatenate([arr[sl] for sl in segs])
    lens_p = [lens[i] for i in perm]
    cu_p = np.concatenate([[0], np.cumsum(lens_p)])
    conv_p, ssm_p = np.empty_like(conv), np.empty_like(ssm)
    conv_p[relabel], ssm_p[relabel] = conv, ssm
    out_p, c_p, s_p = O.prefill_batch(cat(x), cat(a), cat(b), cat(z), cu_p, relabel[slots[perm]], init[perm],
                                      conv_p, ssm_p, p, DIMS)
    assert np.array_equal(out_p, cat(out))
    assert np.array_equal(c_p[relabel], c) and np.array_equal(s_p[relabel], s)
    # padding entry: zero rows, pools untouched
    out_pad, c_pad, s_pad = O.prefill_batch(x[:5], a[:5], b[:5], z[:5], [0, 5], [-1], [1], conv, ssm, p, DIMS)
    assert np.all(out_pad == 0) and np.array_equal(c_pad, conv) and np.array_equal(s_pad, ssm)


def test_state_copy():
    pool = np.arange(5 * 3, dtype=np.float64).reshape(5, 3)
    out = O.state_copy(pool, [0, 3, -1, 2], [4, 1, 2, -1])
    assert np.array_equal(out[[0, 2, 3]], pool[[0, 2, 3]])
    assert np.array_equal(out[4], pool[0]) and np.array_equal(out[1], pool[3])


# ------------------------------------------------------ planted mistakes
def _mut_no_decay(S, k, v, q, g, beta, scale):
    return _orig_step(S, k, v, q, np.zeros_like(g), beta, scale)


def _mut_sign(S, k, v, q, g, beta, scale):
    S = S * np.exp(g)[:, None, None]
    u = beta[:, None] * (v + np.matmul(S, k[:, :, None])[:, :, 0])
    S = S + u[:, :, None] * k[:, None, :]
    return S, scale * np.matmul(S, q[:, :, None])[:, :, 0]


def _mut_transpose(S, k, v, q, g, beta, scale):
    S = S * np.exp(g)[:, None, None]
    u = beta[:, None] * (v - np.matmul(S.transpose(0, 2, 1), k[:, :, None])[:, :, 0])
    S = S + u[:, :, None] * k[:, None, :]
    return S, scale * np.matmul(S, q[:, :, None])[:, :, 0]


def _mut_output_before_update(S, k, v, q, g, beta, scale):
    o = scale * np.matmul(S * np.exp(g)[:, None, None], q[:, :, None])[:, :, 0]
    S, _ = _orig_step(S, k, v, q, g, beta, scale)
    return S, o


def _mut_decay_after_update(S, k, v, q, g, beta, scale):
    u = beta[:, None] * (v - np.matmul(S, k[:, :, None])[:, :, 0])
    S = (S + u[:, :, None] * k[:, None, :]) * np.exp(g)[:, None, None]
    return S, scale * np.matmul(S, q[:, :, None])[:, :, 0]


_orig_step = O.delta_step
_orig_gating = O.gating
_orig_conv = O.causal_conv1d_silu
_orig_qk_head = O.qk_head
_orig_rms = O.gated_rmsnorm

def _mutated(fn_name, old, new):
    """A copy of oracle function fn_name with one source fragment replaced
    (a wiring mistake planted in the oracle; it runs on the CPU only)."""
    src = inspect.getsource(getattr(O, fn_name))
    assert old in src, (fn_name, old)
    ns = dict(vars(O))
    exec(compile(src.replace(old, new), O.__file__, "exec"), ns)
    return ns[fn_name]


MUTATIONS = {
    "no_decay": ("delta_step", _mut_no_decay),
    "update_sign": ("delta_step", _mut_sign),
    "transposed_state": ("delta_step", _mut_transpose),
    "output_before_update": ("delta_step", _mut_output_before_update),
    "decay_after_update": ("delta_step", _mut_decay_after_update),
    "gate_bias_sign": ("gating", lambda a, b, A_log, dtb: _orig_gating(a, b, A_log, -np.asarray(dtb))),
    "beta_not_sigmoid": ("gating", lambda a, b, A_log, dtb: (_orig_gating(a, b, A_log, dtb)[0], np.asarray(b) * 0.5 + 0.5)),
    "conv_taps_reversed": ("causal_conv1d_silu", lambda x, w, bias=None, state0=None:
                           _orig_conv(x, np.asarray(w)[:, ::-1], bias, state0)),
    "head_map_modulo": ("qk_head", lambda h, h_k, h_v: h % h_k),
    "l2norm_missing_sqrt": ("l2norm", lambda x, eps=O.L2NORM_EPS:
                            np.asarray(x) / (np.sum(np.asarray(x) ** 2, -1, keepdims=True) + eps)),
    "rmsnorm_sum_not_mean": ("gated_rmsnorm", lambda o, z, w, eps:
                             _orig_rms(o, z, w, eps) / math.sqrt(np.asarray(o).shape[-1])),
    "gates_a_b_swapped": ("layer_sequence", _mutated("layer_sequence", "gating(a, b,", "gating(b, a,")),
    "z_heads_reversed": ("layer_sequence", _mutated("layer_sequence", "_f64(z)[:, hs]", "_f64(z)[:, hs[::-1]]")),
    "z_first_heads": ("layer_sequence", _mutated("layer_sequence", "_f64(z)[:, hs]", "_f64(z)[:, :len(hs)]")),
    "conv_snapshot_off_by_one": ("layer_sequence", _mutated("layer_sequence", "x[: p + 1]", "x[: p + 2]")),
    "qkv_split_k_before_q": ("split_qkv", _mutated("split_qkv", "q = y[:, : h_k * d_k]", "q = y[:, h_k * d_k: 2 * h_k * d_k]")),
    "mtp_snapshot_of_next_token": ("decode_batch", _mutated("decode_batch", 'r["ssm_states"][p]', 'r["ssm_states"][-1]')),
    "prefill_state_to_wrong_slot": ("prefill_batch", _mutated("prefill_batch", "ssm_pool[s] = r[\"ssm\"]", "ssm_pool[s - 1] = r[\"ssm\"]")),
    "gemma_plain_weight": ("gemma_rmsnorm", _mutated("gemma_rmsnorm", "(1.0 + _f64(w))", "_f64(w)")),
    "gemma_sum_not_mean": ("gemma_rmsnorm", _mutated("gemma_rmsnorm", "np.mean(x * x", "np.sum(x * x")),
    "linear_transposed_weight": ("linear", lambda x, w: np.asarray(x, np.float64) @ np.asarray(w, np.float64)),
    "block_a_b_swapped": ("block_sequence", _mutated("block_sequence", "b, a = q[:, :h_v], q[:, h_v:]",
                                                     "a, b = q[:, :h_v], q[:, h_v:]")),
    "block_z_before_x": ("block_sequence", _mutated(
        "block_sequence", "x, z = p[:, :c_ch], p[:, c_ch:].reshape(T, h_v, d_v)",
        "x, z = p[:, h_v * d_v:], p[:, :h_v * d_v].reshape(T, h_v, d_v)")),
    "block_no_residual": ("block_sequence", _mutated("block_sequence", "y = y + X", "y = y")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for p, (pin, tol) in PINS.items():
        try:
            if not (pin() < tol):
                caught.append(p)
        except (ValueError, IndexError):      # a shape mistake that numpy rejects outright
            caught.append(p)
    assert caught, f"planted mistake {name} passes every pin"


def test_perturbation_hooks_are_neutral_when_identity():
    """layer_sequence's activation-precision hooks change nothing when they
    are the identity, and do change the result when they round."""
    import gdn_inputs as gi
    rng = np.random.default_rng(30)
    p = _params(rng)
    x, a, b, z = _batch(rng, 12)
    conv, ssm = _pools(rng, 1)
    args = (x, a, b, z, p["conv_w"], None, p["A_log"], p["dt_bias"], p["norm_w"], conv[0], ssm[0], DIMS)
    r0 = O.layer_sequence(*args)
    r1 = O.layer_sequence(*args, perturb=lambda t: t, perturb_qk=lambda t: t)
    r2 = O.layer_sequence(*args, perturb=gi.round_bf16, perturb_qk=gi.round_bf16)
    assert np.array_equal(r0["out"], r1["out"]) and np.array_equal(r0["ssm"], r1["ssm"])
    assert 0 < rel_err(r2["out"], r0["out"]) < 0.1

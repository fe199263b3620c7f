"""The oracle side of the GPU parity tests, runnable in worker processes.

This module imports numpy, the input generators and the oracle only (no torch,
no HIP), so its functions can run in a pool of CPU worker processes.  The pool
comes from a fork server that conftest.py starts before the test process
touches the GPU: the workers are forked from that server, never from the
process holding the GPU, and never use it.  Without the server (e.g. a single
test file run directly after the GPU is up) the functions run in-process.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import gdn_inputs as gi
from oracle import gdn_oracle as O

_CTX = None


def start_server() -> None:
    """Start the fork server.  Call before this process initialises the GPU."""
    global _CTX
    if _CTX is not None:
        return
    ctx = mp.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy", "gdn_inputs", "oracle.gdn_oracle", "tests.oracle_pool"])
    from multiprocessing import forkserver
    forkserver.ensure_running()
    _CTX = ctx


def n_workers() -> int:
    """Worker count: the CPU cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _init_worker() -> None:
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def run_map(fn, tasks, progress=None):
    """fn over tasks, results in order: on the worker pool when the server is
    up, else in-process.  progress(k, n) is called as results arrive."""
    tasks = list(tasks)
    out = []
    if _CTX is None or len(tasks) <= 1:
        for t in tasks:
            out.append(fn(t))
            if progress:
                progress(len(out), len(tasks))
        return out
    with _CTX.Pool(min(n_workers(), len(tasks)), initializer=_init_worker) as pool:
        for r in pool.imap(fn, tasks, chunksize=1):
            out.append(r)
            if progress:
                progress(len(out), len(tasks))
    return out


# --------------------------------------------------------------- numerics
def round_act(act: str):
    """Rounding of a conv output to the activation precision (float64 in, float64 out)."""
    if act == "bf16":
        return lambda y: gi.round_bf16(y).astype(np.float64)
    return lambda y: np.asarray(y, np.float64).astype(np.float32).astype(np.float64)


def perturbations(act: str):
    """Two activation-precision realisations of a conv output: rounded to the
    activation type, and rounded after a seeded random relative nudge (a
    second, equally valid realisation of the same values).  The larger change
    of the oracle's result under the two is its sensitivity: one realisation
    alone can understate how far rounding moves an ill-conditioned row.

    The nudge is the working precision of the path: half a unit in the last
    place for bf16, whose operand rounding dominates every other error there;
    for fp32, sqrt(128) 2^-24, the typical relative rounding of a length-128
    fp32 dot product (the contractions over d_k = 128 run in fp32, and the
    conv output and gates come from hardware exp2 and reciprocal, several
    units in the last place from the exact values), so half an fp32 unit
    would understate what the fp32 arithmetic does to a row that amplifies
    input perturbations several hundred times."""
    rnd = round_act(act)
    nudge = 2.0 ** -9 if act == "bf16" else np.sqrt(128.0) * 2.0 ** -24

    def nudged(y):
        y = np.asarray(y, np.float64)
        xi = np.random.default_rng(20251).uniform(-1.0, 1.0, y.shape)
        return rnd(y * (1.0 + nudge * xi))

    return [rnd, nudged]


def row_stats(x, r, rts=None, n=None):
    """(err, mag, sens) per row of the last axis (or of n trailing elements);
    rts: perturbed oracle results (an array or a list of them), sens their
    largest distance from r."""
    r = np.asarray(r, np.float64)
    n = n or (r.shape[-1] if r.ndim else 1)
    r = r.reshape(-1, n)
    x = np.asarray(x, np.float64).reshape(-1, n)
    if rts is None:
        sens = np.zeros(r.shape[0])
    else:
        rts = rts if isinstance(rts, (list, tuple)) else [rts]
        sens = np.max([np.abs(np.asarray(rt, np.float64).reshape(-1, n) - r).max(1) for rt in rts], axis=0)
    return np.abs(x - r).max(1), np.abs(r).max(1), sens


def from_raw(raw: np.ndarray) -> np.ndarray:
    """Device results as copied to the host: bf16 bit patterns (uint16) or fp32."""
    if raw.dtype == np.uint16:
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(raw, np.float64)


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


def prefill_seq_check(task):
    """Oracle (exact, and with its conv output at activation precision) for one
    sequence against the device's results for it.  task = (case, i, heads,
    scale, epilogue, out_raw [L, heads, d_v], ssm [heads, d_v, d_k] or None,
    conv [c_ch, W-1] or None).  Returns per-row output stats, per-head state
    stats and the largest conv-state difference."""
    case, i, heads, scale, epilogue, out_raw, ssm, conv = task
    f = lambda **pe: oracle_prefill_seq(case, i, heads=heads, scale=scale, epilogue=epilogue, **pe)
    r = f()
    rts = [f(perturb=pe) for pe in perturbations(case.act)]
    out = row_stats(from_raw(out_raw), r["out"], [rt["out"] for rt in rts])
    st = None
    if ssm is not None:
        st = [row_stats(ssm[j], r["ssm"][j], [rt["ssm"][j] for rt in rts], n=r["ssm"][j].size)
              for j in range(len(heads))]
    conv_d = 0.0
    if conv is not None and r["conv"].size:
        conv_d = float(np.max(np.abs(from_raw(conv) - r["conv"])))
    return out, st, conv_d


def decode_req_check(task):
    """One decode / MTP request: task = (case, i, out_raw [t_step, h_v, d_v],
    committed ssm [h_v, d_v, d_k] or None, its draft position).  The committed
    state is compared with the oracle's state after that many tokens."""
    case, i, out_raw, ssm, pos = task
    d = case.dims
    s = int(case.slots[i])
    p = case.params
    f = lambda **pe: O.layer_sequence(case.x()[i], case.a()[i], case.b()[i], case.z()[i], p.conv_w, None, p.A_log,
                                      p.dt_bias, p.norm_w, case.slot_conv(s), case.slot_ssm(s),
                                      (d.h_k, d.h_v, d.d_k, d.d_v), 1.0, 1e-6, keep_states=True, **pe)
    r = f()
    rts = [f(perturb=pe) for pe in perturbations(case.act)]
    out = row_stats(from_raw(out_raw), r["out"], [rt["out"] for rt in rts])
    st = None
    if ssm is not None:
        ref = r["ssm_states"][pos]
        st = [row_stats(ssm[h], ref[h], [rt["ssm_states"][pos][h] for rt in rts], n=ref[h].size)
              for h in range(d.h_v)]
    return out, st, r["conv_states"]


def _block_oracle(case, hidden, X, conv0, ssm0, residual, keep=False):
    """The whole layer (oracle.block_sequence) on one sequence or request of a
    case whose layer weights come from the case seed: the exact result and the
    two activation-precision realisations."""
    d = case.dims
    p = case.params
    w = gi.block_weights(case.seed, d, hidden, case.act).as_dict()
    f = lambda **pe: O.block_sequence(X, w, p.conv_w, None, p.A_log, p.dt_bias, p.norm_w, conv0, ssm0,
                                      (d.h_k, d.h_v, d.d_k, d.d_v), 1.0, 1e-6, 1e-6, residual, keep, **pe)
    return f(), [f(perturb=pe) for pe in perturbations(case.act)]


def block_seq_check(task):
    """The whole layer on sequence i of a prefill case against the device's
    results: task = (case, hidden, i, residual, out_raw [L, hidden], ssm
    [h_v, d_v, d_k], conv_raw [c_ch, W-1]) with o_raw [L, h_v, d_v] the core's
    output.  Returns per-token output stats, per-(token, V head) core-output
    stats, per-head state stats and per-channel conv-state stats."""
    case, hidden, i, residual, out_raw, o_raw, ssm, conv_raw = task
    s = int(case.slots[i])
    init = bool(case.has_init[i])
    X = gi.block_input(case.seed, i, int(case.lengths[i]), hidden, case.act)
    r, rts = _block_oracle(case, hidden, X, case.slot_conv(s) if init else None, case.slot_ssm(s) if init else None,
                           residual)
    out = row_stats(from_raw(out_raw), r["block_out"], [rt["block_out"] for rt in rts])
    dv = case.dims.d_v
    o = row_stats(from_raw(o_raw), r["core_out"], [rt["core_out"] for rt in rts], n=dv)
    st = [row_stats(ssm[h], r["ssm"][h], [rt["ssm"][h] for rt in rts], n=r["ssm"][h].size)
          for h in range(case.dims.h_v)]
    cv = row_stats(from_raw(conv_raw), r["conv"], [rt["conv"] for rt in rts])
    return out, o, st, cv


def block_req_check(task):
    """The whole layer on request i of a decode / MTP case: task = (case, hidden,
    i, out_raw [t_step, hidden], o_raw [t_step, h_v, d_v] (the core's output),
    ssm [h_v, d_v, d_k] (the state after pos + 1 tokens) or None, pos)."""
    case, hidden, i, out_raw, o_raw, ssm, pos = task
    s = int(case.slots[i])
    X = gi.block_input(case.seed, i, case.t_step, hidden, case.act)
    r, rts = _block_oracle(case, hidden, X, case.slot_conv(s), case.slot_ssm(s), True, keep=True)
    out = row_stats(from_raw(out_raw), r["block_out"], [rt["block_out"] for rt in rts])
    o = row_stats(from_raw(o_raw), r["core_out"], [rt["core_out"] for rt in rts], n=case.dims.d_v)
    st = None
    if ssm is not None:
        ref = r["ssm_states"][pos]
        st = [row_stats(ssm[h], ref[h], [rt["ssm_states"][pos][h] for rt in rts], n=ref[h].size)
              for h in range(case.dims.h_v)]
    return out, o, st


# ------------------------------------------- host baselines (timing only)
def prefill_oracle_heads(task) -> None:
    """The oracle on sequence i of a prefill case for the given V heads (None =
    all); task = (case, heads) or (case, heads, i).  Nothing is returned: the
    caller times it."""
    case, heads = task[0], task[1]
    i = task[2] if len(task) > 2 else 0
    oracle_prefill_seq(case, i, heads=heads)


def decode_oracle_requests(task) -> None:
    """The oracle on the given requests of a decode / MTP case; task = (case, requests)."""
    case, reqs = task
    d = case.dims
    p = case.params
    x, a, b, z = case.x(), case.a(), case.b(), case.z()
    for i in reqs:
        s = int(case.slots[i])
        O.layer_sequence(x[i], a[i], b[i], z[i], p.conv_w, None, p.A_log, p.dt_bias, p.norm_w, case.slot_conv(s),
                         case.slot_ssm(s), (d.h_k, d.h_v, d.d_k, d.d_v), 1.0, 1e-6, keep_states=case.t_step > 1)

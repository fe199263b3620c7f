"""Guard bands and sentinel pools: every entry point writes exactly the memory
it owns.

Each output buffer is the head of a larger allocation whose tail (a guard
band) and whose own bytes start as a sentinel byte pattern; the pools are
filled with the same pattern (as fp32 and bf16 values it is a tiny negative
number, a valid initial state).  After a call the guard bands must still hold
the sentinel, every slot no request names must be bitwise unchanged, and no
element of an output may still hold the sentinel (every row was written,
zeros for padding requests).  Values are checked elsewhere against the
oracle; these tests check the footprint, on ragged and padded batches.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_conv1d_amd as gdn
from tests.gpu_cases import DEV, i32, log, u8

pytestmark = pytest.mark.gpu

SENT = 0xA5
GUARD = 4096                      # guard band bytes after every buffer
QWEN = gi.QWEN3_NEXT
DIMS = gdn.Dims(QWEN.h_k, QWEN.h_v, QWEN.d_k, QWEN.d_v, QWEN.conv_w)


class Guarded:
    """A device tensor of `shape` at the head of a sentinel-filled allocation."""

    def __init__(self, shape, dtype, fill=None):
        self.n = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((self.n + GUARD,), SENT, dtype=torch.uint8, device=DEV)
        self.t = self.raw[:self.n].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def guard_ok(self) -> bool:
        return bool(torch.all(self.raw[self.n:] == SENT))

    def unwritten(self) -> int:
        """Elements whose bytes all still hold the sentinel."""
        es = self.t.element_size()
        b = self.raw[:self.n].view(-1, es)
        return int(torch.all(b == SENT, dim=1).sum())

    def slot_bytes(self, s: int) -> torch.Tensor:
        per = self.n // self.t.shape[0]
        return self.raw[s * per:(s + 1) * per]


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV, torch.bfloat16)


def _rand(key, shape):
    return _bf(gi.normal(key, shape))


def _pools(n_slots):
    conv = Guarded((n_slots, QWEN.c_ch, QWEN.conv_w - 1), torch.bfloat16)
    ssm = Guarded((n_slots, QWEN.h_v, QWEN.d_v, QWEN.d_k), torch.float32)
    return conv, ssm


def _untouched(pool: Guarded, slots) -> bool:
    return all(bool(torch.all(pool.slot_bytes(s) == SENT)) for s in slots)


@pytest.mark.parametrize("path", ["gdn_prefill", "three calls"])
def test_prefill_footprint(path):
    lengths = np.array([300, 0, 65, 1, 129])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, n, n_slots = int(cu[-1]), len(lengths), 8
    slots = np.array([6, 1, 3, 0, 7], np.int32)
    has_init = np.array([1, 0, 1, 1, 0], np.uint8)
    log(f"prefill footprint ({path}): lengths {lengths.tolist()} slots {slots.tolist()}")
    x, a, b = _rand((40, 1), (T, QWEN.c_ch)), _rand((40, 2), (T, QWEN.h_v)), _rand((40, 3), (T, QWEN.h_v))
    z = _rand((40, 4), (T, QWEN.h_v, QWEN.d_v))
    conv_w, norm_w = _rand((40, 5), (QWEN.c_ch, QWEN.conv_w)), _bf(np.linspace(0.5, 1.5, QWEN.d_v))
    A_log = torch.zeros(QWEN.h_v, device=DEV)
    dt_bias = torch.zeros(QWEN.h_v, device=DEV)
    conv, ssm = _pools(n_slots)
    o = Guarded((T, QWEN.h_v, QWEN.d_v), torch.bfloat16)
    bufs = [o, conv, ssm]
    if path == "gdn_prefill":
        ws = Guarded((gdn.prefill_workspace_size(DIMS, 0, n, T, 64),), torch.uint8)
        gdn.prefill(DIMS, x, conv_w, a, b, A_log, dt_bias, i32(cu), i32(slots), conv.t, ssm.t, u8(has_init), 64,
                    1.0, z, norm_w, o=o.t, workspace=ws.t)
        bufs.append(ws)
    else:
        y = Guarded((T, QWEN.c_ch), torch.bfloat16)
        g, beta = Guarded((T, QWEN.h_v), torch.float32), Guarded((T, QWEN.h_v), torch.float32)
        ws = Guarded((gdn.chunk_prefill_workspace_size(DIMS, 0, n, T, 64),), torch.uint8)
        gdn.conv1d_fwd(DIMS, x, conv_w, i32(cu), i32(slots), conv.t, u8(has_init), y=y.t)
        gdn.gating(a, b, A_log, dt_bias, g=g.t, beta=beta.t)
        gdn.chunk_prefill(DIMS, y.t, g.t, beta.t, i32(cu), i32(slots), ssm.t, u8(has_init), 64, 1.0, z, norm_w,
                          o=o.t, workspace=ws.t)
        bufs += [y, g, beta, ws]
        for t in (y, g, beta):
            assert t.unwritten() == 0
    torch.cuda.synchronize()
    assert all(t.guard_ok() for t in bufs), [t.guard_ok() for t in bufs]
    assert o.unwritten() == 0
    free = sorted(set(range(n_slots)) - set(slots.tolist()))
    assert _untouched(conv, free) and _untouched(ssm, free)
    # every named slot was written (its final state and window)
    assert not any(bool(torch.all(ssm.slot_bytes(s) == SENT)) for s in slots)


@pytest.mark.parametrize("t_step,path", [(1, "gdn_decode"), (3, "gdn_decode"), (1, "two calls"), (3, "two calls")])
def test_decode_footprint(t_step, path):
    n, n_slots = 6, 40
    perm = np.random.default_rng(41).permutation(n_slots).astype(np.int32)
    slots = perm[:n].copy()
    slots[4] = -1                                          # a padding request
    out_slots = None
    if t_step > 1:
        out_slots = perm[n:n + n * t_step].reshape(n, t_step).copy()
        out_slots[2, 1] = -1                               # a position nobody keeps
    log(f"decode footprint ({path}): t_step {t_step} slots {slots.tolist()}")
    x = _rand((42, t_step), (n, t_step, QWEN.c_ch))
    a, b = _rand((43, t_step), (n, t_step, QWEN.h_v)), _rand((44, t_step), (n, t_step, QWEN.h_v))
    z = _rand((45, t_step), (n, t_step, QWEN.h_v, QWEN.d_v))
    conv_w, norm_w = _rand((46, 1), (QWEN.c_ch, QWEN.conv_w)), _bf(np.linspace(0.5, 1.5, QWEN.d_v))
    A_log = torch.zeros(QWEN.h_v, device=DEV)
    dt_bias = torch.zeros(QWEN.h_v, device=DEV)
    conv, ssm = _pools(n_slots)
    o = Guarded((n, t_step, QWEN.h_v, QWEN.d_v), torch.bfloat16)
    os_ = None if out_slots is None else i32(out_slots)
    bufs = [o, conv, ssm]
    if path == "gdn_decode":
        gdn.decode(DIMS, x, conv_w, a, b, A_log, dt_bias, i32(slots), conv.t, ssm.t, os_, 1.0, z, norm_w, o=o.t)
    else:
        y = Guarded((n, t_step, QWEN.c_ch), torch.bfloat16)
        gdn.conv1d_update(DIMS, x, conv_w, conv.t, i32(slots), os_, y=y.t)
        gdn.recurrent_decode(DIMS, y.t, a, b, A_log, dt_bias, ssm.t, i32(slots), os_, 1.0, z, norm_w, o=o.t)
        bufs.append(y)
    torch.cuda.synchronize()
    assert all(t.guard_ok() for t in bufs), [t.guard_ok() for t in bufs]
    assert o.unwritten() == 0
    assert bool(torch.all(o.t[4] == 0))                    # padding request: zero rows
    # a padding request touches no pool entry, its positions included
    live = slots >= 0
    written = set(int(s) for s in slots[live]) if out_slots is None else \
        set(int(s) for s in out_slots[live].ravel() if s >= 0)
    free = sorted(set(range(n_slots)) - written)
    assert _untouched(conv, free) and _untouched(ssm, free)
    assert not any(bool(torch.all(ssm.slot_bytes(s) == SENT)) for s in written)


def test_state_copy_footprint():
    n_slots = 12
    conv, ssm = _pools(n_slots)
    src, dst = np.array([0, 3, -1, 5], np.int32), np.array([7, 9, 2, -1], np.int32)
    for s in (0, 3, 5):
        ssm.t[s].copy_(_rand((52, s), tuple(ssm.t.shape[1:])).float())
        conv.t[s].copy_(_rand((53, s), tuple(conv.t.shape[1:])))
    before = ssm.raw.clone(), conv.raw.clone()
    gdn.state_copy(DIMS, ssm.t, i32(src), i32(dst), conv.t)
    torch.cuda.synchronize()
    assert ssm.guard_ok() and conv.guard_ok()
    assert torch.equal(ssm.t[7], ssm.t[0]) and torch.equal(ssm.t[9], ssm.t[3])
    assert torch.equal(conv.t[7], conv.t[0]) and torch.equal(conv.t[9], conv.t[3])
    for pool, old in zip((ssm, conv), before):
        per = pool.n // n_slots
        for s in set(range(n_slots)) - {7, 9}:
            assert torch.equal(pool.raw[s * per:(s + 1) * per], old[s * per:(s + 1) * per])


@pytest.mark.parametrize("T", [300, 1])
def test_block_footprint(T):
    hidden = 512
    vd = QWEN.h_v * QWEN.d_v
    log(f"block footprint: T {T} hidden {hidden}")
    X = _rand((47, T), (T, hidden))
    w = _rand((48, 1), (hidden,)) * 0.1
    w_qkvz = _rand((49, 1), (QWEN.c_ch + vd, hidden)) * 0.05
    w_ba = _rand((50, 1), (2 * QWEN.h_v, hidden)) * 0.05
    w_out = _rand((51, 1), (hidden, vd)) * 0.05
    xn = Guarded((T, hidden), torch.bfloat16)
    qkv, z = Guarded((T, QWEN.c_ch), torch.bfloat16), Guarded((T, QWEN.h_v, QWEN.d_v), torch.bfloat16)
    b, a = Guarded((T, QWEN.h_v), torch.bfloat16), Guarded((T, QWEN.h_v), torch.bfloat16)
    y = Guarded((T, hidden), torch.bfloat16)
    gdn.rmsnorm_gemma(X, w, 1e-6, out=xn.t)
    gdn.in_proj(DIMS, xn.t, w_qkvz, w_ba, qkv=qkv.t, z=z.t, b=b.t, a=a.t)
    gdn.out_proj(DIMS, z.t, w_out, X, y=y.t)
    torch.cuda.synchronize()
    for t in (xn, qkv, z, b, a, y):
        assert t.guard_ok() and t.unwritten() == 0


def _slot_flags(n_slots, lst):
    seen, out = set(), []
    for v in lst:
        f = 1 if (v < -1 or v >= n_slots) else 0
        if 0 <= v < n_slots:
            f |= 2 if v in seen else 0
            seen.add(v)
        out.append(f)
    return np.array(out, np.int32)


@pytest.mark.parametrize("case", ["valid", "faulty", "large", "empty"])
def test_check_slots(case):
    """gdn_check_slots flags padding other than -1 and repeated in-range slots,
    exactly as a set scan over the concatenated list does."""
    rng = np.random.default_rng(54)
    n_slots = 640
    if case == "valid":
        perm = rng.permutation(n_slots).astype(np.int32)
        slots, out = perm[:128].copy(), perm[128:640].reshape(128, 4).copy()
        slots[[3, 70]] = -1
        out[5, 2] = -1
    elif case == "faulty":
        slots = np.array([4, 9, 4, -1, -1, 640, -7, 12], np.int32)
        out = np.array([[9, 13], [12, 2 ** 30], [13, -1]], np.int32)
    elif case == "large":
        slots = rng.integers(-3, n_slots + 3, 1024).astype(np.int32)
        out = rng.integers(-3, n_slots + 3, (1024, 4)).astype(np.int32)
    else:
        slots, out = np.zeros(0, np.int32), None
    flags = gdn.check_slots(n_slots, i32(slots), None if out is None else i32(out))
    torch.cuda.synchronize()
    ref = _slot_flags(n_slots, np.concatenate([slots.ravel()] + ([] if out is None else [out.ravel()])).tolist())
    got = flags.cpu().numpy()
    assert np.array_equal(got, ref), np.nonzero(got != ref)
    if case == "valid":
        assert not got.any()
    if case == "faulty":
        assert got.tolist() == [0, 0, 2, 0, 0, 1, 1, 0, 2, 0, 2, 1, 2, 0]

"""GPU tests of the layer around the core: the Gemma RMSNorm, the MFMA
projections and the whole layer (norm -> in_proj -> prefill / decode ->
out_proj), all through the C ABI, against the fp64 oracle.

Projections are checked bit-exactly on small integers (every product and
partial sum is exact in fp32, so the result is the one rounding of the exact
integer to bf16).  The norm is checked elementwise to within one bf16 rounding
(unit roundoff 2^-8) plus fp32 slack; the whole layer by the per-row parity rule of
the other GPU tests, with the oracle's sensitivity taken over every activation
the layer hands from one kernel to the next.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_conv1d_amd as gdn
from oracle import gdn_oracle as O
from tests.gpu_cases import ILL_MAX_LAYER, TOL, Score, dev, host, host_raw, i32, log, run_map, u8
from tests.oracle_pool import block_req_check, block_seq_check

pytestmark = pytest.mark.gpu

QWEN = gi.QWEN3_NEXT
SMALL = gi.Dims(1, 2, 16, 16, 4)


def _bf(x):
    return dev(x, torch.bfloat16)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns of x (exact values below 2^24) rounded to bf16."""
    return (gi.round_bf16(np.asarray(x, np.float32)).view(np.uint32) >> 16).astype(np.uint16)


def _small_ints(seed, shape, lo=-2, hi=2, density=0.5):
    rng = np.random.default_rng(seed)
    v = rng.integers(lo, hi + 1, shape).astype(np.float32)
    return v * (rng.random(shape) < density)


# kernel and tile choices (in_proj / out_proj): 64 x 128 staged through LDS /
# 64 x 32 split over k; 128 x 128 / 64 x 32 split over k (a partial last row
# tile); 128 x 128 / 64 x 64; 256 x 256 straight into LDS plus the 64-wide
# last column tile as 64 x 32 / 128 x 128; 256 x 256 plus the last column
# tile / 128 x 256 with three LDS buffers, at 4096 rows and with a partial
# last row tile at 4100; one row (64 x 32 split over k, the four output
# segments / the same); k not a multiple of 64 with 2-column segments (column
# by column)
@pytest.mark.parametrize("dims,hidden,T", [(QWEN, 2048, 256), (QWEN, 2048, 300), (QWEN, 2048, 600),
                                           (QWEN, 2048, 2600), (QWEN, 2048, 4096), (QWEN, 2048, 4100),
                                           (QWEN, 1024, 1), (SMALL, 24, 37)])
def test_projections_exact_on_small_integers(dims, hidden, T):
    log(f"projections: dims {dims} hidden {hidden} T {T}")
    vd = dims.h_v * dims.d_v
    X = _small_ints((1, T), (T, hidden))
    Wq = _small_ints((2, T), (dims.c_ch + vd, hidden))
    Wba = _small_ints((3, T), (2 * dims.h_v, hidden))
    Wo = _small_ints((4, T), (hidden, vd), density=0.25)
    O_ = _small_ints((5, T), (T, vd))
    R = _small_ints((6, T), (T, hidden), -8, 8, 1.0)
    gd = gdn.Dims(dims.h_k, dims.h_v, dims.d_k, dims.d_v, dims.conv_w)
    qkv, z, b, a = gdn.in_proj(gd, _bf(X), _bf(Wq), _bf(Wba))
    y = gdn.out_proj(gd, _bf(O_), _bf(Wo), _bf(R))
    y0 = gdn.out_proj(gd, _bf(O_), _bf(Wo))
    torch.cuda.synchronize()
    P, Q = O.linear(X, Wq), O.linear(X, Wba)
    assert np.abs(P).max() < 2 ** 24 and np.abs(O.linear(O_, Wo)).max() < 2 ** 24   # exact in fp32
    c = dims.c_ch
    assert np.array_equal(_bits(qkv), _bf16_bits(P[:, :c]))
    assert np.array_equal(_bits(z).reshape(T, vd), _bf16_bits(P[:, c:]))
    assert np.array_equal(_bits(b), _bf16_bits(Q[:, :dims.h_v]))
    assert np.array_equal(_bits(a), _bf16_bits(Q[:, dims.h_v:]))
    assert np.array_equal(_bits(y0), _bf16_bits(O.linear(O_, Wo)))
    assert np.array_equal(_bits(y), _bf16_bits(O.linear(O_, Wo) + R))


@pytest.mark.parametrize("rows,hidden", [(1, 2048), (513, 2048), (7, 24)])
def test_gemma_rmsnorm(rows, hidden):
    X = gi.round_bf16(gi.normal((7, rows), (rows, hidden)) * np.float32(3.0))
    w = gi.uniform((8, rows), (hidden,), -0.5, 0.5, "bf16")
    w[:3] = (-1.0, 0.0, 1.0)[: min(3, hidden)]
    out = gdn.rmsnorm_gemma(_bf(X), _bf(w), 1e-6)
    torch.cuda.synchronize()
    ref = O.gemma_rmsnorm(X, w, 1e-6)
    err = np.abs(host(out) - ref)
    # one RNE rounding to bf16 (unit roundoff 2^-8) plus fp32 arithmetic
    bound = 2.0 ** -8 * (1 + 2e-3) * np.abs(ref) + 1e-30
    assert np.all(err <= bound), float((err / bound).max())
    assert np.all(host(out)[:, 0] == 0.0)      # weight -1


def _weights(case, hidden):
    w = gi.block_weights(case.seed, case.dims, hidden, case.act)
    return gdn.BlockWeights(_bf(w.norm_w), _bf(w.w_qkvz), _bf(w.w_ba), _bf(w.w_out))


@pytest.mark.parametrize("lengths,init,residual", [((300, 77), True, False), ((2600,), False, True)])
def test_block_prefill_parity(lengths, init, residual):
    hidden = gi.HIDDEN
    case = gi.varlen_case(seed=11, lengths=np.array(lengths), n_slots=4, dims=QWEN)
    if not init:
        case.has_init[:] = 0
    log(f"block prefill: lengths {lengths} init {init} residual {residual}")
    d, p = case.dims, case.params
    X = np.concatenate([gi.block_input(case.seed, i, L, hidden) for i, L in enumerate(lengths)])
    conv0 = np.stack([case.slot_conv(s) for s in range(case.n_slots)])
    ssm0 = np.stack([case.slot_ssm(s) for s in range(case.n_slots)])
    conv_pool, ssm_pool = _bf(conv0), dev(ssm0, torch.float32)
    y = gdn.block_prefill(gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w), _bf(X), _weights(case, hidden), _bf(p.conv_w), dev(p.A_log, torch.float32),
                          dev(p.dt_bias, torch.float32), i32(case.cu_seqlens), i32(case.slots), conv_pool, ssm_pool,
                          u8(case.has_init), 64, 1.0, _bf(p.norm_w), 1e-6, 1e-6, residual, intermediates=True)
    y, mid = y
    torch.cuda.synchronize()
    y_raw, o_raw, ssm_h, conv_raw = host_raw(y), host_raw(mid["o"]), ssm_pool.cpu().numpy(), host_raw(conv_pool)
    cu = case.cu_seqlens
    tasks = [(case, hidden, i, residual, y_raw[cu[i]:cu[i + 1]], o_raw[cu[i]:cu[i + 1]], ssm_h[case.slots[i]],
              conv_raw[case.slots[i]]) for i in range(case.n_seq)]
    res = run_map(block_seq_check, tasks)
    so, sco = Score(TOL["bf16"], ill_max=None), Score(TOL["bf16"], ill_max=ILL_MAX_LAYER)
    ss, sc = Score(TOL["bf16"]), Score(TOL["bf16"])
    for i, (out, o, st, cv) in enumerate(res):
        so.add_stats(*out, label=f"seq {i}")
        sco.add_stats(*o, label=f"seq {i} core")
        for h, stat in enumerate(st):
            ss.add_stats(*stat, label=f"seq {i} head {h}")
        sc.add_stats(*cv, label=f"seq {i} conv")
    log(f"block prefill out: {so}\ncore out: {sco}\nstates: {ss}\nconv states: {sc}")
    assert so.ok() and sco.ok() and ss.ok() and sc.ok()
    # slots no sequence owns are untouched
    owned = set(int(s) for s in case.slots)
    for s in range(case.n_slots):
        if s not in owned:
            assert np.array_equal(ssm_h[s], ssm0[s].astype(np.float32))


@pytest.mark.parametrize("n,t_step", [(8, 1), (6, 3)])
def test_block_decode_parity(n, t_step):
    hidden = gi.HIDDEN
    case = (gi.decode_case(seed=12, n=n, n_slots=2 * n) if t_step == 1 else gi.mtp_case(seed=13, n=n, t_step=t_step))
    log(f"block decode: n {n} t_step {t_step}")
    d, p = case.dims, case.params
    X = np.stack([gi.block_input(case.seed, i, t_step, hidden) for i in range(n)])
    conv0 = np.stack([case.slot_conv(s) for s in range(case.n_slots)])
    ssm0 = np.stack([case.slot_ssm(s) for s in range(case.n_slots)])
    conv_pool, ssm_pool = _bf(conv0), dev(ssm0, torch.float32)
    out_slots = None if case.out_slots is None else i32(case.out_slots)
    y = gdn.block_decode(gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w), _bf(X), _weights(case, hidden), _bf(p.conv_w), dev(p.A_log, torch.float32),
                         dev(p.dt_bias, torch.float32), i32(case.slots), conv_pool, ssm_pool, out_slots, 1.0,
                         _bf(p.norm_w), 1e-6, 1e-6, True, intermediates=True)
    y, mid = y
    torch.cuda.synchronize()
    y_raw, o_raw, ssm_h = host_raw(y), host_raw(mid["o"]), ssm_pool.cpu().numpy()
    tasks = []
    for i in range(n):
        pos = t_step - 1
        slot = case.slots[i] if case.out_slots is None else case.out_slots[i][pos]
        tasks.append((case, hidden, i, y_raw[i], o_raw[i], ssm_h[slot], pos))
    so, sco, ss = Score(TOL["bf16"], ill_max=None), Score(TOL["bf16"], ill_max=ILL_MAX_LAYER), Score(TOL["bf16"])
    for i, (out, o, st) in enumerate(run_map(block_req_check, tasks)):
        so.add_stats(*out, label=f"req {i}")
        sco.add_stats(*o, label=f"req {i} core")
        for h, stat in enumerate(st):
            ss.add_stats(*stat, label=f"req {i} head {h}")
    log(f"block decode out: {so}\ncore out: {sco}\nstates: {ss}")
    assert so.ok() and sco.ok() and ss.ok()
    if case.out_slots is not None:    # MTP: home slots are read only
        for s in case.slots:
            assert np.array_equal(ssm_h[s], ssm0[s].astype(np.float32))

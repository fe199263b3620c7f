"""Every row of the chain launch table gives results equal to those of the
same sequences run one call each (one sequence is 32 chains: the first row's
shape).  States and conv states are bitwise equal for every shape: each
chain's accumulators see the same MFMA order whatever the d_v tiles per
workgroup and prefetch depth.  Outputs are bitwise equal too, except for the
whole-d_v chain (ntw 8), which computes them itself with its products and
norm sum in another order: there every output is within one bf16 unit in the
last place of the output pass's."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_conv1d_amd as gdn
from tests.gpu_cases import bf16_ulps, dev, host_raw, i32, log, u8
from tests.test_launch_table import table_rows

pytestmark = pytest.mark.gpu

ROWS, _ = table_rows()
D = gdn.Dims(16, 32, 128, 128, 4)


def _n_seq(r: int) -> int:
    """A sequence count whose 32 n chains select row r (and no earlier row)."""
    lo = ROWS[r - 1][0] if r else 0
    hi = ROWS[r][0]
    n = hi // D.h_v if hi is not None else lo // D.h_v + 1
    assert lo < n * D.h_v and (hi is None or n * D.h_v <= hi)
    return n


@pytest.mark.parametrize("r", range(len(ROWS)))
def test_table_row_matches_single_sequence_calls(r):
    n = _n_seq(r)
    lengths = np.random.default_rng(60 + r).integers(40, 200, n)
    log(f"launch table row {r} {ROWS[r]}: {n} sequences, {int(lengths.sum())} tokens")
    _check_batch_against_single_calls(lengths, 60 + r, ROWS[r][2] >= 8)


def test_longest_first_chains_match_single_sequence_calls():
    """More than 8 sequences: the chunk index kernel runs and the chain with
    output takes its sequences longest first (ties by index).  Lengths with
    ties, an empty and a one-token sequence; results as one call each."""
    lengths = np.array([150, 40, 150, 0, 300, 1, 64, 65, 150, 200, 7, 129])
    assert len(lengths) * D.h_v > ROWS[-2][0]  # the whole-d_v row
    log(f"longest-first order: {len(lengths)} sequences, {int(lengths.sum())} tokens")
    _check_batch_against_single_calls(lengths, 70, True)


def _check_batch_against_single_calls(lengths, seed, whole_dv):
    n = len(lengths)
    case = gi.varlen_case(seed=seed, lengths=lengths, n_slots=n, dims=gi.QWEN3_NEXT)
    p = case.params
    bf = lambda v: dev(v, torch.bfloat16)
    f32 = lambda v: dev(v, torch.float32)
    conv0 = np.stack([case.slot_conv(s) for s in range(n)])
    ssm0 = np.stack([case.slot_ssm(s) for s in range(n)])
    xs = [case.seq_x(i) for i in range(n)]
    a_s, b_s, z_s = [case.seq_a(i) for i in range(n)], [case.seq_b(i) for i in range(n)], [case.seq_z(i) for i in range(n)]
    common = (bf(p.conv_w),)
    conv_pool, ssm_pool = bf(conv0), f32(ssm0)
    out = gdn.prefill(D, bf(np.concatenate(xs)), *common, bf(np.concatenate(a_s)), bf(np.concatenate(b_s)),
                      f32(p.A_log), f32(p.dt_bias), i32(case.cu_seqlens), i32(case.slots), conv_pool, ssm_pool,
                      u8(case.has_init), 64, 1.0, bf(np.concatenate(z_s)), bf(p.norm_w))
    torch.cuda.synchronize()
    out_b, ssm_b, conv_b = host_raw(out), ssm_pool.cpu().numpy(), host_raw(conv_pool)
    for i in range(n):
        s = int(case.slots[i])
        if lengths[i] == 0:  # no tokens: the slot's states stay as they were
            assert np.array_equal(ssm0[s], ssm_b[s]), f"sequence {i}: state of an empty sequence"
            assert np.array_equal(host_raw(bf(conv0))[s], conv_b[s]), f"sequence {i}: conv state of an empty sequence"
            continue
        cp, sp = bf(conv0), f32(ssm0)
        o1 = gdn.prefill(D, bf(xs[i]), *common, bf(a_s[i]), bf(b_s[i]), f32(p.A_log), f32(p.dt_bias),
                         i32([0, len(xs[i])]), i32([s]), cp, sp, u8([1]), 64, 1.0, bf(z_s[i]), bf(p.norm_w))
        torch.cuda.synchronize()
        lo, hi = case.cu_seqlens[i], case.cu_seqlens[i + 1]
        if whole_dv:
            assert bf16_ulps(host_raw(o1), out_b[lo:hi]) <= 1, f"sequence {i}: output beyond one unit in the last place"
        else:
            assert np.array_equal(host_raw(o1), out_b[lo:hi]), f"sequence {i}: output"
        assert np.array_equal(sp.cpu().numpy()[s], ssm_b[s]), f"sequence {i}: state"
        assert np.array_equal(host_raw(cp)[s], conv_b[s]), f"sequence {i}: conv state"

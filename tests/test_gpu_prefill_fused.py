"""The single-call prefill (gdn_prefill): conv1d + SiLU and the gates
computed inside the chunk kernels.  It must reproduce the three separate calls
(gdn_conv1d_fwd, gdn_gating, gdn_chunk_prefill on the split path) bit for bit,
since it runs the same arithmetic in the same order, and it is checked
against the oracle on its own as well."""
from __future__ import annotations


import numpy as np
import pytest
import torch

import gdn_inputs as gi
from tests.gpu_cases import DevPrefill, compare_prefill, log
from tests.test_gpu_parity import SMALL_LENGTHS

pytestmark = pytest.mark.gpu


def _small_case(act, d, chunk, conv_w, seed=31):
    dims = gi.Dims(2, 4, d, d, conv_w)
    case = gi.varlen_case(seed=seed, dims=dims, act=act, lengths=np.array(SMALL_LENGTHS), n_slots=12, chunk=chunk)
    case.has_init = np.array([1, 0, 1, 1, 0, 1, 0, 1], np.uint8)
    case.slots[5] = -1                                           # padding entry
    return case


@pytest.mark.parametrize("act,d,chunk,conv_w", [("bf16", 128, 64, 4), ("f32", 128, 64, 4), ("f32", 128, 32, 4), ("bf16", 64, 32, 3),
                                                ("f32", 16, 16, 2), ("bf16", 32, 16, 4), ("bf16", 128, 16, 2)])
def test_fused_equals_separate_calls(act, d, chunk, conv_w):
    case = _small_case(act, d, chunk, conv_w)
    dp = DevPrefill(case)
    conv0, ssm0 = dp.conv_pool.clone(), dp.ssm_pool.clone()
    ref, *_ = dp.run()
    ref_ssm, ref_conv = dp.ssm_pool.clone(), dp.conv_pool.clone()
    dp.conv_pool.copy_(conv0)
    dp.ssm_pool.copy_(ssm0)
    out = dp.run_fused()
    torch.cuda.synchronize()
    diff = float((out.float() - ref.float()).abs().max())
    log(f"{act} d={d} C={chunk} W={conv_w}: max |fused - separate| = {diff:.3g}")
    assert torch.equal(out, ref)
    assert torch.equal(dp.ssm_pool, ref_ssm)
    assert torch.equal(dp.conv_pool, ref_conv)


@pytest.mark.parametrize("act,d,chunk", [("bf16", 128, 64), ("f32", 64, 32)])
def test_fused_small_varlen_vs_oracle(act, d, chunk):
    case = _small_case(act, d, chunk, 4, seed=32)
    dp = DevPrefill(case)
    conv_before, ssm_before = dp.conv_pool.clone(), dp.ssm_pool.clone()
    out = dp.run_fused()
    torch.cuda.synchronize()
    real = [i for i in range(case.n_seq) if case.slots[i] >= 0]
    w = compare_prefill(dp, out, seqs=real)
    lo, hi = case.cu_seqlens[5], case.cu_seqlens[6]
    assert torch.all(out[lo:hi] == 0), "padding rows must be zero"
    untouched = sorted(set(range(case.n_slots)) - {int(s) for s in case.slots if s >= 0})
    assert torch.equal(dp.conv_pool[untouched], conv_before[untouched])
    assert torch.equal(dp.ssm_pool[untouched], ssm_before[untouched])
    log(f"fused {act} d={d} C={chunk}: out [{w['out']}] ssm [{w['ssm']}] conv {w['conv']:.1e}")
    assert w["conv"] == 0.0 and w["out"].ok() and w["ssm"].ok()


def test_fused_single_4096_vs_oracle():
    case = gi.prefill_case()
    dp = DevPrefill(case)
    out = dp.run_fused()
    torch.cuda.synchronize()
    w = compare_prefill(dp, out)
    log(f"fused prefill 4096: out [{w['out']}] ssm [{w['ssm']}]")
    assert w["out"].ok() and w["ssm"].ok() and w["conv"] == 0.0


@pytest.mark.parametrize("h_k,h_v", [(8, 16), (4, 8)])
def test_fused_at_tensor_parallel_rank_heads(h_k, h_v):
    """gdn_prefill at one tensor-parallel rank's head counts (tp = 2 and 4 of
    the 16/32-head layout), against the oracle: two sequences, one with
    history, sampled V heads spanning both halves of each QK pairing."""
    dims = gi.Dims(h_k, h_v, 128, 128, 4)
    case = gi.varlen_case(seed=41 + h_k, dims=dims, lengths=np.array([300, 77]), n_slots=4)
    case.has_init = np.array([0, 1], np.uint8)
    dp = DevPrefill(case)
    out = dp.run_fused()
    torch.cuda.synchronize()
    w = compare_prefill(dp, out, heads=[0, 1, h_v - 2, h_v - 1])
    log(f"h_k={h_k} h_v={h_v}: out [{w['out']}] ssm [{w['ssm']}] conv {w['conv']:.1e}")
    assert w["out"].ok() and w["ssm"].ok() and w["conv"] == 0.0

"""gdn_prefill_noalloc (the static-scratch prefill for callers that cannot
allocate) against gdn_prefill with a caller workspace: bitwise equal outputs,
recurrent states and conv states, on two calls in a row, the second smaller,
through the C ABI; and the size limit rejected before any launch."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_conv1d_amd as gdn
from gated_deltanet_conv1d_amd import binding
from tests.gpu_cases import DevPrefill, log

pytestmark = pytest.mark.gpu

def _lib():
    return gdn.lib()  # (argument types from the binding's signature table)


def _noalloc(L, dp, T, n):
    """gdn_prefill_noalloc on the first n sequences (T tokens) of a DevPrefill."""
    d = dp.dims
    o = torch.empty((T, d.h_v, d.d_v), dtype=dp.x.dtype, device="cuda")
    p = lambda t: None if t is None else t.data_ptr()
    rc = L.gdn_prefill_noalloc(ctypes.byref(binding._CDims(*d)), binding._act(dp.x), n, T, dp.case.chunk, 1.0,
                               p(dp.x), p(dp.conv_w), None, p(dp.a), p(dp.b), p(dp.A_log), p(dp.dt_bias), p(dp.cu),
                               p(dp.slots), p(dp.has_init), p(dp.conv_pool), p(dp.ssm_pool), dp.ssm_pool.shape[0],
                               p(o), p(dp.z), p(dp.norm_w), 1e-6, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, L.gdn_status_string(rc)
    return o


def test_noalloc_equals_prefill_on_two_calls():
    L = _lib()
    case = gi.varlen_case(seed=51, lengths=np.array([700, 65, 1, 300, 129]), n_slots=8)
    dp = DevPrefill(case)
    conv0, ssm0 = dp.conv_pool.clone(), dp.ssm_pool.clone()
    for n in (5, 2):  # the second call is smaller
        T = int(case.cu_seqlens[n])
        cu = dp.cu[:n + 1]
        dp.conv_pool.copy_(conv0)
        dp.ssm_pool.copy_(ssm0)
        ref = gdn.prefill(dp.dims, dp.x[:T], dp.conv_w, dp.a[:T], dp.b[:T], dp.A_log, dp.dt_bias, cu, dp.slots[:n],
                          dp.conv_pool, dp.ssm_pool, dp.has_init[:n], case.chunk, 1.0, dp.z[:T], dp.norm_w)
        torch.cuda.synchronize()
        ref_state, ref_conv = dp.ssm_pool.clone(), dp.conv_pool.clone()
        dp.conv_pool.copy_(conv0)
        dp.ssm_pool.copy_(ssm0)
        saved = (dp.cu, dp.slots, dp.has_init)
        dp.cu, dp.slots, dp.has_init = cu, dp.slots[:n], dp.has_init[:n]
        got = _noalloc(L, dp, T, n)
        dp.cu, dp.slots, dp.has_init = saved
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{n} sequences: output"
        assert torch.equal(dp.ssm_pool, ref_state), f"{n} sequences: recurrent states"
        assert torch.equal(dp.conv_pool, ref_conv), f"{n} sequences: conv states"
        log(f"gdn_prefill_noalloc == gdn_prefill bitwise: {n} sequences, {T} tokens")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    L = _lib()
    limit = L.gdn_prefill_noalloc_limit()
    assert limit == 256 << 20
    d = binding._CDims(16, 32, 128, 128, 4)
    ws = lambda n, T: binding.lib().gdn_prefill_workspace_size(ctypes.byref(d), 0, n, T, 64)
    assert ws(20, 4096) <= limit < ws(1, 8192)
    fake = 0x1000  # never launched with: the size check returns first
    rc = L.gdn_prefill_noalloc(ctypes.byref(d), 0, 1, 8192, 64, 1.0, *([fake] * 12), 1, fake, None, None, 1e-6, None)
    assert rc == -8  # GDN_ERR_TOO_LARGE

"""HIP-graph capture of the hot path.

Every entry point launches kernels only (no allocation, no host sync, no
memset), so a prefill step (conv1d + gating + chunked rule) and a decode step
(conv update + recurrent step) can be captured once and replayed.  Each replay
is checked bitwise against the eager result, with the program's own eager work
and synchronisations between replays.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_conv1d_amd as gdn
from tests.gpu_cases import DevPrefill, dev, i32

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up off the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


# 4 sequences: no chunk index, the split chain and the output pass; 40 (160
# chains): the chunk index with the longest-first order and the chain that
# computes the output itself
PREFILL_BATCHES = {"4 sequences": [77, 190, 64, 1],
                   "40 sequences": list(np.random.default_rng(22).integers(0, 101, 40))}


@pytest.mark.parametrize("single_call", [False, True])
@pytest.mark.parametrize("batch", list(PREFILL_BATCHES))
def test_prefill_graph_replays_match_eager(batch, single_call):
    dims = gi.Dims(2, 4, 128, 128, 4)
    lengths = np.array(PREFILL_BATCHES[batch])
    case = gi.varlen_case(seed=21, dims=dims, lengths=lengths, n_slots=len(lengths) + 2)
    dp = DevPrefill(case)
    d = dp.dims
    T = case.t_total
    conv0, ssm0 = dp.conv_pool.clone(), dp.ssm_pool.clone()
    y = torch.empty_like(dp.x)
    g = torch.empty((T, d.h_v), dtype=torch.float32, device="cuda")
    beta = torch.empty_like(g)
    o = torch.empty((T, d.h_v, d.d_v), dtype=dp.x.dtype, device="cuda")
    ws = torch.empty(max(gdn.chunk_prefill_workspace_size(d, 0, case.n_seq, T, case.chunk),
                         gdn.prefill_workspace_size(d, 0, case.n_seq, T, case.chunk)), dtype=torch.uint8,
                     device="cuda")

    def step():
        if single_call:
            gdn.prefill(d, dp.x, dp.conv_w, dp.a, dp.b, dp.A_log, dp.dt_bias, dp.cu, dp.slots, dp.conv_pool,
                        dp.ssm_pool, dp.has_init, case.chunk, 1.0, dp.z, dp.norm_w, 1e-6, o=o, workspace=ws)
            return
        gdn.conv1d_fwd(d, dp.x, dp.conv_w, dp.cu, dp.slots, dp.conv_pool, dp.has_init, y=y)
        gdn.gating(dp.a, dp.b, dp.A_log, dp.dt_bias, g=g, beta=beta)
        gdn.chunk_prefill(d, y, g, beta, dp.cu, dp.slots, dp.ssm_pool, dp.has_init, case.chunk, 1.0, dp.z,
                          dp.norm_w, 1e-6, o=o, workspace=ws)

    def reset():
        dp.conv_pool.copy_(conv0)
        dp.ssm_pool.copy_(ssm0)

    reset()
    step()
    torch.cuda.synchronize()
    ref = (o.clone(), dp.ssm_pool.clone(), dp.conv_pool.clone())

    reset()
    graph = _capture(step)
    for k in range(3):
        reset()
        o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]), f"replay {k}: out"
        assert torch.equal(dp.ssm_pool, ref[1]), f"replay {k}: state"
        assert torch.equal(dp.conv_pool, ref[2]), f"replay {k}: conv state"
        # eager work between replays, on other buffers
        dp.run()
        torch.cuda.synchronize()


@pytest.mark.parametrize("single_call", [False, True])
@pytest.mark.parametrize("pad", [0, 3])
def test_decode_graph_replays_match_eager(pad, single_call):
    """The decode step (gdn_conv1d_update + gdn_recurrent_decode, or the single
    gdn_decode call) captured once and replayed; with pad > 0 the last entries
    of the bucket are pad slots (-1), as a serving loop fills a fixed-size
    bucket: their output rows are zero and no pool slot they could name changes."""
    case = gi.decode_case(seed=22, n=8, n_slots=16, dims=gi.Dims(2, 4, 128, 128, 4))
    if pad:
        case.slots[case.n - pad:] = -1
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    bf = lambda v: dev(v, torch.bfloat16)
    x, a, b, z = bf(case.x()), bf(case.a()), bf(case.b()), bf(case.z())
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log, dt_bias = dev(p.A_log, torch.float32), dev(p.dt_bias, torch.float32)
    slots = i32(case.slots)
    gen = torch.Generator(device="cuda").manual_seed(3)
    ssm0 = torch.randn((case.n_slots, d.h_v, d.d_v, d.d_k), device="cuda", generator=gen) * 0.02
    conv0 = torch.randn((case.n_slots, d.c_ch, d.conv_w - 1), device="cuda", generator=gen).to(torch.bfloat16)
    ssm, conv = ssm0.clone(), conv0.clone()
    y = torch.empty_like(x)
    o = torch.empty((case.n, 1, d.h_v, d.d_v), dtype=torch.bfloat16, device="cuda")

    def step():
        if single_call:
            gdn.decode(dims, x, conv_w, a, b, A_log, dt_bias, slots, conv, ssm, None, 1.0, z, norm_w, 1e-6, o=o)
            return
        gdn.conv1d_update(dims, x, conv_w, conv, slots, y=y)
        gdn.recurrent_decode(dims, y, a, b, A_log, dt_bias, ssm, slots, None, 1.0, z, norm_w, 1e-6, o=o)

    def reset():
        ssm.copy_(ssm0)
        conv.copy_(conv0)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), ssm.clone(), conv.clone())
    reset()
    graph = _capture(step)
    for k in range(3):
        reset()
        o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(ssm, ref[1]) and torch.equal(conv, ref[2]), f"replay {k}"
        if pad:
            assert torch.all(o[case.n - pad:] == 0), "pad rows must be zero"
            live = set(int(v) for v in case.slots[:case.n - pad])
            for sl in range(case.n_slots):
                if sl not in live:
                    assert torch.equal(ssm[sl], ssm0[sl]) and torch.equal(conv[sl], conv0[sl]), f"slot {sl} touched"
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("single_call", [False, True])
def test_mtp_bucket_graph(single_call):
    """The MTP draft step as a serving loop runs it: a fixed bucket of requests,
    each with mtp_step + 1 rows (so the bucket's row count is a multiple of
    mtp_step + 1), the draft step and the commit copy captured as one graph.
    Pad requests (slot -1, out slots -1) leave zero rows and no pool slot
    changed.  The accept lengths live in device index buffers the graph reads
    at replay: two different accept patterns replay bitwise equal to eager."""
    mtp_step = 3
    t_step = mtp_step + 1
    bucket, live = 8, 5
    case = gi.mtp_case(seed=23, n=bucket, t_step=t_step, dims=gi.Dims(2, 4, 128, 128, 4))
    slots_np, out_np = case.slots.copy(), case.out_slots.copy()
    slots_np[live:] = -1
    out_np[live:] = -1
    assert (bucket * t_step) % (mtp_step + 1) == 0
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    bf = lambda v: dev(v, torch.bfloat16)
    x, a, b, z = bf(case.x()), bf(case.a()), bf(case.b()), bf(case.z())
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log, dt_bias = dev(p.A_log, torch.float32), dev(p.dt_bias, torch.float32)
    slots, out_slots = i32(slots_np), i32(out_np)
    gen = torch.Generator(device="cuda").manual_seed(5)
    ssm0 = torch.randn((case.n_slots, d.h_v, d.d_v, d.d_k), device="cuda", generator=gen) * 0.02
    conv0 = torch.randn((case.n_slots, d.c_ch, d.conv_w - 1), device="cuda", generator=gen).to(torch.bfloat16)
    ssm, conv = ssm0.clone(), conv0.clone()
    y = torch.empty_like(x)
    o = torch.empty((bucket, t_step, d.h_v, d.d_v), dtype=torch.bfloat16, device="cuda")
    src = torch.full((bucket,), -1, dtype=torch.int32, device="cuda")
    dst = torch.full((bucket,), -1, dtype=torch.int32, device="cuda")

    def set_accept(acc):
        s_np = np.full(bucket, -1, np.int32)
        d_np = np.full(bucket, -1, np.int32)
        for i in range(live):
            if acc[i] > 0:
                s_np[i], d_np[i] = out_np[i, acc[i] - 1], slots_np[i]
        src.copy_(torch.from_numpy(s_np))
        dst.copy_(torch.from_numpy(d_np))

    def step():
        if single_call:
            gdn.decode(dims, x, conv_w, a, b, A_log, dt_bias, slots, conv, ssm, out_slots, 1.0, z, norm_w, 1e-6, o=o)
        else:
            gdn.conv1d_update(dims, x, conv_w, conv, slots, out_slots, y=y)
            gdn.recurrent_decode(dims, y, a, b, A_log, dt_bias, ssm, slots, out_slots, 1.0, z, norm_w, 1e-6, o=o)
        gdn.state_copy(dims, ssm, src, dst, conv)

    def reset():
        ssm.copy_(ssm0)
        conv.copy_(conv0)

    graph = None
    for acc in (case.accept, (case.accept + 2) % (t_step + 1)):
        set_accept(acc)
        reset()
        step()
        torch.cuda.synchronize()
        ref = (o.clone(), ssm.clone(), conv.clone())
        if graph is None:
            reset()
            graph = _capture(step)
        for k in range(2):
            reset()
            o.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(o, ref[0]) and torch.equal(ssm, ref[1]) and torch.equal(conv, ref[2]), f"replay {k}"
            assert torch.all(o[live:] == 0), "pad rows must be zero"
            named = set(int(v) for v in slots_np[:live]) | set(int(v) for v in out_np[:live].reshape(-1))
            for sl in range(case.n_slots):
                if sl not in named:
                    assert torch.equal(ssm[sl], ssm0[sl]) and torch.equal(conv[sl], conv0[sl]), f"slot {sl} touched"
            step()  # eager work between replays
            torch.cuda.synchronize()

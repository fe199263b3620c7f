"""The single-call decode / MTP step (gdn_decode): the conv window update and
the fused recurrent step in one kernel, the conv output held in fp32 inside it.
Checked against the oracle under the same row rule as the two-call path, with
every index effect (in-place slots, per-position slots, pad slots, untouched
slots, the conv windows holding raw inputs) bit-exact."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_conv1d_amd as gdn
from tests.gpu_cases import TOL, Score, act_dtype, decode_req_check, dev, host_raw, i32, log, run_map

pytestmark = pytest.mark.gpu


def _upload(case: gi.DecodeCase):
    d = case.dims
    dt = act_dtype(case.act)
    ssm = torch.empty((case.n_slots, d.h_v, d.d_v, d.d_k), dtype=torch.float32, device="cuda")
    for s in range(case.n_slots):
        ssm[s] = dev(case.slot_ssm(s), torch.float32)
    conv = dev(np.stack([case.slot_conv(s) for s in range(case.n_slots)]), dt)
    p = case.params
    return dict(x=dev(case.x(), dt), a=dev(case.a(), dt), b=dev(case.b(), dt), z=dev(case.z(), dt),
                conv_w=dev(p.conv_w, dt), norm_w=dev(p.norm_w, dt), A_log=dev(p.A_log, torch.float32),
                dt_bias=dev(p.dt_bias, torch.float32), conv=conv, ssm=ssm)


def _run(case, t, out_slots=None):
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    return gdn.decode(dims, t["x"], t["conv_w"], t["a"], t["b"], t["A_log"], t["dt_bias"], i32(case.slots), t["conv"],
                      t["ssm"], None if out_slots is None else i32(out_slots), 1.0, t["z"], t["norm_w"], 1e-6)


def _check_in_place(case, t, out, ssm_before, conv_before):
    """Outputs and in-place states against the oracle; pad and untouched slots bitwise."""
    tol = TOL[case.act]
    so, ss = Score(tol), Score(tol)
    live = [i for i in range(case.n) if case.slots[i] >= 0]
    out_raw = host_raw(out)
    tasks = [(case, i, out_raw[i], t["ssm"][int(case.slots[i])].cpu().numpy(), case.t_step - 1) for i in live]
    conv_after = t["conv"].float().cpu().numpy()
    for i, (o_st, s_st, conv_states) in zip(live, run_map(decode_req_check, tasks)):
        so.add_stats(*o_st, label=f"request {i}")
        for h, st in enumerate(s_st):
            ss.add_stats(*st, label=f"request {i} head {h} state")
        assert np.array_equal(conv_after[int(case.slots[i])], conv_states[-1]), f"conv window of request {i}"
    pads = [i for i in range(case.n) if case.slots[i] < 0]
    for i in pads:
        assert torch.all(out[i] == 0), "pad rows must be zero"
    untouched = sorted(set(range(case.n_slots)) - {int(s) for s in case.slots if s >= 0})
    assert torch.equal(t["ssm"][untouched], ssm_before[untouched])
    assert torch.equal(t["conv"][untouched], conv_before[untouched])
    return so, ss


def test_decode_batched_256_single_call():
    """The 256-request decode workload through gdn_decode."""
    case = gi.decode_case()
    t = _upload(case)
    ssm0, conv0 = t["ssm"].clone(), t["conv"].clone()
    out = _run(case, t)
    torch.cuda.synchronize()
    so, ss = _check_in_place(case, t, out, ssm0, conv0)
    log(f"gdn_decode 256: out [{so}] ssm [{ss}]")
    assert so.ok() and ss.ok()


@pytest.mark.parametrize("act,d,h_k,h_v,conv_w,t_step", [("bf16", 128, 2, 4, 4, 1), ("bf16", 128, 2, 4, 3, 6),
                                                         ("f32", 64, 2, 2, 4, 9), ("f32", 16, 1, 2, 2, 5),
                                                         ("bf16", 32, 3, 3, 4, 2)])
def test_decode_small_in_place(act, d, h_k, h_v, conv_w, t_step):
    """Small shapes, several tokens per request in place (spanning the kernel's
    4-token blocks), 1 or 2 V heads per QK head, pad entries."""
    dims = gi.Dims(h_k, h_v, d, d, conv_w)
    case = gi.decode_case(seed=41, n=6, n_slots=10, dims=dims, act=act)
    case.t_step = t_step
    case.slots[2] = -1
    t = _upload(case)
    ssm0, conv0 = t["ssm"].clone(), t["conv"].clone()
    out = _run(case, t)
    torch.cuda.synchronize()
    so, ss = _check_in_place(case, t, out, ssm0, conv0)
    log(f"gdn_decode {act} d={d} {h_k}/{h_v} W={conv_w} T={t_step}: out [{so}] ssm [{ss}]")
    assert so.ok() and ss.ok()


@pytest.mark.parametrize("n,t_step,dims", [(128, 4, gi.QWEN3_NEXT), (5, 7, gi.Dims(2, 4, 64, 64, 4))])
def test_mtp_single_call_and_commit(n, t_step, dims):
    """MTP draft step through gdn_decode: per-position states and conv windows
    to their own slots (home slots read-only), then the accepted positions
    committed with gdn_state_copy; committed slots hold exactly the bytes of
    the GPU's own position states, and match the oracle's replay."""
    case = gi.mtp_case(n=n, t_step=t_step, dims=dims)
    t = _upload(case)
    ssm0, conv0 = t["ssm"].clone(), t["conv"].clone()
    out = _run(case, t, case.out_slots)
    torch.cuda.synchronize()
    home = case.slots.tolist()
    assert torch.equal(t["ssm"][home], ssm0[home]) and torch.equal(t["conv"][home], conv0[home])
    pos_ssm, pos_conv = t["ssm"].clone(), t["conv"].clone()
    acc = case.accept
    sel = acc > 0
    src = case.out_slots[np.arange(case.n), np.maximum(acc - 1, 0)][sel]
    dst = case.slots[sel]
    gdn.state_copy(gdn.Dims(dims.h_k, dims.h_v, dims.d_k, dims.d_v, dims.conv_w), t["ssm"], i32(src), i32(dst), t["conv"])
    torch.cuda.synchronize()
    assert torch.equal(t["ssm"][dst.tolist()], pos_ssm[src.tolist()])
    assert torch.equal(t["conv"][dst.tolist()], pos_conv[src.tolist()])
    rejected = case.slots[~sel].tolist()
    assert torch.equal(t["ssm"][rejected], ssm0[rejected]) and torch.equal(t["conv"][rejected], conv0[rejected])
    so, ss = Score(TOL["bf16"]), Score(TOL["bf16"])
    out_raw = host_raw(out)
    tasks = [(case, i, out_raw[i], t["ssm"][int(case.slots[i])].cpu().numpy() if acc[i] > 0 else None,
              int(acc[i]) - 1) for i in range(case.n)]
    pos_conv_h = pos_conv.float().cpu().numpy()
    for i, (o_st, s_st, conv_states) in enumerate(run_map(decode_req_check, tasks)):
        so.add_stats(*o_st, label=f"request {i}")
        for h, st in enumerate(s_st or []):
            ss.add_stats(*st, label=f"request {i} head {h} committed state")
        for p in range(case.t_step):  # every position's conv window, bitwise
            assert np.array_equal(pos_conv_h[case.out_slots[i][p]], conv_states[p]), f"request {i} position {p}"
    log(f"gdn_decode mtp {n}x{t_step}: out [{so}] committed ssm [{ss}]; accepted {int(sel.sum())}/{case.n}")
    assert so.ok() and ss.ok()


def test_conv_windows_match_the_two_call_path():
    """The conv windows gdn_decode stores are the raw inputs, so they equal the
    windows of gdn_conv1d_update bit for bit, in place and per position."""
    case = gi.mtp_case(seed=43, n=6, t_step=3, dims=gi.Dims(2, 4, 128, 128, 4))
    t = _upload(case)
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    conv0 = t["conv"].clone()
    _run(case, t, case.out_slots)
    ref = conv0.clone()
    gdn.conv1d_update(dims, t["x"], t["conv_w"], ref, i32(case.slots), i32(case.out_slots))
    torch.cuda.synchronize()
    assert torch.equal(t["conv"], ref)

"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Sizes: small multi-chunk cases with ragged tails and the full-size workloads
(single 4096-token prefill, decode, MTP and the ~271k-token varlen batch) are
all checked element by element: every output row, every final state, every
conv window.  The varlen batch's oracle runs on a process pool over the
host's cores.
"""
from __future__ import annotations


import numpy as np
import pytest
import torch

import gdn_inputs as gi
import gated_deltanet_conv1d_amd as gdn
from oracle import gdn_oracle as O
from tests.gpu_cases import (TOL, DevPrefill, Score, act_dtype, bf16_ulps, compare_prefill, decode_req_check, dev, host, host_raw,
                             i32, log, oracle_prefill_seq, oracle_with_perturbed, rel, run_map, u8)
from tests.test_launch_table import table_rows

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- tiny case
def test_tiny_case_recurrent_and_chunked():
    """One sequence, T=64, 1 QK + 1 V head, d=16, fp32, no conv: recurrent and
    chunked (C=16) outputs and final states against the oracle at 1e-4."""
    c = gi.tiny_case()
    dims = gdn.Dims(1, 1, 16, 16, 4)
    qkv = np.concatenate([c.q[:, 0], c.k[:, 0], c.v[:, 0]], axis=1)          # [64, 48]
    g_ref, b_ref = O.gating(c.a, c.b, c.A_log, c.dt_bias)
    o_ref, S_ref, _ = O.gated_delta_rule(O.l2norm(c.q), O.l2norm(c.k), c.v, g_ref, b_ref, None, 1.0)

    # recurrent: one request, 64 tokens, in place
    state = torch.zeros((1, 1, 16, 16), dtype=torch.float32, device="cuda")
    o_rec = gdn.recurrent_decode(dims, dev(qkv[None], torch.float32), dev(c.a[None], torch.float32),
                                 dev(c.b[None], torch.float32), dev(c.A_log, torch.float32),
                                 dev(c.dt_bias, torch.float32), state, i32([0]))
    torch.cuda.synchronize()
    e_rec = rel(host(o_rec[0, :, 0]), o_ref[:, 0])
    e_rec_s = rel(host(state[0, 0]), S_ref[0])

    # chunked, C = 16
    state2 = torch.zeros_like(state)
    g, beta = gdn.gating(dev(c.a, torch.float32), dev(c.b, torch.float32), dev(c.A_log, torch.float32),
                         dev(c.dt_bias, torch.float32))
    assert rel(host(g), g_ref) < 1e-6 and rel(host(beta), b_ref) < 1e-6
    o_chk = gdn.chunk_prefill(dims, dev(qkv, torch.float32), g, beta, i32([0, 64]), i32([0]), state2,
                              u8([0]), chunk=16)
    torch.cuda.synchronize()
    e_chk = rel(host(o_chk[:, 0]), o_ref[:, 0])
    e_chk_s = rel(host(state2[0, 0]), S_ref[0])
    log(f"tiny: recurrent o {e_rec:.2e} S {e_rec_s:.2e}; chunked o {e_chk:.2e} S {e_chk_s:.2e}")
    assert max(e_rec, e_rec_s, e_chk, e_chk_s) < TOL["f32"]


# --------------------------------------------------- small varlen prefills
SMALL_LENGTHS = [1, 3, 17, 64, 65, 200, 0, 130]


@pytest.mark.parametrize("act,d,chunk", [("bf16", 128, 64), ("f32", 128, 64), ("f32", 128, 32), ("bf16", 64, 32),
                                         ("f32", 16, 16), ("bf16", 32, 16), ("f32", 64, 64)])
def test_prefill_small_varlen(act, d, chunk):
    """Several sequences (ragged tails, len 0 and 1, mixed has_init, permuted
    slots, one padding entry) through conv -> gating -> chunked rule ->
    gated RMSNorm; outputs, recurrent states and conv states per slot."""
    dims = gi.Dims(2, 4, d, d, 4)
    case = gi.varlen_case(seed=11, dims=dims, act=act, lengths=np.array(SMALL_LENGTHS), n_slots=12, chunk=chunk)
    case.has_init = np.array([1, 0, 1, 1, 0, 1, 0, 1], np.uint8)
    case.slots[5] = -1                                           # padding entry
    dp = DevPrefill(case)
    conv_before = dp.conv_pool.clone()
    ssm_before = dp.ssm_pool.clone()
    out, *_ = dp.run()
    torch.cuda.synchronize()
    real = [i for i in range(case.n_seq) if case.slots[i] >= 0]
    w = compare_prefill(dp, out, seqs=real)
    lo, hi = case.cu_seqlens[5], case.cu_seqlens[6]
    assert torch.all(out[lo:hi] == 0), "padding rows must be zero"
    untouched = sorted(set(range(case.n_slots)) - {int(s) for s in case.slots if s >= 0})
    assert torch.equal(dp.conv_pool[untouched], conv_before[untouched])
    assert torch.equal(dp.ssm_pool[untouched], ssm_before[untouched])
    log(f"{act} d={d} C={chunk}: out [{w['out']}] ssm [{w['ssm']}] conv {w['conv']:.1e}")
    assert w["conv"] == 0.0
    assert w["out"].ok() and w["ssm"].ok()


def test_prefill_raw_output_scale():
    """No epilogue, scale = d^-1/2: raw o against the oracle (bf16)."""
    dims = gi.Dims(2, 4, 128, 128, 4)
    case = gi.varlen_case(seed=12, dims=dims, lengths=np.array([100, 70]), n_slots=3)
    dp = DevPrefill(case, with_z=False)
    out, *_ = dp.run(scale=128 ** -0.5, epilogue=False)
    torch.cuda.synchronize()
    w = compare_prefill(dp, out, scale=128 ** -0.5, epilogue=False)
    log(f"raw output: out [{w['out']}] ssm [{w['ssm']}]")
    assert w["out"].ok() and w["ssm"].ok()


# -------------------------------------------------------- full workloads
def test_prefill_single_4096():
    """Batch 1, T=4096, 16 QK / 32 V heads, d=128, bf16, C=64, zero initial
    state: every output and the final state against the oracle."""
    case = gi.prefill_case()
    dp = DevPrefill(case)
    out, *_ = dp.run()
    torch.cuda.synchronize()
    w = compare_prefill(dp, out)
    log(f"prefill 4096: out [{w['out']}] ssm [{w['ssm']}]")
    assert w["out"].ok() and w["ssm"].ok() and w["conv"] == 0.0


def _decode_dev(case: gi.DecodeCase):
    d = case.dims
    dt = act_dtype(case.act)
    conv0 = np.stack([case.slot_conv(s) for s in range(case.n_slots)])
    ssm_pool = torch.empty((case.n_slots, d.h_v, d.d_v, d.d_k), dtype=torch.float32, device="cuda")
    for s in range(case.n_slots):
        ssm_pool[s] = dev(case.slot_ssm(s), torch.float32)
    return dict(x=dev(case.x(), dt), a=dev(case.a(), dt), b=dev(case.b(), dt), z=dev(case.z(), dt),
                conv_w=dev(case.params.conv_w, dt), norm_w=dev(case.params.norm_w, dt),
                A_log=dev(case.params.A_log, torch.float32), dt_bias=dev(case.params.dt_bias, torch.float32),
                conv_pool=dev(conv0, dt), ssm_pool=ssm_pool, conv0=conv0)


def _oracle_decode_seq(case: gi.DecodeCase, x, a, b, z, i, keep_states=False, **pert):
    d = case.dims
    s = int(case.slots[i])
    p = case.params
    return O.layer_sequence(x[i], a[i], b[i], z[i], p.conv_w, None, p.A_log, p.dt_bias, p.norm_w,
                            case.slot_conv(s), case.slot_ssm(s), (d.h_k, d.h_v, d.d_k, d.d_v), 1.0, 1e-6,
                            keep_states=keep_states, **pert)


def test_decode_batched_256():
    """256 requests x 1 token, 512-slot pools, permuted slot table, in place:
    outputs and updated states against the oracle; untouched slots bitwise."""
    case = gi.decode_case()
    t = _decode_dev(case)
    dims = gdn.Dims(*case.dims.__dict__.values())
    ssm_before, conv_before = t["ssm_pool"].clone(), t["conv_pool"].clone()
    out, _ = gdn.decode_layer(dims, t["x"], t["conv_w"], t["A_log"], t["dt_bias"], t["a"], t["b"], i32(case.slots),
                              t["conv_pool"], t["ssm_pool"], z=t["z"], norm_w=t["norm_w"])
    torch.cuda.synchronize()
    so, ss = Score(TOL["bf16"]), Score(TOL["bf16"])
    worst_c = 0.0
    conv_pool = t["conv_pool"].float().cpu().numpy()
    out_raw = host_raw(out)
    tasks = [(case, i, out_raw[i], t["ssm_pool"][int(case.slots[i])].cpu().numpy(), 0) for i in range(case.n)]
    for i, (o_st, s_st, conv_states) in enumerate(run_map(decode_req_check, tasks)):
        so.add_stats(*o_st, label=f"request {i}")
        for h, st in enumerate(s_st):
            ss.add_stats(*st, label=f"request {i} head {h} state")
        worst_c = max(worst_c, float(np.max(np.abs(conv_pool[int(case.slots[i])] - conv_states[0]))))
    untouched = sorted(set(range(case.n_slots)) - set(case.slots.tolist()))
    assert torch.equal(t["ssm_pool"][untouched], ssm_before[untouched])
    assert torch.equal(t["conv_pool"][untouched], conv_before[untouched])
    log(f"decode 256: out [{so}] ssm [{ss}] conv {worst_c:.1e}")
    assert so.ok() and ss.ok() and worst_c == 0.0


def test_mtp_draft_and_commit():
    """128 requests x 4 draft tokens: per-position states to their own slots,
    then the accepted position's state committed with gdn_state_copy.
    Indexing is bit-exact: a committed slot holds exactly the bytes of the
    GPU's own position state, accept 0 leaves the home slot untouched, and
    untouched slots are unchanged; values match the oracle's replay."""
    case = gi.mtp_case()
    t = _decode_dev(case)
    dims = gdn.Dims(*case.dims.__dict__.values())
    ssm_before, conv_before = t["ssm_pool"].clone(), t["conv_pool"].clone()
    out, _ = gdn.decode_layer(dims, t["x"], t["conv_w"], t["A_log"], t["dt_bias"], t["a"], t["b"], i32(case.slots),
                              t["conv_pool"], t["ssm_pool"], out_slots=i32(case.out_slots), z=t["z"],
                              norm_w=t["norm_w"])
    torch.cuda.synchronize()
    # home slots are read-only during the draft step
    assert torch.equal(t["ssm_pool"][case.slots.tolist()], ssm_before[case.slots.tolist()])
    assert torch.equal(t["conv_pool"][case.slots.tolist()], conv_before[case.slots.tolist()])
    pos_ssm = t["ssm_pool"].clone()
    pos_conv = t["conv_pool"].clone()
    acc = case.accept
    sel = acc > 0
    src = case.out_slots[np.arange(case.n), np.maximum(acc - 1, 0)][sel]
    dst = case.slots[sel]
    gdn.state_copy(dims, t["ssm_pool"], i32(src), i32(dst), t["conv_pool"])
    torch.cuda.synchronize()
    assert torch.equal(t["ssm_pool"][dst.tolist()], pos_ssm[src.tolist()])
    assert torch.equal(t["conv_pool"][dst.tolist()], pos_conv[src.tolist()])
    rejected = case.slots[~sel].tolist()
    assert torch.equal(t["ssm_pool"][rejected], ssm_before[rejected])
    # values against the oracle's replay
    so, ss = Score(TOL["bf16"]), Score(TOL["bf16"])
    out_raw = host_raw(out)
    ssm_after = t["ssm_pool"]
    tasks = [(case, i, out_raw[i], ssm_after[int(case.slots[i])].cpu().numpy() if acc[i] > 0 else None,
              int(acc[i]) - 1) for i in range(case.n)]
    conv_after = t["conv_pool"].float().cpu().numpy()
    for i, (o_st, s_st, conv_states) in enumerate(run_map(decode_req_check, tasks)):
        so.add_stats(*o_st, label=f"request {i}")
        for h, st in enumerate(s_st or []):
            ss.add_stats(*st, label=f"request {i} head {h} committed state")
        if acc[i] > 0:
            assert np.array_equal(conv_after[case.slots[i]], conv_states[acc[i] - 1])
    log(f"mtp: out [{so}] committed ssm [{ss}]; accepted {int(sel.sum())}/{case.n}")
    assert so.ok() and ss.ok()


def test_varlen_full():
    """64 sequences, 271,311 tokens, nonzero initial states, permuted slots:
    the whole batch runs on the GPU and every sequence is checked against the
    oracle: all 32 V heads of every output row, every final recurrent state,
    and every conv state bitwise.  The last sequences start past token 262,144,
    where element offsets into the packed rows exceed 2^31."""
    case = gi.varlen_case()
    log(f"varlen: {case.n_seq} seqs, {case.t_total} tokens")
    dp = DevPrefill(case)
    out, *_ = dp.run()
    torch.cuda.synchronize()
    assert int(case.cu_seqlens[-2]) * case.dims.c_ch > 2 ** 31
    w = compare_prefill(dp, out)
    log(f"varlen full: out [{w['out']}] ssm [{w['ssm']}] conv {w['conv']:.1e}")
    assert w["out"].ok() and w["ssm"].ok() and w["conv"] == 0.0


# ------------------------------------------------------------ consistency
def test_chunked_matches_recurrent_on_gpu():
    """The same tokens through the chunked kernel and the recurrent kernel:
    both meet the bound against the oracle, and their states agree."""
    dims = gi.Dims(2, 4, 128, 128, 4)
    case = gi.varlen_case(seed=13, dims=dims, lengths=np.array([150]), n_slots=2)
    dp = DevPrefill(case)
    ssm0 = dp.ssm_pool.clone()
    out_c, y, g, beta = dp.run()
    torch.cuda.synchronize()
    s = int(case.slots[0])
    st = ssm0.clone()
    out_r = gdn.recurrent_decode(dp.dims, y[None], dp.a[None], dp.b[None], dp.A_log, dp.dt_bias, st, i32([s]),
                                 z=dp.z[None], norm_w=dp.norm_w)
    torch.cuda.synchronize()
    r, rts = oracle_with_perturbed(lambda **pe: oracle_prefill_seq(case, 0, **pe), "bf16")
    sc, sr, st_c, st_r = (Score(TOL["bf16"]) for _ in range(4))
    sc.add(host(out_c), r["out"], [rt["out"] for rt in rts])
    sr.add(host(out_r[0]), r["out"], [rt["out"] for rt in rts])
    for h in range(4):
        st_c.add_slice(host(dp.ssm_pool[s, h]), r["ssm"][h], [rt["ssm"][h] for rt in rts])
        st_r.add_slice(host(st[s, h]), r["ssm"][h], [rt["ssm"][h] for rt in rts])
    e_s = max(rel(host(dp.ssm_pool[s, h]), host(st[s, h])) for h in range(4))
    log(f"chunked [{sc}] recurrent [{sr}] states chunked [{st_c}] recurrent [{st_r}] chunked-vs-recurrent {e_s:.2e}")
    assert sc.ok() and sr.ok() and st_c.ok() and st_r.ok() and e_s < TOL["bf16"]


def test_split_prefill_carries_state():
    """Prefill of T tokens as T1 then T2 tokens with the states carried through
    the slot pools (chunk boundaries differ from a single pass) meets the
    bound against the oracle, and the conv state matches a single pass bitwise."""
    dims = gi.Dims(2, 4, 128, 128, 4)
    case = gi.varlen_case(seed=14, dims=dims, lengths=np.array([300]), n_slots=2)
    dp = DevPrefill(case)
    conv0, ssm0 = dp.conv_pool.clone(), dp.ssm_pool.clone()
    dp.run()
    torch.cuda.synchronize()
    full_conv = dp.conv_pool.clone()
    dp.conv_pool.copy_(conv0)
    dp.ssm_pool.copy_(ssm0)
    outs = []
    for lo, hi in ((0, 100), (100, 300)):
        o, *_ = gdn.prefill_layer(dp.dims, dp.x[lo:hi].contiguous(), dp.conv_w, dp.A_log, dp.dt_bias,
                                  dp.a[lo:hi].contiguous(), dp.b[lo:hi].contiguous(), i32([0, hi - lo]), dp.slots,
                                  dp.conv_pool, dp.ssm_pool, dp.has_init, 64, 1.0, dp.z[lo:hi].contiguous(),
                                  dp.norm_w)
        outs.append(o)
    torch.cuda.synchronize()
    split = torch.cat(outs)
    assert torch.equal(dp.conv_pool, full_conv)
    w = compare_prefill(dp, split)
    log(f"split prefill: out [{w['out']}] ssm [{w['ssm']}]")
    assert w["out"].ok() and w["ssm"].ok() and w["conv"] == 0.0


def test_deterministic():
    """Two runs on fresh copies give bitwise-identical outputs and states."""
    dims = gi.Dims(2, 4, 128, 128, 4)
    case = gi.varlen_case(seed=15, dims=dims, lengths=np.array([77, 190, 64]), n_slots=6)
    dp = DevPrefill(case)
    conv0, ssm0 = dp.conv_pool.clone(), dp.ssm_pool.clone()
    o1, *_ = dp.run()
    s1, c1 = dp.ssm_pool.clone(), dp.conv_pool.clone()
    dp.conv_pool.copy_(conv0)
    dp.ssm_pool.copy_(ssm0)
    o2, *_ = dp.run()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, dp.ssm_pool) and torch.equal(c1, dp.conv_pool)


def test_batch_composition_does_not_change_a_sequence():
    """One sequence's final state and conv state are bitwise the same whether
    it runs alone or packed with 3 or 8 more sequences (32, 128 and 288
    (sequence, V head) chains: the launch table's split shapes and the chain
    that computes the output itself), on both entry points; its outputs are
    bitwise the same on the split shapes and within one bf16 unit in the last
    place on the chain with output (another order of its products and norm
    sum).  The packed runs also meet the oracle on the first sequence."""
    lengths = np.array([300, 129, 64, 1, 700, 65, 0, 200, 333])
    case = gi.varlen_case(seed=16, lengths=lengths, n_slots=12)
    dp = DevPrefill(case)
    conv0, ssm0 = dp.conv_pool.clone(), dp.ssm_pool.clone()
    s0 = int(case.slots[0])
    T0 = int(lengths[0])
    res = {}
    for n in (1, 4, 9):
        T = int(case.cu_seqlens[n])
        for fused in (False, True):
            dp.conv_pool.copy_(conv0)
            dp.ssm_pool.copy_(ssm0)
            if fused:
                o = gdn.prefill(dp.dims, dp.x[:T], dp.conv_w, dp.a[:T], dp.b[:T], dp.A_log, dp.dt_bias, dp.cu[:n + 1],
                                dp.slots[:n], dp.conv_pool, dp.ssm_pool, dp.has_init[:n], 64, 1.0, dp.z[:T],
                                dp.norm_w)
            else:
                o, *_ = gdn.prefill_layer(dp.dims, dp.x[:T], dp.conv_w, dp.A_log, dp.dt_bias, dp.a[:T], dp.b[:T],
                                          dp.cu[:n + 1], dp.slots[:n], dp.conv_pool, dp.ssm_pool, dp.has_init[:n],
                                          64, 1.0, dp.z[:T], dp.norm_w)
            torch.cuda.synchronize()
            res[(n, fused)] = (o[:T0].clone(), dp.ssm_pool[s0].clone(), dp.conv_pool[s0].clone())
            if n == 9 and not fused:
                w = compare_prefill(dp, o, seqs=[0], heads=[0, 5, 31])
                log(f"packed 9: out [{w['out']}] ssm [{w['ssm']}] conv {w['conv']:.1e}")
                assert w["out"].ok() and w["ssm"].ok() and w["conv"] == 0.0
    rows, _ = table_rows()

    def whole_dv(n):  # the table's shape for n sequences x 32 V heads
        for mc, _ml, ntw, _pd in rows:
            if mc is None or n * 32 <= mc:
                return ntw >= 8

    for key, got in res.items():
        ref = res[(1, False)]
        o_r, o_g = ref[0], got[0]
        if whole_dv(key[0]):
            assert bf16_ulps(host_raw(o_r), host_raw(o_g)) <= 1, \
                f"sequence 0 output beyond one unit in the last place with {key[0]} sequences (fused={key[1]})"
        else:
            assert torch.equal(o_r, o_g), f"sequence 0 output differs with {key[0]} sequences (fused={key[1]})"
        for r, g in zip(ref[1:], got[1:]):
            assert torch.equal(r, g), f"sequence 0 state differs with {key[0]} sequences (fused={key[1]})"


def test_many_short_sequences():
    """300 sequences of 0..40 tokens (more than the kernels prefix-sum
    themselves, so the chunk index table is built first): every output and
    state against the oracle, on both entry points."""
    rng = np.random.default_rng(17)
    lengths = rng.integers(0, 41, size=300)
    case = gi.varlen_case(seed=17, dims=gi.Dims(1, 2, 32, 32, 4), lengths=lengths, n_slots=320, chunk=16)
    dp = DevPrefill(case)
    conv0, ssm0 = dp.conv_pool.clone(), dp.ssm_pool.clone()
    out, *_ = dp.run()
    torch.cuda.synchronize()
    w = compare_prefill(dp, out)
    log(f"300 short sequences: out [{w['out']}] ssm [{w['ssm']}] conv {w['conv']:.1e}")
    assert w["out"].ok() and w["ssm"].ok() and w["conv"] == 0.0
    ref = (out.clone(), dp.ssm_pool.clone(), dp.conv_pool.clone())
    dp.conv_pool.copy_(conv0)
    dp.ssm_pool.copy_(ssm0)
    out_f = dp.run_fused()
    torch.cuda.synchronize()
    assert torch.equal(out_f, ref[0]) and torch.equal(dp.ssm_pool, ref[1]) and torch.equal(dp.conv_pool, ref[2])


def test_many_chains_fp32():
    """The fp32 mode above 128 chains: the launch table picks the whole-d_v
    chain, which the fp32 operands do not fit, so the widest split chain runs
    (with the chunk index, more than 8 sequences).  40 sequences of 0..150
    tokens at d = 128, chunk 32, 4 V heads (160 chains): every output, state
    and conv window against the oracle, and both entry points equal."""
    rng = np.random.default_rng(19)
    lengths = rng.integers(0, 151, size=40)
    case = gi.varlen_case(seed=19, dims=gi.Dims(2, 4, 128, 128, 4), act="f32", lengths=lengths, n_slots=48,
                          chunk=32)
    assert case.n_seq * case.dims.h_v > 128
    dp = DevPrefill(case)
    conv0, ssm0 = dp.conv_pool.clone(), dp.ssm_pool.clone()
    out, *_ = dp.run()
    torch.cuda.synchronize()
    w = compare_prefill(dp, out)
    log(f"fp32, 160 chains: out [{w['out']}] ssm [{w['ssm']}] conv {w['conv']:.1e}")
    assert w["out"].ok() and w["ssm"].ok() and w["conv"] == 0.0
    ref = (out.clone(), dp.ssm_pool.clone(), dp.conv_pool.clone())
    dp.conv_pool.copy_(conv0)
    dp.ssm_pool.copy_(ssm0)
    out_f = dp.run_fused()
    torch.cuda.synchronize()
    assert torch.equal(out_f, ref[0]) and torch.equal(dp.ssm_pool, ref[1]) and torch.equal(dp.conv_pool, ref[2])


def test_state_copy_bitwise_and_skips():
    dims = gdn.Dims(2, 4, 64, 64, 4)
    g = torch.Generator(device="cuda").manual_seed(0)
    state = torch.randn((6, 4, 64, 64), device="cuda", generator=g)
    conv = torch.randn((6, dims.c_ch, 3), device="cuda", generator=g).to(torch.bfloat16)
    s0, c0 = state.clone(), conv.clone()
    gdn.state_copy(dims, state, i32([0, 2, -1, 4, 3]), i32([1, 5, 3, -1, 3]), conv)
    torch.cuda.synchronize()
    assert torch.equal(state[1], s0[0]) and torch.equal(state[5], s0[2])
    assert torch.equal(conv[1], c0[0]) and torch.equal(conv[5], c0[2])
    for k in (0, 2, 3, 4):
        assert torch.equal(state[k], s0[k]) and torch.equal(conv[k], c0[k])

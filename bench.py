"""Benchmark of the GDN hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

One step = one pass of the prefill hot path over one batch: causal conv1d +
SiLU, gating, the chunked gated delta rule with fused q/k L2 norm and the
gated-RMSNorm epilogue, as the single gdn_prefill call (conv output and gates
stay inside the chunk kernels), on the single-sequence workload: batch 1,
T=4096, 16 QK / 32 V heads, d=128, bf16 activations, fp32 state, chunk 64,
synthetic seeded inputs resident in HBM.  Steps alternate between two copies
of every input, output, pool and workspace (about 0.6 GB together, more than
the 256 MiB memory-side cache).  The timed steps replay one captured HIP
graph per copy (how a serving loop runs it; --eager times plain launches);
per-call times (median, p10, p90 and mean) come from an eager pass with HIP
events on the launch stream.  The same step as three calls (gdn_conv1d_fwd,
gdn_gating, gdn_chunk_prefill) is reported beside it.

Prints ONE JSON line: tokens/s for that step (value), the roofline of the
dominant call (gdn_prefill), then the other workloads as extra rows: the
decode step (256 requests x 1 token over 512-slot pools, gdn_decode and the two
separate calls, pools rotated so states come from HBM) and its padded-bucket
graph, the 128 x 4-token MTP step (gdn_decode, the two separate calls, the
commit copy) and its bucket graph, the ~271k-token varlen prefill on the
seeded inputs of the parity tests, the prefill at one tensor-parallel rank's
head counts (tp = 2, 4), the whole layer around the core (Gemma RMSNorm and
the projections at hidden 2048) for the 4096-token prefill and the 256-request
decode, and the fp64 CPU oracle timed on the host's cores on a sample of every
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "GDN prefill tokens/s (MFMA util) + decode state-update GB/s vs HBM peak"


def chunk_algorithmic(T: int, n_seq: int, h_k: int, h_v: int, d: int, act_bytes: int, has_init: bool,
                      chunk: int) -> tuple[float, float]:
    """Algorithmic bytes and flops of one gdn_chunk_prefill launch.

    Bytes per token: q, k, v rows read once (2*h_k*d + h_v*d activations),
    g and beta (2*h_v fp32), z read and out written (2*h_v*d activations);
    per sequence: the fp32 state written (and read when it has history).
    Flops per chunk and V head (C = chunk, d_k = d_v = d): Gram K K^T and Q K^T
    (2dC^2 shared by h_v/h_k V heads, triangular), W, Ut and (M o QK^T) U
    (3dC(C+1)), the UT inverse (C^3/3), and W S^T, Q S^T, K^T U (6Cd^2).
    """
    per_tok = (2 * h_k * d + h_v * d) * act_bytes + 2 * h_v * 4 + 2 * h_v * d * act_bytes
    state = n_seq * h_v * d * d * 4 * (2 if has_init else 1)
    nbytes = T * per_tok + state
    C = chunk
    per_chunk_head = 2 * d * C * C * h_k / h_v + 3 * d * C * (C + 1) + C ** 3 / 3 + 6 * C * d * d
    flops = (T / C) * h_v * per_chunk_head
    return float(nbytes), float(flops)


def prefill_algorithmic(T: int, n_seq: int, h_k: int, h_v: int, d: int, act_bytes: int, has_init: bool,
                        chunk: int, conv_w: int) -> tuple[float, float]:
    """Algorithmic bytes and flops of one gdn_prefill call: per token the conv
    input row (2*h_k*d + h_v*d activations), a and b (2*h_v activations), z
    read and out written; per sequence the fp32 state and the conv window
    (written, and read when it has history).  Flops as chunk_algorithmic plus
    the conv (2*conv_w per channel and token)."""
    c_ch = 2 * h_k * d + h_v * d
    per_tok = c_ch * act_bytes + 2 * h_v * act_bytes + 2 * h_v * d * act_bytes
    per_seq = (h_v * d * d * 4 + c_ch * (conv_w - 1) * act_bytes) * (2 if has_init else 1)
    _, flops = chunk_algorithmic(T, n_seq, h_k, h_v, d, act_bytes, has_init, chunk)
    return float(T * per_tok + n_seq * per_seq), float(flops + 2 * conv_w * c_ch * T)


def decode_algorithmic(n: int, t_step: int, h_k: int, h_v: int, d: int, act_bytes: int, n_pos_writes: int) -> float:
    """Bytes of one gdn_recurrent_decode launch: each state read once and written
    n_pos_writes times, plus per token q/k/v, a/b, z and out."""
    state = h_v * d * d * 4
    per_tok = (2 * h_k * d + h_v * d) * act_bytes + 2 * h_v * act_bytes + 2 * h_v * d * act_bytes
    return float(n * (state * (1 + n_pos_writes) + t_step * per_tok))


def decode_fused_algorithmic(n: int, t_step: int, h_k: int, h_v: int, d: int, act_bytes: int, conv_w: int,
                             n_pos_writes: int) -> float:
    """Bytes of one gdn_decode launch: per request the state and the conv window
    read once and written n_pos_writes times; per token the conv input row, a
    and b, z read and out written."""
    c_ch = 2 * h_k * d + h_v * d
    state = h_v * d * d * 4 + c_ch * (conv_w - 1) * act_bytes
    per_tok = c_ch * act_bytes + 2 * h_v * act_bytes + 2 * h_v * d * act_bytes
    return float(n * (state * (1 + n_pos_writes) + t_step * per_tok))


def pct(ms) -> dict:
    """Median, p10, p90 and mean of a list of times (ms)."""
    a = np.asarray(ms, np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4)}


def kernel_src_sha() -> str:
    """Hash of the HIP sources; counter figures apply only to the sources they were taken on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gated_deltanet_conv1d_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str, kernels) -> float | None:
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    (profiles/<workload>_traffic.json), summed over `kernels`; None when the kernel
    sources changed since the counters were taken or a kernel is missing."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("src_sha") != kernel_src_sha():
        return None
    per = rec["per_dispatch"]
    try:
        return float(sum(per[k]["read_bytes"] + per[k]["write_bytes"] for k in kernels))
    except KeyError:
        return None


def chain_shape(chains: int, mean_len: int) -> tuple[int, int]:
    """(d_v tiles per workgroup, prefetch stages) of the chain pass for a call
    with this many (sequence, V head) chains: the first matching row of the
    launch table in csrc/launch_table.hpp."""
    import re
    src = open(os.path.join(ROOT, "gated_deltanet_conv1d_amd", "csrc", "launch_table.hpp")).read()
    body = src[src.index("kChainTable[] = {"):]
    rows = re.findall(r"\{(\w+), (\w+), (\d+), (\d+)\}", body[:body.index("};")])
    for mc, ml, ntw, pd in rows:
        if (mc == "INT64_MAX" or chains <= int(mc)) and (ml == "INT64_MAX" or mean_len <= int(ml)):
            return int(ntw), int(pd)
    return int(rows[-1][2]), int(rows[-1][3])


_NTW, _PD = chain_shape(32, 4096)   # the single 4096-token sequence: 32 chains
# kernels one gdn_chunk_prefill call launches on the split path (one sequence:
# no chunk index kernel)
CHUNK_SPLIT_KERNELS = ("void split::chunk_prep_kernel<__bf16, __bf16, 128, 64, false, 4, 2>",
                       f"void split::chunk_state_kernel<__bf16, 128, 64, {_NTW}, {_PD}>",
                       "void split::chunk_out_kernel<__bf16, __bf16, 128, 64, false, 4>")
# kernels one gdn_prefill call launches (the chain kernel also stores the conv windows)
PREFILL_KERNELS = ("void split::chunk_prep_kernel<__bf16, __bf16, 128, 64, true, 4, 2>",
                   f"void split::chunk_state_kernel<__bf16, 128, 64, {_NTW}, {_PD}>",
                   "void split::chunk_out_kernel<__bf16, __bf16, 128, 64, true, 4>")
# the single-call decode (in place, one token) and MTP draft step kernels
DECODE_KERNEL = "void decode_fused_kernel<__bf16, 128, 2, 4, false, true, true>"
MTP_KERNEL = "void decode_fused_kernel<__bf16, 128, 2, 4, true, true, false>"
# the layer's projection kernels at 4096 tokens (in_proj_qkvz/ba, out_proj with the residual)
# in_proj at 4096 rows: 48 column tiles of 256 x 256 straight into LDS, then
# the 64-wide last tile (b and a) as small register-staged tiles
IN_PROJ_KERNELS = ("void proj_lds_kernel<256, 256, 2, 4, false, 2>", "void proj_kernel<64, 32, 2, 2, 2, true, false>")
OUT_PROJ_KERNELS = ("void proj_lds_kernel<128, 256, 2, 4, true, 3>",)


def counter_mfma(workload: str, kernels) -> dict | None:
    """MFMA utilisation from the committed rocprofv3 counter pass
    (profiles/<workload>_mfma.json): the kernels' MFMA-busy cycles (summed
    over every SIMD) over their GPU-busy cycles (per XCD) x 1024 SIMDs, summed
    over the kernels; None when the sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{workload}_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("src_sha") != kernel_src_sha():
        return None
    per = rec["per_dispatch"]
    try:
        busy = sum(per[k]["mfma_busy_cycles"] for k in kernels)
        total = sum(per[k]["gpu_busy_cycles_per_xcd"] * per[k]["simds"] for k in kernels)
        flops = sum(per[k]["mfma_flops"] for k in kernels)
    except KeyError:
        return None
    return {"mfma_util": round(busy / total, 4) if total else None, "mfma_flops_issued": flops,
            "counters": rec.get("counters"), "formula": rec.get("util_formula")}


def capture_graph(torch, fn):
    """One HIP graph of fn's launches (a warm-up run off the capture first)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def device_info() -> dict:
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "cus": p.multi_processor_count, "arch": getattr(p, "gcnArchName", "")}


def fill_bandwidth_gbs(torch) -> float:
    """Measured device write-only bandwidth (a 1 GiB fill: bytes written / time)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        a.fill_(1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        a.fill_(1)
    e1.record()
    torch.cuda.synchronize()
    return n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9


def copy_bandwidth_gbs(torch) -> float:
    """Measured device-to-device copy bandwidth (read + write bytes / time)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9


def bench_prefill(args, torch, gdn, gi):
    case = gi.prefill_case()
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    dev = torch.device("cuda")
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev, torch.bfloat16)
    T = case.t_total
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log = torch.from_numpy(p.A_log).to(dev)
    dt_bias = torch.from_numpy(p.dt_bias).to(dev)
    cu = torch.tensor(case.cu_seqlens, dtype=torch.int32, device=dev)
    slots = torch.zeros(1, dtype=torch.int32, device=dev)
    has_init = torch.zeros(1, dtype=torch.uint8, device=dev)
    # (one workspace serves both entry points: the larger of their sizes)
    ws_bytes = max(gdn.chunk_prefill_workspace_size(dims, 0, 1, T, case.chunk),
                   gdn.prefill_workspace_size(dims, 0, 1, T, case.chunk))
    x0, a0, b0, z0 = case.seq_x(0), case.seq_a(0), case.seq_b(0), case.seq_z(0)
    copies = []
    for _ in range(args.prefill_copies):  # (default 2: the steps alternate, the footprint exceeds the memory-side cache)
        copies.append(dict(
            x=bf(x0), a=bf(a0), b=bf(b0), z=bf(z0),
            conv_pool=torch.zeros((1, d.c_ch, d.conv_w - 1), dtype=torch.bfloat16, device=dev),
            ssm_pool=torch.zeros((1, d.h_v, d.d_v, d.d_k), dtype=torch.float32, device=dev),
            y=torch.empty((T, d.c_ch), dtype=torch.bfloat16, device=dev),
            g=torch.empty((T, d.h_v), dtype=torch.float32, device=dev),
            beta=torch.empty((T, d.h_v), dtype=torch.float32, device=dev),
            o=torch.empty((T, d.h_v, d.d_v), dtype=torch.bfloat16, device=dev),
            ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev)))
    footprint = sum(t.numel() * t.element_size() for c in copies for t in c.values())

    nc = len(copies)

    def step_sep(k, e=None):
        c = copies[k % nc]
        if e: e[0].record()
        gdn.conv1d_fwd(dims, c["x"], conv_w, cu, slots, c["conv_pool"], has_init, y=c["y"])
        if e: e[1].record()
        gdn.gating(c["a"], c["b"], A_log, dt_bias, g=c["g"], beta=c["beta"])
        if e: e[2].record()
        gdn.chunk_prefill(dims, c["y"], c["g"], c["beta"], cu, slots, c["ssm_pool"], has_init, case.chunk, 1.0,
                          c["z"], norm_w, 1e-6, o=c["o"], workspace=c["ws"])
        if e: e[3].record()

    def step(k, e=None):
        c = copies[k % nc]
        if e: e[0].record()
        gdn.prefill(dims, c["x"], conv_w, c["a"], c["b"], A_log, dt_bias, cu, slots, c["conv_pool"], c["ssm_pool"],
                    has_init, case.chunk, 1.0, c["z"], norm_w, 1e-6, o=c["o"], workspace=c["ws"])
        if e: e[1].record()

    def timed(fn, n_ev):
        """eager pass with events, then (unless --eager) graph replays, one graph
        per copy; returns (wall seconds of the timed pass, eager wall, events)"""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
        for k in range(args.warmup):
            fn(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            fn(k, evs[k])
        torch.cuda.synchronize()
        wall_eager = time.perf_counter() - t0
        if args.eager:
            return wall_eager, wall_eager, evs
        graphs = [capture_graph(torch, lambda k=k: fn(k)) for k in range(nc)]
        for k in range(args.warmup):
            graphs[k % nc].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            graphs[k % nc].replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, wall_eager, evs

    wall_sep, wall_sep_eager, ev = timed(step_sep, 4)
    wall, wall_eager, evf = timed(step, 2)
    ms = lambda evs, i, j: [e[i].elapsed_time(e[j]) for e in evs]
    t_pre = pct(ms(evf, 0, 1))
    nbytes, flops = prefill_algorithmic(T, 1, d.h_k, d.h_v, d.d_k, 2, False, case.chunk, d.conv_w)
    achieved = nbytes / (t_pre["mean"] * 1e-3) / 1e9
    mfma_tflops = flops / (t_pre["mean"] * 1e-3) / 1e12
    return dict(
        T=T, wall_s=wall, ms_per_step=wall / args.steps * 1e3, eager_ms_per_step=wall_eager / args.steps * 1e3,
        kernels_ms={"gdn_prefill": t_pre}, footprint_bytes=footprint,
        separate_calls={"ms_per_step": round(wall_sep / args.steps * 1e3, 4),
                        "tokens_per_s": round(T * args.steps / wall_sep, 1),
                        "eager_ms_per_step": round(wall_sep_eager / args.steps * 1e3, 4),
                        "kernels_ms": {"gdn_conv1d_fwd": pct(ms(ev, 0, 1)), "gdn_gating": pct(ms(ev, 1, 2)),
                                       "gdn_chunk_prefill": pct(ms(ev, 2, 3))},
                        "chunk_traffic": counter_traffic("prefill_4096", CHUNK_SPLIT_KERNELS)},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4),
                  "traffic": counter_traffic("prefill_4096", PREFILL_KERNELS),
                  "kernel": "gdn_prefill (chunk_prep + chunk_state + chunk_out)",
                  "algorithmic_bytes": nbytes,
                  "launch_ms": t_pre["mean"],
                  "mfma": {"algorithmic_flops": flops, "achieved_tflops": round(mfma_tflops, 2),
                           "peak_tflops": BF16_PEAK_TFLOPS, "frac": round(mfma_tflops / BF16_PEAK_TFLOPS, 5),
                           "counters": counter_mfma("prefill_4096", PREFILL_KERNELS)}},
        inputs=dict(case=case))


def bench_tp_shapes(args, torch, gdn, gi):
    """The 4096-token single-sequence prefill (gdn_prefill) at one tensor-parallel
    rank's head counts: h_k/h_v = 8/16 (tp = 2) and 4/8 (tp = 4), event-timed eager
    launches.  A head-sharded layer runs these per rank with no exchange inside it."""
    dev = torch.device("cuda")
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev, torch.bfloat16)
    out = {}
    for tp in (2, 4):
        base = gi.QWEN3_NEXT
        d = gi.Dims(base.h_k // tp, base.h_v // tp, base.d_k, base.d_v, base.conv_w)
        case = gi.prefill_case(dims=d)
        dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
        p = case.params
        x, a, b, z = bf(case.seq_x(0)), bf(case.seq_a(0)), bf(case.seq_b(0)), bf(case.seq_z(0))
        conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
        A_log, dt_bias = torch.from_numpy(p.A_log).to(dev), torch.from_numpy(p.dt_bias).to(dev)
        cu = torch.tensor(case.cu_seqlens, dtype=torch.int32, device=dev)
        slots = torch.zeros(1, dtype=torch.int32, device=dev)
        has_init = torch.zeros(1, dtype=torch.uint8, device=dev)
        conv_pool = torch.zeros((1, d.c_ch, d.conv_w - 1), dtype=torch.bfloat16, device=dev)
        ssm_pool = torch.zeros((1, d.h_v, d.d_v, d.d_k), dtype=torch.float32, device=dev)
        T = case.t_total
        o = torch.empty((T, d.h_v, d.d_v), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(gdn.prefill_workspace_size(dims, 0, 1, T, case.chunk), dtype=torch.uint8, device=dev)
        steps = max(min(args.steps, 50), 1)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]

        def step(e=None):
            if e: e[0].record()
            gdn.prefill(dims, x, conv_w, a, b, A_log, dt_bias, cu, slots, conv_pool, ssm_pool, has_init, case.chunk,
                        1.0, z, norm_w, 1e-6, o=o, workspace=ws)
            if e: e[1].record()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        for k in range(steps):
            step(ev[k])
        torch.cuda.synchronize()
        t = pct([e[0].elapsed_time(e[1]) for e in ev])
        out[f"tp{tp}_h{d.h_k}_{d.h_v}"] = {"gdn_prefill_ms": t, "tokens_per_s_per_rank": round(T / (t["mean"] * 1e-3), 1)}
    return out


def bench_decode_bucket(args, torch, gdn, gi):
    """The decode step as a serving loop runs it: gdn_decode captured once per
    state pool as a HIP graph for a fixed bucket of 256 requests, of which 200
    are live and 56 are pad entries (slot -1), replayed over 3 pools so states
    come from HBM."""
    case = gi.decode_case()
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    dev = torch.device("cuda")
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev, torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(case.seed + 1)
    live = 200
    slots_np = case.slots.copy()
    slots_np[live:] = -1
    slots = torch.from_numpy(slots_np).to(dev)
    x, a, b, z = bf(case.x()), bf(case.a()), bf(case.b()), bf(case.z())
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log, dt_bias = torch.from_numpy(p.A_log).to(dev), torch.from_numpy(p.dt_bias).to(dev)
    o = torch.empty((case.n, 1, d.h_v, d.d_v), dtype=torch.bfloat16, device=dev)
    graphs = []
    for _ in range(3):
        ssm = torch.randn((case.n_slots, d.h_v, d.d_v, d.d_k), device=dev, generator=gen) * 0.02
        conv = torch.randn((case.n_slots, d.c_ch, d.conv_w - 1), device=dev, generator=gen).to(torch.bfloat16)

        def step(ssm=ssm, conv=conv):
            gdn.decode(dims, x, conv_w, a, b, A_log, dt_bias, slots, conv, ssm, None, 1.0, z, norm_w, 1e-6, o=o)

        graphs.append((capture_graph(torch, step), ssm, conv))
    steps = max(args.steps, 30)
    for k in range(6):
        graphs[k % 3][0].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        graphs[k % 3][0].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    return {"workload": "decode_bucket256_live200", "call": "gdn_decode", "bucket": case.n, "live": live,
            "graph_ms_per_step": round(ms, 4), "tokens_per_s": round(live / (ms * 1e-3), 1)}


def bench_decode(args, torch, gdn, gi):
    """256 requests x 1 token, in place, rotating over 3 state pools of 512
    slots: the single gdn_decode call, and the two calls gdn_conv1d_update +
    gdn_recurrent_decode."""
    case = gi.decode_case()
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    dev = torch.device("cuda")
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev, torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(case.seed)
    pools = []
    for _ in range(3):
        ssm = torch.randn((case.n_slots, d.h_v, d.d_v, d.d_k), device=dev, generator=gen) * 0.02
        conv = torch.randn((case.n_slots, d.c_ch, d.conv_w - 1), device=dev, generator=gen).to(torch.bfloat16)
        pools.append((ssm, conv))
    x, a, b, z = bf(case.x()), bf(case.a()), bf(case.b()), bf(case.z())
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log = torch.from_numpy(p.A_log).to(dev)
    dt_bias = torch.from_numpy(p.dt_bias).to(dev)
    slots = torch.from_numpy(case.slots).to(dev)
    y = torch.empty_like(x)
    o = torch.empty((case.n, 1, d.h_v, d.d_v), dtype=torch.bfloat16, device=dev)
    steps = max(args.steps, 30)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(k, e=None):
        ssm, conv = pools[k % 3]
        if e: e[0].record()
        gdn.conv1d_update(dims, x, conv_w, conv, slots, y=y)
        if e: e[1].record()
        gdn.recurrent_decode(dims, y, a, b, A_log, dt_bias, ssm, slots, None, 1.0, z, norm_w, 1e-6, o=o)
        if e: e[2].record()
        ssm, conv = pools[(k + 1) % 3]
        gdn.decode(dims, x, conv_w, a, b, A_log, dt_bias, slots, conv, ssm, None, 1.0, z, norm_w, 1e-6, o=o)
        if e: e[3].record()

    for k in range(6):
        step(k)
    torch.cuda.synchronize()
    for k in range(steps):
        step(k, ev[k])
    torch.cuda.synchronize()
    ms = lambda i, j: pct([e[i].elapsed_time(e[j]) for e in ev])
    t_conv, t_rec, t_dec = ms(0, 1), ms(1, 2), ms(2, 3)
    nb_dec = decode_fused_algorithmic(case.n, 1, d.h_k, d.h_v, d.d_k, 2, d.conv_w, 1)
    nb_rec = decode_algorithmic(case.n, 1, d.h_k, d.h_v, d.d_k, 2, 1)
    gbs = nb_dec / (t_dec["mean"] * 1e-3) / 1e9
    gbs_rec = nb_rec / (t_rec["mean"] * 1e-3) / 1e9
    return {"workload": "decode_256x1", "call": "gdn_decode", "kernel": DECODE_KERNEL,
            "traffic": counter_traffic("decode_mtp", (DECODE_KERNEL,)),
            "launch_ms": t_dec, "algorithmic_bytes": nb_dec, "value": round(gbs, 1), "unit": "GB/s",
            "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(case.n / (t_dec["mean"] * 1e-3), 1),
            "separate_calls": {"conv_update_ms": t_conv, "recurrent_ms": t_rec, "recurrent_algorithmic_bytes": nb_rec,
                               "recurrent_gbs": round(gbs_rec, 1), "recurrent_frac": round(gbs_rec / HBM_PEAK_GBS, 4),
                               "tokens_per_s": round(case.n / ((t_conv["mean"] + t_rec["mean"]) * 1e-3), 1)}}


def bench_varlen(args, torch, gdn, gi):
    """The ~271k-token varlen prefill: 64 sequences (lengths 128..8192, seed 0),
    nonzero initial states from a 128-slot pool, on the seeded inputs of the
    parity tests (generated on host threads, sequence by sequence)."""
    from concurrent.futures import ThreadPoolExecutor
    case = gi.varlen_case()
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    dev = torch.device("cuda")
    T, N = case.t_total, case.n_seq
    x = torch.empty((T, d.c_ch), dtype=torch.bfloat16, device=dev)
    a = torch.empty((T, d.h_v), dtype=torch.bfloat16, device=dev)
    b = torch.empty((T, d.h_v), dtype=torch.bfloat16, device=dev)
    z = torch.empty((T, d.h_v, d.d_v), dtype=torch.bfloat16, device=dev)
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev, torch.bfloat16)

    def gen(i):
        return i, case.seq_x(i), case.seq_a(i), case.seq_b(i), case.seq_z(i)

    t_gen = time.perf_counter()
    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        for i, xs, as_, bs, zs in ex.map(gen, range(N)):
            lo, hi = int(case.cu_seqlens[i]), int(case.cu_seqlens[i + 1])
            x[lo:hi], a[lo:hi], b[lo:hi], z[lo:hi] = bf(xs), bf(as_), bf(bs), bf(zs)
    t_gen = time.perf_counter() - t_gen
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log = torch.from_numpy(p.A_log).to(dev)
    dt_bias = torch.from_numpy(p.dt_bias).to(dev)
    cu = torch.from_numpy(case.cu_seqlens).to(dev)
    slots = torch.from_numpy(case.slots).to(dev)
    has_init = torch.ones(N, dtype=torch.uint8, device=dev)
    conv_pool = bf(np.stack([case.slot_conv(s) for s in range(case.n_slots)]))
    ssm_pool = torch.from_numpy(np.stack([case.slot_ssm(s) for s in range(case.n_slots)])).to(dev)
    y = torch.empty_like(x)
    g = torch.empty((T, d.h_v), dtype=torch.float32, device=dev)
    beta = torch.empty_like(g)
    o = torch.empty((T, d.h_v, d.d_v), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(gdn.chunk_prefill_workspace_size(dims, 0, N, T, case.chunk),
                         gdn.prefill_workspace_size(dims, 0, N, T, case.chunk)), dtype=torch.uint8, device=dev)
    steps = max(3, args.steps // 4)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(e=None):
        if e: e[0].record()
        gdn.conv1d_fwd(dims, x, conv_w, cu, slots, conv_pool, has_init, y=y)
        if e: e[1].record()
        gdn.gating(a, b, A_log, dt_bias, g=g, beta=beta)
        if e: e[2].record()
        gdn.chunk_prefill(dims, y, g, beta, cu, slots, ssm_pool, has_init, case.chunk, 1.0, z, norm_w, 1e-6, o=o,
                          workspace=ws)
        if e: e[3].record()

    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]

    def step_fused(e=None):
        if e: e[0].record()
        gdn.prefill(dims, x, conv_w, a, b, A_log, dt_bias, cu, slots, conv_pool, ssm_pool, has_init, case.chunk,
                    1.0, z, norm_w, 1e-6, o=o, workspace=ws)
        if e: e[1].record()

    for fn, evs in ((step, ev), (step_fused, evf)):
        fn()
        torch.cuda.synchronize()
        for k in range(steps):
            fn(evs[k])
        torch.cuda.synchronize()
    ms = lambda evs, i, j: pct([e[i].elapsed_time(e[j]) for e in evs])
    t_step, t_chunk, t_fused = ms(ev, 0, 3), ms(ev, 2, 3), ms(evf, 0, 1)
    nbytes, flops = chunk_algorithmic(T, N, d.h_k, d.h_v, d.d_k, 2, True, case.chunk)
    pbytes, pflops = prefill_algorithmic(T, N, d.h_k, d.h_v, d.d_k, 2, True, case.chunk, d.conv_w)
    del x, y, z, o, ws
    best = min(t_step["mean"], t_fused["mean"])
    rate = lambda nb, t: round(nb / (t["mean"] * 1e-3) / 1e9, 1)
    return {"workload": f"varlen_prefill_{N}seq_{T}tok", "tokens_per_s": round(T / (best * 1e-3), 1),
            "path": "separate calls" if t_step["mean"] <= t_fused["mean"] else "gdn_prefill",
            "inputs": f"seeded (the parity tests' recipe), generated in {t_gen:.1f} s",
            "separate_calls": {"ms_per_step": t_step,
                               "kernels_ms": {"gdn_conv1d_fwd": ms(ev, 0, 1), "gdn_gating": ms(ev, 1, 2),
                                              "gdn_chunk_prefill": t_chunk},
                               "chunk_achieved_gbs": rate(nbytes, t_chunk),
                               "chunk_hbm_frac": round(rate(nbytes, t_chunk) / HBM_PEAK_GBS, 4),
                               "chunk_mfma_frac": round(flops / (t_chunk["mean"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5)},
            "gdn_prefill": {"ms_per_step": t_fused, "achieved_gbs": rate(pbytes, t_fused),
                            "hbm_frac": round(rate(pbytes, t_fused) / HBM_PEAK_GBS, 4),
                            "mfma_frac": round(pflops / (t_fused["mean"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5)}}


def bench_mtp(args, torch, gdn, gi):
    """128 requests x 4 MTP draft tokens: the draft step with per-position state
    and conv-window writes (gdn_decode, and the two calls gdn_conv1d_update +
    gdn_recurrent_decode), then the accepted states committed with
    gdn_state_copy; pools rotated over 3 copies of 640 slots."""
    case = gi.mtp_case()
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    dev = torch.device("cuda")
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev, torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(case.seed)
    pools = []
    for _ in range(3):
        ssm = torch.randn((case.n_slots, d.h_v, d.d_v, d.d_k), device=dev, generator=gen) * 0.02
        conv = torch.randn((case.n_slots, d.c_ch, d.conv_w - 1), device=dev, generator=gen).to(torch.bfloat16)
        pools.append((ssm, conv))
    x, a, b, z = bf(case.x()), bf(case.a()), bf(case.b()), bf(case.z())
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log = torch.from_numpy(p.A_log).to(dev)
    dt_bias = torch.from_numpy(p.dt_bias).to(dev)
    slots = torch.from_numpy(case.slots).to(dev)
    out_slots = torch.from_numpy(case.out_slots).to(dev)
    sel = case.accept > 0
    src = torch.from_numpy(case.out_slots[np.arange(case.n), np.maximum(case.accept - 1, 0)][sel]).to(dev)
    dst = torch.from_numpy(case.slots[sel]).to(dev)
    y = torch.empty_like(x)
    o = torch.empty((case.n, case.t_step, d.h_v, d.d_v), dtype=torch.bfloat16, device=dev)
    steps = max(args.steps, 30)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]

    def step(k, e=None):
        ssm, conv = pools[k % 3]
        if e: e[0].record()
        gdn.conv1d_update(dims, x, conv_w, conv, slots, out_slots, y=y)
        if e: e[1].record()
        gdn.recurrent_decode(dims, y, a, b, A_log, dt_bias, ssm, slots, out_slots, 1.0, z, norm_w, 1e-6, o=o)
        if e: e[2].record()
        gdn.state_copy(dims, ssm, src, dst, conv)
        if e: e[3].record()
        ssm, conv = pools[(k + 1) % 3]
        gdn.decode(dims, x, conv_w, a, b, A_log, dt_bias, slots, conv, ssm, out_slots, 1.0, z, norm_w, 1e-6, o=o)
        if e: e[4].record()
        gdn.state_copy(dims, ssm, src, dst, conv)
        if e: e[5].record()

    for k in range(6):
        step(k)
    torch.cuda.synchronize()
    for k in range(steps):
        step(k, ev[k])
    torch.cuda.synchronize()
    ms = lambda i, j: pct([e[i].elapsed_time(e[j]) for e in ev])
    t_conv, t_rec, t_copy, t_dec, t_copy2 = ms(0, 1), ms(1, 2), ms(2, 3), ms(3, 4), ms(4, 5)
    nb_dec = decode_fused_algorithmic(case.n, case.t_step, d.h_k, d.h_v, d.d_k, 2, d.conv_w, case.t_step)
    nb_rec = decode_algorithmic(case.n, case.t_step, d.h_k, d.h_v, d.d_k, 2, case.t_step)
    copy_bytes = 2.0 * int(sel.sum()) * (d.h_v * d.d_v * d.d_k * 4 + d.c_ch * (d.conv_w - 1) * 2)
    gbs = nb_dec / (t_dec["mean"] * 1e-3) / 1e9
    gbs_rec = nb_rec / (t_rec["mean"] * 1e-3) / 1e9
    return {"workload": f"mtp_{case.n}x{case.t_step}", "call": "gdn_decode",
            "kernel": MTP_KERNEL, "traffic": counter_traffic("decode_mtp", (MTP_KERNEL,)),
            "launch_ms": t_dec, "algorithmic_bytes": nb_dec,
            "value": round(gbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
            "state_copy_ms": t_copy2, "state_copy_gbs": round(copy_bytes / (t_copy2["mean"] * 1e-3) / 1e9, 1),
            "draft_tokens_per_s": round(case.n * case.t_step / ((t_dec["mean"] + t_copy2["mean"]) * 1e-3), 1),
            "separate_calls": {"conv_update_ms": t_conv, "recurrent_ms": t_rec, "state_copy_ms": t_copy,
                               "recurrent_algorithmic_bytes": nb_rec, "recurrent_gbs": round(gbs_rec, 1),
                               "recurrent_frac": round(gbs_rec / HBM_PEAK_GBS, 4),
                               "draft_tokens_per_s": round(case.n * case.t_step /
                                                           ((t_conv["mean"] + t_rec["mean"] + t_copy["mean"]) * 1e-3),
                                                           1)}}


def bench_mtp_bucket(args, torch, gdn, gi):
    """The MTP step as a serving loop runs it: a bucket of 128 requests x
    (mtp_step + 1) = 4 rows, 100 live and 28 pad requests, the draft step
    (gdn_decode) and the commit copy captured as one HIP graph per state pool,
    replayed over 3 pools."""
    case = gi.mtp_case()
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    dev = torch.device("cuda")
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev, torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(case.seed + 1)
    live = 100
    slots_np, out_np = case.slots.copy(), case.out_slots.copy()
    slots_np[live:] = -1
    out_np[live:] = -1
    acc = case.accept.copy()
    acc[live:] = 0
    sel = acc > 0
    src_np = np.where(sel, out_np[np.arange(case.n), np.maximum(acc - 1, 0)], -1).astype(np.int32)
    dst_np = np.where(sel, slots_np, -1).astype(np.int32)
    slots, out_slots = torch.from_numpy(slots_np).to(dev), torch.from_numpy(out_np).to(dev)
    src, dst = torch.from_numpy(src_np).to(dev), torch.from_numpy(dst_np).to(dev)
    x, a, b, z = bf(case.x()), bf(case.a()), bf(case.b()), bf(case.z())
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log, dt_bias = torch.from_numpy(p.A_log).to(dev), torch.from_numpy(p.dt_bias).to(dev)
    o = torch.empty((case.n, case.t_step, d.h_v, d.d_v), dtype=torch.bfloat16, device=dev)
    graphs = []
    for _ in range(3):
        ssm = torch.randn((case.n_slots, d.h_v, d.d_v, d.d_k), device=dev, generator=gen) * 0.02
        conv = torch.randn((case.n_slots, d.c_ch, d.conv_w - 1), device=dev, generator=gen).to(torch.bfloat16)

        def step(ssm=ssm, conv=conv):
            gdn.decode(dims, x, conv_w, a, b, A_log, dt_bias, slots, conv, ssm, out_slots, 1.0, z, norm_w, 1e-6, o=o)
            gdn.state_copy(dims, ssm, src, dst, conv)

        graphs.append((capture_graph(torch, step), ssm, conv))
    steps = max(args.steps, 30)
    for k in range(6):
        graphs[k % 3][0].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        graphs[k % 3][0].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    return {"workload": f"mtp_bucket{case.n}x{case.t_step}_live{live}", "call": "gdn_decode + gdn_state_copy",
            "bucket_requests": case.n, "rows_per_request": case.t_step, "live": live,
            "graph_ms_per_step": round(ms, 4), "draft_tokens_per_s": round(live * case.t_step / (ms * 1e-3), 1)}


def bench_layer(args, torch, gdn, gi):
    """The whole layer around the core at hidden 2048 (a reading: the hidden
    size the pages do not give): Gemma RMSNorm, in_proj_qkvz/ba (one MFMA
    kernel), gdn_prefill, out_proj with the residual, over the 4096-token
    single sequence (two rotating copies, as the prefill row), and the same
    four calls around gdn_decode for 256 requests x 1 token.  Per-call times
    from HIP events on the launch stream; the projections' MFMA fraction
    against the dense bf16 peak, and torch's own GEMM (F.linear, hipBLASLt) on
    the same shapes beside them for reference."""
    import torch.nn.functional as F
    hidden = gi.HIDDEN
    case = gi.prefill_case()
    d = case.dims
    dims = gdn.Dims(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_w)
    dev = torch.device("cuda")
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev, torch.bfloat16)
    T, vd = case.t_total, d.h_v * d.d_v
    n_in = d.c_ch + vd + 2 * d.h_v
    W = gi.block_weights(case.seed, d, hidden)
    wts = gdn.BlockWeights(bf(W.norm_w), bf(W.w_qkvz), bf(W.w_ba), bf(W.w_out))
    p = case.params
    conv_w, norm_w = bf(p.conv_w), bf(p.norm_w)
    A_log, dt_bias = torch.from_numpy(p.A_log).to(dev), torch.from_numpy(p.dt_bias).to(dev)
    cu = torch.tensor(case.cu_seqlens, dtype=torch.int32, device=dev)
    slots = torch.zeros(1, dtype=torch.int32, device=dev)
    has_init = torch.zeros(1, dtype=torch.uint8, device=dev)
    ws_bytes = gdn.prefill_workspace_size(dims, 0, 1, T, case.chunk)
    X0 = gi.block_input(case.seed, 0, T, hidden)
    mk = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device=dev)
    copies = [dict(X=bf(X0), xn=mk(T, hidden), qkv=mk(T, d.c_ch), z=mk(T, d.h_v, d.d_v), b=mk(T, d.h_v),
                   a=mk(T, d.h_v), o=mk(T, d.h_v, d.d_v), y=mk(T, hidden),
                   conv_pool=torch.zeros((1, d.c_ch, d.conv_w - 1), dtype=torch.bfloat16, device=dev),
                   ssm_pool=torch.zeros((1, d.h_v, d.d_v, d.d_k), dtype=torch.float32, device=dev),
                   ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev)) for _ in range(2)]

    def step(k, e=None):
        c = copies[k % 2]
        if e: e[0].record()
        gdn.rmsnorm_gemma(c["X"], wts.norm_w, 1e-6, out=c["xn"])
        if e: e[1].record()
        gdn.in_proj(dims, c["xn"], wts.w_qkvz, wts.w_ba, c["qkv"], c["z"], c["b"], c["a"])
        if e: e[2].record()
        gdn.prefill(dims, c["qkv"], conv_w, c["a"], c["b"], A_log, dt_bias, cu, slots, c["conv_pool"],
                    c["ssm_pool"], has_init, case.chunk, 1.0, c["z"], norm_w, 1e-6, o=c["o"], workspace=c["ws"])
        if e: e[3].record()
        gdn.out_proj(dims, c["o"].view(T, vd), wts.w_out, c["X"], c["y"])
        if e: e[4].record()

    steps = max(min(args.steps, 100), 20)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for k in range(4):
        step(k)
    torch.cuda.synchronize()
    for k in range(steps):
        step(k, evs[k])
    torch.cuda.synchronize()
    graphs = [capture_graph(torch, lambda k=k: step(k)) for k in range(2)]
    for k in range(4):
        graphs[k % 2].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        graphs[k % 2].replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / steps * 1e3
    ms = lambda i, j: pct([e[i].elapsed_time(e[j]) for e in evs])
    t_norm, t_in, t_pre, t_out = ms(0, 1), ms(1, 2), ms(2, 3), ms(3, 4)

    def lib_gemm(x, w):
        """torch's GEMM (F.linear) on the same operands: mean ms of 20 calls."""
        for _ in range(3):
            F.linear(x, w)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            F.linear(x, w)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 20

    c = copies[0]
    w_in = torch.cat([wts.w_qkvz, wts.w_ba])
    lib_in, lib_out = lib_gemm(c["xn"], w_in), lib_gemm(c["o"].view(T, vd), wts.w_out)
    fl_in, fl_out = 2.0 * T * hidden * n_in, 2.0 * T * vd * hidden
    tf = lambda fl, t: fl / (t * 1e-3) / 1e12
    proj = lambda fl, t, lib, kerns: {"kernels": list(kerns), "algorithmic_flops": fl, "launch_ms": t,
                                      "achieved_tflops": round(tf(fl, t["mean"]), 1), "peak_tflops": BF16_PEAK_TFLOPS,
                                      "frac": round(tf(fl, t["mean"]) / BF16_PEAK_TFLOPS, 4),
                                      "traffic": counter_traffic("layer_4096", kerns),
                                      "counters": counter_mfma("layer_4096", kerns),
                                     "torch_f_linear_ms": round(lib, 4), "torch_f_linear_tflops": round(tf(fl, lib), 1)}
    prefill_row = {
        "workload": f"layer_prefill_single_{T}", "hidden": hidden, "calls": "gdn_rmsnorm_gemma, gdn_in_proj, "
        "gdn_prefill, gdn_out_proj (+ residual)", "graph_ms_per_step": round(ms_step, 4),
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "kernels_ms": {"gdn_rmsnorm_gemma": t_norm, "gdn_in_proj": t_in, "gdn_prefill": t_pre, "gdn_out_proj": t_out},
        "in_proj": proj(fl_in, t_in, lib_in, IN_PROJ_KERNELS), "out_proj": proj(fl_out, t_out, lib_out, OUT_PROJ_KERNELS),
        "rmsnorm_gbs": round(2.0 * T * hidden * 2 / (t_norm["mean"] * 1e-3) / 1e9, 1)}
    del copies, graphs
    torch.cuda.empty_cache()

    # decode: 256 requests x 1 token, states in place on a 512-slot pool
    dc = gi.decode_case()
    n = dc.n
    slots_d = torch.from_numpy(dc.slots).to(dev)
    gen = torch.Generator(device=dev).manual_seed(dc.seed + 1)
    ssm = torch.randn((dc.n_slots, d.h_v, d.d_v, d.d_k), device=dev, generator=gen) * 0.02
    conv = torch.randn((dc.n_slots, d.c_ch, d.conv_w - 1), device=dev, generator=gen).to(torch.bfloat16)
    Xd = bf(np.stack([gi.block_input(dc.seed, i, 1, hidden) for i in range(n)]).reshape(n, hidden))
    xn, qkv, z, b, a = mk(n, hidden), mk(n, d.c_ch), mk(n, d.h_v, d.d_v), mk(n, d.h_v), mk(n, d.h_v)
    o, y = mk(n, 1, d.h_v, d.d_v), mk(n, hidden)

    def dstep(e=None):
        if e: e[0].record()
        gdn.rmsnorm_gemma(Xd, wts.norm_w, 1e-6, out=xn)
        if e: e[1].record()
        gdn.in_proj(dims, xn, wts.w_qkvz, wts.w_ba, qkv, z, b, a)
        if e: e[2].record()
        gdn.decode(dims, qkv.view(n, 1, d.c_ch), conv_w, a.view(n, 1, d.h_v), b.view(n, 1, d.h_v), A_log, dt_bias,
                   slots_d, conv, ssm, None, 1.0, z.view(n, 1, d.h_v, d.d_v), norm_w, 1e-6, o=o)
        if e: e[3].record()
        gdn.out_proj(dims, o.view(n, vd), wts.w_out, Xd, y)
        if e: e[4].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for _ in range(4):
        dstep()
    torch.cuda.synchronize()
    for k in range(steps):
        dstep(evs[k])
    torch.cuda.synchronize()
    g = capture_graph(torch, dstep)
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms_dec = (time.perf_counter() - t0) / steps * 1e3
    t_norm, t_in, t_dec, t_out = ms(0, 1), ms(1, 2), ms(2, 3), ms(3, 4)
    w_bytes_in, w_bytes_out = 2.0 * n_in * hidden, 2.0 * hidden * vd
    gbs = lambda nb, t: round(nb / (t["mean"] * 1e-3) / 1e9, 1)
    decode_row = {
        "workload": f"layer_decode_{n}x1", "hidden": hidden, "graph_ms_per_step": round(ms_dec, 4),
        "tokens_per_s": round(n / (ms_dec * 1e-3), 1),
        "kernels_ms": {"gdn_rmsnorm_gemma": t_norm, "gdn_in_proj": t_in, "gdn_decode": t_dec, "gdn_out_proj": t_out},
        "in_proj_weight_gbs": gbs(w_bytes_in + 2.0 * n * (hidden + n_in), t_in),
        "out_proj_weight_gbs": gbs(w_bytes_out + 2.0 * n * (vd + 2 * hidden), t_out),
        "torch_f_linear_ms": {"in_proj": round(lib_gemm(xn, w_in), 4), "out_proj": round(lib_gemm(o.view(n, vd),
                                                                                                   wts.w_out), 4)}}
    return {"prefill": prefill_row, "decode": decode_row}


def cpu_baseline(case2) -> dict:
    """The fp64 oracle, as it stands, on the host's cores: a pool of
    single-threaded worker processes (started before this process touched the
    GPU), one task per V-head pair (prefill) or per group of requests
    (decode, MTP), on every workload or a stated sample of it."""
    from tests import oracle_pool as P
    import gdn_inputs as gi

    cores = P.n_workers()
    res = {}

    def timed(name, fn, tasks, tokens, sample):
        t0 = time.perf_counter()
        P.run_map(fn, tasks)
        dt = time.perf_counter() - t0
        res[name] = {"value": round(tokens / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                     "sample": f"{sample}; {dt:.1f} s wall"}

    T = case2.t_total
    timed("prefill_single_4096", P.prefill_oracle_heads, [(case2, [2 * j, 2 * j + 1]) for j in range(16)], T,
          f"the whole {T}-token sequence, all 32 V heads, one task per V-head pair")
    dec = gi.decode_case()
    timed("decode_256x1", P.decode_oracle_requests, [(dec, list(range(r, r + 16))) for r in range(0, dec.n, 16)],
          dec.n, "all 256 requests, 16 per task")
    mtp = gi.mtp_case()
    timed("mtp_128x4", P.decode_oracle_requests, [(mtp, list(range(r, r + 8))) for r in range(0, mtp.n, 8)],
          mtp.n * mtp.t_step, "all 128 requests x 4 draft tokens, 8 requests per task")
    var = gi.varlen_case()
    seqs = [int(i) for i in np.argsort(var.lengths)[:16]]
    timed("varlen_prefill", P.prefill_oracle_heads, [(var, None, i) for i in seqs],
          int(sum(var.lengths[i] for i in seqs)), "the 16 shortest of the 64 sequences, all heads, one per task")
    out = dict(res["prefill_single_4096"])
    out["per_workload"] = res
    return out


def rocminfo_gpu() -> dict | None:
    """CU count and peak engine clock of the first GPU agent, from rocminfo
    (run before this process touches the GPU)."""
    import subprocess
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.TimeoutExpired):
        return None
    for agent in out.split("*******")[1:]:
        if "Device Type:" in agent and "GPU" in agent.split("Device Type:")[1].split("\n")[0]:
            info = {}
            for line in agent.splitlines():
                key, _, val = line.strip().partition(":")
                if key == "Compute Unit":
                    info["compute_units"] = int(val.split()[0])
                elif key == "Max Clock Freq. (MHz)":
                    info["max_clock_mhz"] = int(val.split()[0])
                elif key == "Name" and "name" not in info:
                    info["name"] = val.strip()
            return info
    return None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-mtp", action="store_true")
    ap.add_argument("--no-tp", action="store_true", help="skip the per-rank (tp = 2, 4) prefill rows")
    ap.add_argument("--no-bucket", action="store_true", help="skip the padded decode and MTP bucket graph rows")
    ap.add_argument("--no-layer", action="store_true", help="skip the whole-layer rows (norm, projections, core)")
    ap.add_argument("--eager", action="store_true", help="time plain launches instead of graph replays")
    ap.add_argument("--prefill-copies", type=int, default=2,
                    help="copies of the prefill buffers the steps rotate over (2: more than the memory-side cache)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the GDN layer's multi-GPU sharding "
              "is a design, not a measured path", file=sys.stderr)
        return 2

    # before anything touches the GPU: the device's CU count and clock, and the
    # CPU worker pool of the oracle baseline (forked from a clean server process)
    rinfo = rocminfo_gpu()
    if not args.no_cpu_baseline:
        from tests.oracle_pool import start_server
        start_server()

    import torch
    import gdn_inputs as gi
    import gated_deltanet_conv1d_amd as gdn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    gdn.lib()
    info = device_info()
    t_start = time.perf_counter()

    def run(name, skip, fn, *a):
        # one progress line per row on stderr; the JSON line is the only stdout
        if skip:
            return None
        r = fn(*a)
        print(f"bench: {name} done ({time.perf_counter() - t_start:.0f} s)", file=sys.stderr, flush=True)
        return r

    pre = run("prefill 4096", False, bench_prefill, args, torch, gdn, gi)
    dec = run("decode 256x1", args.no_decode, bench_decode, args, torch, gdn, gi)
    bucket = run("decode bucket", args.no_decode or args.no_bucket, bench_decode_bucket, args, torch, gdn, gi)
    tp = run("tp shapes", args.no_tp, bench_tp_shapes, args, torch, gdn, gi)
    mtp = run("mtp 128x4", args.no_mtp, bench_mtp, args, torch, gdn, gi)
    mtp_bucket = run("mtp bucket", args.no_mtp or args.no_bucket, bench_mtp_bucket, args, torch, gdn, gi)
    torch.cuda.empty_cache()
    layer = run("layer", args.no_layer, bench_layer, args, torch, gdn, gi)
    torch.cuda.empty_cache()
    var = run("varlen", args.no_varlen, bench_varlen, args, torch, gdn, gi)
    torch.cuda.empty_cache()
    copy_gbs = copy_bandwidth_gbs(torch)
    fill_gbs = fill_bandwidth_gbs(torch)
    cpu = run("cpu baseline", args.no_cpu_baseline, cpu_baseline, pre["inputs"]["case"])
    T = pre["T"]
    line = {
        "metric": METRIC,
        "value": round(T * args.steps / pre["wall_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_single_4096", "batch": 1, "seq_len": T, "h_k": 16, "h_v": 32,
                   "head_dim": 128, "conv_w": 4, "chunk": 64, "state": "fp32",
                   "input_copies": args.prefill_copies, "footprint_bytes": pre["footprint_bytes"]},
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
        "kernels_ms": pre["kernels_ms"],
        "timing": "graph replay" if not args.eager else "eager launches",
        "eager_ms_per_step": round(pre["eager_ms_per_step"], 4),
        "separate_calls": pre["separate_calls"],
        "decode": dec,
        "decode_bucket": bucket,
        "mtp": mtp,
        "mtp_bucket": mtp_bucket,
        "varlen": var,
        "tp_shapes": tp,
        "layer": layer,
        "device": {**info, "rocminfo": rinfo, "copy_gbs": round(copy_gbs, 1), "fill_gbs": round(fill_gbs, 1)},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Offline tuning of the chunked prefill's chain launch shape on this GPU.

    python -m gated_deltanet_conv1d_amd.tune [--out csrc/launch_table.hpp] [--reps 10]
    python -m gated_deltanet_conv1d_amd.tune --build-only --variants DIR   # compile the candidates (no GPU)
    python -m gated_deltanet_conv1d_amd.tune --time-only --variants DIR    # time prebuilt candidates
    python -m gated_deltanet_conv1d_amd.tune --from-json FILE              # table from stored timings

For every candidate shape (d_v tiles per chain workgroup, prefetch stages) it
copies the kernel sources, pins the launch table to that one shape, builds the
copy (under --variants, default _build/tune/), and times gdn_prefill with it on
a grid of workloads: n_seq sequences of L tokens each at the 16 QK / 32 V head,
d = 128 layout, bf16, chunk 64, two copies of every buffer alternated.  Each
variant is timed in its own process (one library per process).  For each
sequence count the shape fastest over its lengths becomes a row of the launch
table the library consults at run time (csrc/launch_table.hpp), and the
timings are written next to it as JSON.  The states do not depend on the
shape; the outputs of the whole-d_v chain (ntw 8), which computes them
itself, can differ from the output pass's in the last bit.
"""
from __future__ import annotations

import argparse
import json
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")

# candidate (ntw, pd): tiles per chain workgroup, register stages of the
# prefetch; ntw 8 (all of d_v) is the chain that computes the output itself
CANDIDATES = [(1, 2), (1, 3), (1, 4), (1, 5), (1, 6), (2, 2), (2, 3), (2, 4), (4, 2), (4, 3), (8, 2), (8, 3)]
# grid: sequences per batch x tokens per sequence (at most 2^19 tokens per batch)
N_SEQ = [1, 2, 4, 8, 16, 32, 64]
LENGTHS = [512, 2048, 8192]
MAX_TOKENS = 1 << 19
H_K, H_V, D, W, CHUNK = 16, 32, 128, 4, 64


def table_source(rows, shapes) -> str:
    """launch_table.hpp for the given rows [(max_chains, max_len, ntw, pd)]."""
    lim = lambda v: "INT64_MAX" if v is None else str(v)
    body = "\n".join(f"    {{{lim(c)}, {lim(l)}, {n}, {p}}}," for c, l, n, p in rows)
    cases = " ".join(f"X({n}, {p})" for n, p in shapes)
    return f"""// Launch shapes of the chunked prefill's chain pass, by workload: written by
// gated_deltanet_conv1d_amd/tune.py from timings of every candidate shape on
// one MI355X (the table below is that script's output; rerun it to retune).
//
// A row applies to a call whose number of (sequence, V head) chains is at most
// max_chains and whose mean sequence length is at most max_len (the first
// matching row wins).  ntw: 16-wide d_v tiles per chain workgroup (they share
// each -W and K^T load), 8 = all of d_v in one workgroup, which then also
// computes the output (no output pass); pd: register stages of the
// chunk-operand prefetch.  The states do not depend on the shape (every
// accumulator sees the same MFMA order); the outputs of the whole-d_v chain
// can differ from the output pass's in the last bit (its products and norm
// sum run in another order).
#pragma once
#include <stdint.h>

namespace gdn {{

struct ChainShape {{
  int64_t max_chains;  // sequences x V heads
  int64_t max_len;     // mean tokens per sequence
  int ntw, pd;
}};

constexpr ChainShape kChainTable[] = {{
{body}
}};

// The (ntw, pd) pairs the table uses, each instantiated once per kernel type.
#define GDN_CHAIN_SHAPES(X) {cases}

inline ChainShape chain_shape(int64_t chains, int64_t mean_len) {{
  for (const ChainShape& s : kChainTable)
    if (chains <= s.max_chains && mean_len <= s.max_len) return s;
  return kChainTable[sizeof(kChainTable) / sizeof(kChainTable[0]) - 1];
}}

}}  // namespace gdn
"""


def variant_lib(vroot: str, ntw: int, pd: int) -> str:
    return os.path.join(vroot, f"ntw{ntw}_pd{pd}", "libgdn.so")


def build_variant(vroot: str, ntw: int, pd: int) -> str:
    """Compile a copy of the sources with the launch table pinned to (ntw, pd)."""
    from gated_deltanet_conv1d_amd.build import build
    vdir = os.path.join(vroot, f"ntw{ntw}_pd{pd}")
    src = os.path.join(vdir, "src", "csrc")
    shutil.rmtree(vdir, ignore_errors=True)
    shutil.copytree(CSRC, src)
    with open(os.path.join(src, "launch_table.hpp"), "w") as f:
        f.write(table_source([(None, None, ntw, pd)], [(ntw, pd)]))
    # the C-ABI sources reach include/gdn.h by a relative path: keep it valid
    os.makedirs(os.path.join(vdir, "include"), exist_ok=True)
    shutil.copy(os.path.join(ROOT, "include", "gdn.h"), os.path.join(vdir, "include", "gdn.h"))
    lib = build(verbose=False, csrc=src, lib=variant_lib(vroot, ntw, pd), build_dir=os.path.join(vdir, "obj"))
    shutil.rmtree(os.path.join(vdir, "src"))
    shutil.rmtree(os.path.join(vdir, "obj"))
    shutil.rmtree(os.path.join(vdir, "include"))
    return lib


def time_variant(lib_path: str, reps: int) -> dict:
    """Median gdn_prefill time (ms) per grid cell with the library at lib_path."""
    import numpy as np
    import torch

    from gated_deltanet_conv1d_amd import binding as B
    B.lib(lib_path)
    dev = torch.device("cuda")
    dims = B.Dims(H_K, H_V, D, D, W)
    g = torch.Generator(device=dev).manual_seed(0)
    out = {}
    for n in N_SEQ:
        for L in LENGTHS:
            if n * L > MAX_TOKENS:
                continue
            T = n * L
            rnd = lambda *s: torch.randn(s, device=dev, generator=g).to(torch.bfloat16)
            conv_w, norm_w = rnd(dims.c_ch, W), rnd(D)
            A_log = torch.rand(H_V, device=dev, generator=g) * 2.7
            dt_bias = torch.rand(H_V, device=dev, generator=g) * 2 - 1
            cu = torch.arange(0, T + 1, L, dtype=torch.int32, device=dev)
            slots = torch.arange(n, dtype=torch.int32, device=dev)
            has_init = torch.ones(n, dtype=torch.uint8, device=dev)
            # two copies of every buffer, alternated, so the calls see HBM, not
            # the memory-side cache, as the layers of a model do
            sets = [dict(x=rnd(T, dims.c_ch), a=rnd(T, H_V), b=rnd(T, H_V), z=rnd(T, H_V, D),
                         conv_pool=rnd(n, dims.c_ch, W - 1),
                         ssm_pool=torch.randn((n, H_V, D, D), device=dev, generator=g) * 0.02,
                         o=torch.empty((T, H_V, D), dtype=torch.bfloat16, device=dev),
                         ws=torch.empty(B.prefill_workspace_size(dims, 0, n, T, CHUNK), dtype=torch.uint8,
                                        device=dev)) for _ in range(2)]

            def call(k):
                c = sets[k % 2]
                B.prefill(dims, c["x"], conv_w, c["a"], c["b"], A_log, dt_bias, cu, slots, c["conv_pool"],
                          c["ssm_pool"], has_init, CHUNK, 1.0, c["z"], norm_w, 1e-6, o=c["o"], workspace=c["ws"])

            call(0)
            call(1)
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for k, (e0, e1) in enumerate(ev):
                e0.record()
                call(k)
                e1.record()
            torch.cuda.synchronize()
            out[f"{n}x{L}"] = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
            del sets
            torch.cuda.empty_cache()
    return out


def choose(times: dict) -> list:
    """Table rows from {shape: {cell: ms}}: for each sequence count (chain
    count n * h_v) the shape with the smallest sum over lengths of time / best
    time of the cell, so one shape serves all lengths of a chain count; runs of
    chain counts that pick the same shape merge, the last row is open-ended."""
    ns = [n for n in N_SEQ if any(n * L <= MAX_TOKENS for L in LENGTHS)]
    picks = []
    for n in ns:
        cells = [f"{n}x{L}" for L in LENGTHS if n * L <= MAX_TOKENS]
        best = {c: min(times[s][c] for s in times) for c in cells}
        score = {s: sum(times[s][c] / best[c] for c in cells) for s in times}
        picks.append((n * H_V, min(score, key=score.get)))
    rows = []
    for chains, shape in picks:
        ntw, pd = (int(v) for v in shape.split(","))
        if rows and rows[-1][2:] == (ntw, pd):
            rows[-1] = (chains, None, ntw, pd)
        else:
            rows.append((chains, None, ntw, pd))
    rows[-1] = (None, None) + rows[-1][2:]
    return rows


def write_table(out: str, rows) -> None:
    shapes = sorted({(n, p) for _, _, n, p in rows})
    with open(out, "w") as f:
        f.write(table_source(rows, shapes))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(CSRC, "launch_table.hpp"))
    ap.add_argument("--json", default=os.path.join(ROOT, "profiles", "chain_launch_tuning.json"))
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--variants", default=os.path.join(ROOT, "_build", "tune"), help="where the candidate builds go")
    ap.add_argument("--build-only", action="store_true")
    ap.add_argument("--build-jobs", type=int, default=4, help="variants compiled at once")
    ap.add_argument("--time-only", action="store_true")
    ap.add_argument("--from-json", help="rewrite the table from the timings stored in this JSON file")
    ap.add_argument("--time", help=argparse.SUPPRESS)       # internal: time one built variant
    ap.add_argument("--time-out", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.from_json:      # rewrite the table from stored timings
        with open(args.from_json) as f:
            rec = json.load(f)
        rows = choose(rec["median_ms"])
        rec["table"] = [list(r) for r in rows]
        write_table(args.out, rows)
        with open(args.json, "w") as f:
            json.dump(rec, f, indent=1)
        print(f"tune: wrote {args.out} ({len(rows)} rows) and {args.json}", file=sys.stderr)
        return 0
    if args.time:
        with open(args.time_out, "w") as f:
            json.dump(time_variant(args.time, args.reps), f)
        return 0
    if not args.time_only:
        # the variants compile independently: a few at a time (each build runs
        # its own sources in parallel as well)
        import concurrent.futures as cf

        def one(shape):
            t0 = time.time()
            build_variant(args.variants, *shape)
            print(f"tune: built shape {shape} in {time.time() - t0:.0f} s", file=sys.stderr, flush=True)

        with cf.ThreadPoolExecutor(max_workers=args.build_jobs) as ex:
            list(ex.map(one, CANDIDATES))
    if args.build_only:
        return 0
    times = {}
    for ntw, pd in CANDIDATES:
        t0 = time.time()
        lib = variant_lib(args.variants, ntw, pd)
        res = os.path.join(os.path.dirname(lib), "times.json")
        r = subprocess.run([sys.executable, "-m", "gated_deltanet_conv1d_amd.tune", "--time", lib, "--time-out", res,
                            "--reps", str(args.reps)], cwd=ROOT)
        if r.returncode != 0:
            print(f"tune: shape ({ntw}, {pd}) failed to run (rc {r.returncode}); left out", file=sys.stderr)
            continue
        with open(res) as f:
            times[f"{ntw},{pd}"] = json.load(f)
        print(f"tune: shape ({ntw}, {pd}) timed in {time.time() - t0:.0f} s", file=sys.stderr, flush=True)
    rows = choose(times)
    write_table(args.out, rows)
    with open(args.json, "w") as f:
        json.dump({"command": " ".join(["python -m gated_deltanet_conv1d_amd.tune"] + sys.argv[1:]),
                   "grid": {"n_seq": N_SEQ, "lengths": LENGTHS, "max_tokens": MAX_TOKENS,
                            "layout": f"h_k {H_K}, h_v {H_V}, d {D}, conv_w {W}, chunk {CHUNK}, bf16"},
                   "median_ms": times, "table": [list(r) for r in rows]}, f, indent=1)
    print(f"tune: wrote {args.out} ({len(rows)} rows) and {args.json}", file=sys.stderr)
    return 0


if __name__ == "__main__":
    sys.exit(main())

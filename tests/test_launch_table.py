"""The chain launch table (csrc/launch_table.hpp) is well formed and is the
tuner's choice from the timings stored beside it.  No GPU needed."""
from __future__ import annotations

import json
import os
import re

from gated_deltanet_conv1d_amd import tune

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "gated_deltanet_conv1d_amd", "csrc", "launch_table.hpp")
TIMINGS = os.path.join(ROOT, "profiles", "chain_launch_tuning.json")
D_V = 128


def table_rows():
    """[(max_chains or None, max_len or None, ntw, pd)] and the instantiated shapes."""
    src = open(HEADER).read()
    body = src[src.index("kChainTable[] = {"):src.index("};", src.index("kChainTable[] = {"))]
    lim = lambda v: None if v == "INT64_MAX" else int(v)
    rows = [(lim(a), lim(b), int(c), int(d))
            for a, b, c, d in re.findall(r"\{(\w+), (\w+), (\d+), (\d+)\}", body)]
    shapes = [(int(a), int(b)) for a, b in re.findall(r"X\((\d+), (\d+)\)", src.split("#define GDN_CHAIN_SHAPES(X)")[1]
                                                      .splitlines()[0])]
    return rows, shapes


def test_table_well_formed():
    rows, shapes = table_rows()
    assert rows, "empty table"
    limits = [r[0] for r in rows[:-1]]
    assert all(v is not None for v in limits) and limits == sorted(limits) and len(set(limits)) == len(limits)
    assert rows[-1][0] is None and rows[-1][1] is None          # the last row takes every call
    used = {(n, p) for _, _, n, p in rows}
    assert used == set(shapes) and len(shapes) == len(set(shapes))
    for n, p in used:
        assert (n, p) in tune.CANDIDATES
        assert (D_V // 16) % n == 0 and p >= 1


def test_table_is_the_tuners_choice():
    rows, _ = table_rows()
    with open(TIMINGS) as f:
        rec = json.load(f)
    assert [tuple(r) for r in rec["table"]] == rows
    assert tune.choose(rec["median_ms"]) == rows
    # every candidate was timed on every grid cell
    cells = {f"{n}x{L}" for n in tune.N_SEQ for L in tune.LENGTHS if n * L <= tune.MAX_TOKENS}
    assert set(rec["median_ms"]) == {f"{n},{p}" for n, p in tune.CANDIDATES}
    assert all(set(v) == cells for v in rec["median_ms"].values())


def test_table_source_round_trip(tmp_path):
    rows, _ = table_rows()
    out = tmp_path / "t.hpp"
    tune.write_table(str(out), rows)
    assert out.read_text() == open(HEADER).read()

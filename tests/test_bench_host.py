"""Host-side checks of bench.py: the algorithmic byte and flop counts behind
the roofline fields, recounted here from first principles for the workloads'
shapes, the rule that counter traffic applies only to the kernel sources it
was taken on, and the one-GPU guard.  No GPU needed."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

H_K, H_V, D, W = 16, 32, 128, 4
C_CH = 2 * H_K * D + H_V * D  # 8192 packed conv channels
STATE = H_V * D * D * 4       # one request's fp32 states: 2 MiB


def test_decode_bytes_per_request_token():
    # per token: the q, k, v row (bf16), a and b (bf16 per V head), z read and o written (bf16)
    per_tok = C_CH * 2 + 2 * H_V * 2 + 2 * H_V * D * 2
    assert per_tok == 32_896
    # in place: every state read once and written once
    assert bench.decode_algorithmic(256, 1, H_K, H_V, D, 2, 1) == 256 * (2 * STATE + per_tok) == 1_082_163_200
    # MTP, 4 drafts: the home state read once, one state written per draft position
    assert bench.decode_algorithmic(128, 4, H_K, H_V, D, 2, 4) == 128 * (5 * STATE + 4 * per_tok) == 1_359_020_032


def test_prefill_bytes():
    T = 4096
    per_tok = C_CH * 2 + 2 * H_V * 2 + 2 * H_V * D * 2        # x row, a/b, z and o
    per_seq = STATE + C_CH * (W - 1) * 2                        # final state and conv window, no history
    nbytes, _ = bench.prefill_algorithmic(T, 1, H_K, H_V, D, 2, False, 64, W)
    assert nbytes == T * per_tok + per_seq == 136_888_320
    # with history the state and the window are read as well
    nbytes_h, _ = bench.prefill_algorithmic(T, 1, H_K, H_V, D, 2, True, 64, W)
    assert nbytes_h == nbytes + per_seq


def test_prefill_flops_by_term():
    """Per (64-token chunk, V head), 2 flops per multiply-add, only the entries the
    method uses: K K^T strictly below the diagonal and Q K^T on and below it,
    over d_k, once per QK head (its two V heads share them); W = T diag(..) K,
    Ut = T diag(b) V and (M o Q K^T) U with a lower-triangular C x C factor,
    C (C + 1) / 2 terms per column of d; the unit lower-triangular inverse,
    C^3 / 3; W S^T, Q S^T and K^T U, C d^2 multiply-adds each."""
    T, Cn = 4096, 64
    gram = 2 * D * (Cn * (Cn - 1) // 2 + Cn * (Cn + 1) // 2) / (H_V // H_K)
    chunk_products = 3 * (2 * D * Cn * (Cn + 1) / 2)
    inverse = Cn ** 3 / 3
    state_products = 3 * (2 * Cn * D * D)
    per_chunk_head = gram + chunk_products + inverse + state_products
    conv = 2 * W * C_CH * T
    _, flops = bench.prefill_algorithmic(T, 1, H_K, H_V, D, 2, False, Cn, W)
    assert flops == pytest.approx((T // Cn) * H_V * per_chunk_head + conv, rel=1e-12)
    # about 4.25 MFLOP per token for the chunked rule alone
    assert (flops - conv) / T == pytest.approx(4.25e6, rel=2e-3)


def test_counter_traffic_only_for_the_sources_it_was_taken_on(monkeypatch):
    path = os.path.join(ROOT, "profiles", "prefill_4096_traffic.json")
    with open(path) as f:
        rec = json.load(f)
    per = rec["per_dispatch"]
    expect = sum(per[k]["read_bytes"] + per[k]["write_bytes"] for k in bench.PREFILL_KERNELS)
    monkeypatch.setattr(bench, "kernel_src_sha", lambda: rec["src_sha"])
    assert bench.counter_traffic("prefill_4096", bench.PREFILL_KERNELS) == pytest.approx(expect)
    monkeypatch.setattr(bench, "kernel_src_sha", lambda: "0" * 16)
    assert bench.counter_traffic("prefill_4096", bench.PREFILL_KERNELS) is None
    monkeypatch.setattr(bench, "kernel_src_sha", lambda: rec["src_sha"])
    assert bench.counter_traffic("prefill_4096", ("no such kernel",)) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_single_call_decode_bytes():
    # gdn_decode reads the conv input row instead of the conv output, and moves the
    # conv window (bf16, c_ch x (W-1)) with each state read or write
    per_tok = C_CH * 2 + 2 * H_V * 2 + 2 * H_V * D * 2
    window = C_CH * (W - 1) * 2
    assert bench.decode_fused_algorithmic(256, 1, H_K, H_V, D, 2, W, 1) == 256 * (2 * (STATE + window) + per_tok)
    assert bench.decode_fused_algorithmic(128, 4, H_K, H_V, D, 2, W, 4) == 128 * (5 * (STATE + window) + 4 * per_tok)


def test_percentiles():
    p = bench.pct([1.0, 2.0, 3.0, 4.0, 100.0])
    assert p["median"] == 3.0 and p["mean"] == 22.0
    assert p["p10"] == pytest.approx(1.4) and p["p90"] == pytest.approx(61.6)

"""Host-only checks of the C ABI (no GPU needed).

The library must load and export every entry point declared in
include/gdn.h, and argument validation must return the documented status
codes before anything touches the device.
"""
import ctypes
import os
import re

import pytest

import gated_deltanet_conv1d_amd as gdn
from gated_deltanet_conv1d_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, DTYPE, UNSUP, WS, HIP, ALIGN = 0, -1, -2, -3, -4, -5, -6, -7


def header_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return gdn.lib()


def D(h_k=16, h_v=32, d=128, w=4):
    return ctypes.byref(binding._CDims(h_k, h_v, d, d, w))


FAKE = 0x1000  # a 16-byte-aligned non-null address: every call below must fail validation,
# so nothing is ever launched with it


def test_exports_every_header_symbol(L):
    names = header_functions()
    assert len(names) == 18
    for n in names:
        assert hasattr(L, n), n
        assert n in binding.SIGNATURES, n


def test_version_and_status_strings(L):
    assert gdn.version() == "0.1.0"
    for code in (OK, NULL, SHAPE, DTYPE, UNSUP, WS, HIP, ALIGN):
        assert L.gdn_status_string(code).decode().startswith(binding._STATUS[code])


def test_dims_validation(L):
    args = (0, 1, 8, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1, FAKE + 16, None)
    assert L.gdn_conv1d_fwd(None, *args) == NULL
    assert L.gdn_conv1d_fwd(D(h_k=3, h_v=32), *args) == SHAPE          # h_v % h_k
    assert L.gdn_conv1d_fwd(D(d=96), *args) == UNSUP
    assert L.gdn_conv1d_fwd(D(w=5), *args) == UNSUP
    assert L.gdn_conv1d_fwd(D(h_k=0), *args) == SHAPE
    assert L.gdn_conv1d_fwd(D(), 7, *args[1:]) == DTYPE


def test_conv_fwd_argument_errors(L):
    assert L.gdn_conv1d_fwd(D(), 0, -1, 8, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1, FAKE + 16, None) == SHAPE
    assert L.gdn_conv1d_fwd(D(), 0, 0, 8, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1, FAKE + 16, None) == SHAPE
    assert L.gdn_conv1d_fwd(D(), 0, 0, 0, None, None, None, None, None, None, None, 1, None, None) == OK
    assert L.gdn_conv1d_fwd(D(), 0, 1, 8, None, FAKE, None, FAKE, FAKE, None, FAKE, 1, FAKE + 16, None) == NULL
    assert L.gdn_conv1d_fwd(D(), 0, 1, 8, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1, FAKE, None) == SHAPE  # y == x
    assert L.gdn_conv1d_fwd(D(), 0, 1, 8, FAKE + 2, FAKE, None, FAKE, FAKE, None, FAKE, 1, FAKE + 16, None) == ALIGN


def test_update_and_gating_errors(L):
    assert L.gdn_conv1d_update(D(), 0, -1, 1, FAKE, FAKE, None, FAKE, 4, FAKE, None, FAKE + 16, None) == SHAPE
    assert L.gdn_conv1d_update(D(), 0, 2, 1, None, FAKE, None, FAKE, 4, FAKE, None, FAKE + 16, None) == NULL
    assert L.gdn_conv1d_update(D(), 0, 0, 1, None, None, None, None, 4, None, None, None, None) == OK
    assert L.gdn_gating(0, 10, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_gating(2, 10, 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == DTYPE
    assert L.gdn_gating(0, 10, 32, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == NULL
    assert L.gdn_gating(0, 0, 32, None, None, None, None, None, None, None) == OK


def chunk_call(L, dims=None, act=0, n_seq=1, t_total=64, chunk=64, z=None, norm_w=None, eps=1e-6, qkv=FAKE,
               ws=None, ws_bytes=0):
    return L.gdn_chunk_prefill(dims or D(), act, n_seq, t_total, chunk, 1.0, qkv, FAKE, FAKE, FAKE, FAKE, None,
                               FAKE, 4, FAKE + 16, z, norm_w, eps, ws, ws_bytes, None)


def test_chunk_prefill_errors(L):
    assert chunk_call(L, chunk=48) == UNSUP
    assert chunk_call(L, chunk=128) == UNSUP
    assert chunk_call(L, act=1, chunk=64) == WS             # fp32 at d=128, C=64 is supported
    assert chunk_call(L, z=FAKE) == NULL                     # z without norm_w
    assert chunk_call(L, eps=-1.0) == SHAPE
    assert chunk_call(L, qkv=None) == NULL
    assert chunk_call(L, qkv=FAKE + 8) == ALIGN
    assert chunk_call(L, n_seq=0, t_total=5) == SHAPE
    assert chunk_call(L, n_seq=0, t_total=0) == OK


def test_chunk_prefill_workspace(L):
    ws = L.gdn_chunk_prefill_workspace_size(D(), 0, 1, 4096, 64)
    # a 256-byte-aligned chunk index, then one 256-byte-aligned unit
    # per (chunk, V head) holding -W, K^T, Ut (bf16, C x D each), P (bf16 hi and lo, C x C each),
    # the chunk-start state (bf16, D x D), e^{G_n} (16 bytes), f_q and f_k (fp32,
    # C each) and the old conv window of the q channels (bf16, D x 3; single-call prefill)
    unit = (3 * 64 * 128 * 2 + 2 * 64 * 64 * 2 + 128 * 128 * 2 + 16 + 2 * 64 * 4 + 128 * 3 * 2 + 255) // 256 * 256
    assert ws == 256 + (4096 // 64 + 1) * 32 * unit
    # (same sizes as the query, so these calls stop at validation and never launch)
    assert chunk_call(L, t_total=4096) == WS
    assert chunk_call(L, t_total=4096, ws=FAKE, ws_bytes=ws - 1) == WS
    assert L.gdn_chunk_prefill_workspace_size(None, 0, 1, 4096, 64) == 0


def prefill_call(L, dims=None, act=0, n_seq=1, t_total=64, chunk=64, x=FAKE, a=FAKE, conv_state=FAKE, z=None,
                 norm_w=None, eps=1e-6, ws=None, ws_bytes=0):
    return L.gdn_prefill(dims or D(), act, n_seq, t_total, chunk, 1.0, x, FAKE, None, a, FAKE, FAKE, FAKE, FAKE,
                         FAKE, None, conv_state, FAKE, 4, FAKE + 16, z, norm_w, eps, ws, ws_bytes, None)


def test_prefill_errors_and_workspace(L):
    assert prefill_call(L, chunk=48) == UNSUP
    assert prefill_call(L, act=1, chunk=64) == WS             # fp32 at d=128, C=64 is supported
    assert prefill_call(L, z=FAKE) == NULL                     # z without norm_w
    assert prefill_call(L, eps=-1.0) == SHAPE
    assert prefill_call(L, x=None) == NULL
    assert prefill_call(L, a=None) == NULL
    assert prefill_call(L, conv_state=None) == NULL
    assert prefill_call(L, x=FAKE + 8) == ALIGN
    assert prefill_call(L, n_seq=0, t_total=5) == SHAPE
    assert prefill_call(L, n_seq=0, t_total=0) == OK
    # the same workspace as gdn_chunk_prefill
    ws = L.gdn_prefill_workspace_size(D(), 0, 1, 4096, 64)
    unit = (3 * 64 * 128 * 2 + 2 * 64 * 64 * 2 + 128 * 128 * 2 + 16 + 2 * 64 * 4 + 128 * 3 * 2 + 255) // 256 * 256
    assert ws == 256 + (4096 // 64 + 1) * 32 * unit
    assert prefill_call(L, t_total=4096) == WS                # (these stop at validation, never launch)
    assert prefill_call(L, t_total=4096, ws=FAKE, ws_bytes=ws - 1) == WS


def test_recurrent_and_copy_errors(L):
    base = (1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, None, FAKE + 16, None, None, 1e-6, None)
    assert L.gdn_recurrent_decode(D(), 0, -2, 1, *base) == SHAPE
    assert L.gdn_recurrent_decode(D(), 0, 0, 1, *base) == OK
    assert L.gdn_recurrent_decode(D(), 0, 2, 1, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 8, FAKE, None,
                                  FAKE + 16, None, None, 1e-6, None) == NULL
    assert L.gdn_recurrent_decode(D(), 0, 2, 1, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, None,
                                  FAKE + 16, FAKE, None, 1e-6, None) == NULL
    assert L.gdn_state_copy(D(), 0, FAKE, None, 8, FAKE, FAKE, -1, None) == SHAPE
    assert L.gdn_state_copy(D(), 0, None, None, 8, FAKE, FAKE, 3, None) == NULL
    assert L.gdn_state_copy(D(), 0, FAKE, FAKE + 4, 8, FAKE, FAKE, 3, None) == ALIGN
    assert L.gdn_state_copy(D(), 0, None, None, 8, None, None, 0, None) == OK


def decode_call(L, dims=None, act=0, n_seq=2, t_step=1, x=FAKE, conv_state=FAKE, state=FAKE, z=None, norm_w=None,
                eps=1e-6, out_slots=None):
    return L.gdn_decode(dims or D(), act, n_seq, t_step, 1.0, x, FAKE, None, FAKE, FAKE, FAKE, FAKE, conv_state, state,
                        8, FAKE, out_slots, FAKE + 16, z, norm_w, eps, None)


def test_decode_errors(L):
    assert decode_call(L, n_seq=-1) == SHAPE
    assert decode_call(L, t_step=-1) == SHAPE
    assert decode_call(L, n_seq=0) == OK
    assert decode_call(L, t_step=0) == OK
    assert decode_call(L, x=None) == NULL
    assert decode_call(L, conv_state=None) == NULL
    assert decode_call(L, state=None) == NULL
    assert decode_call(L, z=FAKE) == NULL                     # z without norm_w
    assert decode_call(L, eps=-1.0) == SHAPE
    assert decode_call(L, x=FAKE + 8) == ALIGN
    assert decode_call(L, act=5) == DTYPE
    assert decode_call(L, dims=D(h_k=4, h_v=16)) == UNSUP     # 4 V heads per QK head


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, gdn.Dims().c_ch, dtype=torch.bfloat16)
    with pytest.raises(gdn.GdnError):
        gdn.conv1d_fwd(gdn.Dims(), x, torch.zeros(gdn.Dims().c_ch, 4, dtype=torch.bfloat16),
                       torch.tensor([0, 4], dtype=torch.int32), torch.tensor([0], dtype=torch.int32),
                       torch.zeros(1, gdn.Dims().c_ch, 3, dtype=torch.bfloat16))


def test_block_argument_errors(L):
    F1, F2, F3 = FAKE + 4096, FAKE + 8192, FAKE + 12288
    assert L.gdn_rmsnorm_gemma(0, 4, 12, FAKE, F1, 1e-6, F2, None) == SHAPE        # hidden % 8
    assert L.gdn_rmsnorm_gemma(0, -1, 16, FAKE, F1, 1e-6, F2, None) == SHAPE
    assert L.gdn_rmsnorm_gemma(0, 4, 16, FAKE, F1, -1.0, F2, None) == SHAPE         # eps < 0
    assert L.gdn_rmsnorm_gemma(0, 0, 16, None, None, 1e-6, None, None) == OK
    assert L.gdn_rmsnorm_gemma(0, 4, 16, None, F1, 1e-6, F2, None) == NULL
    assert L.gdn_rmsnorm_gemma(2, 4, 16, FAKE, F1, 1e-6, F2, None) == DTYPE
    assert L.gdn_rmsnorm_gemma(0, 4, 16, FAKE + 8, F1, 1e-6, F2, None) == ALIGN
    ptrs = [FAKE, F1, F2, F3, F3 + 4096, F3 + 8192, F3 + 12288]
    assert L.gdn_in_proj(D(), 1, 8, 2048, *ptrs, None) == UNSUP                      # fp32 projections
    assert L.gdn_in_proj(D(), 0, 8, 2047, *ptrs, None) == SHAPE
    assert L.gdn_in_proj(D(), 0, -1, 2048, *ptrs, None) == SHAPE
    assert L.gdn_in_proj(D(), 0, 0, 2048, *([None] * 7), None) == OK
    assert L.gdn_in_proj(D(), 0, 8, 2048, *ptrs[:2], None, *ptrs[3:], None) == NULL   # no w_ba
    assert L.gdn_in_proj(D(d=96), 0, 8, 2048, *ptrs, None) == UNSUP
    assert L.gdn_out_proj(D(), 0, 8, 2048, FAKE, F1, F2 + 2, F3, None) == ALIGN    # residual
    assert L.gdn_out_proj(D(), 1, 8, 2048, FAKE, F1, None, F3, None) == UNSUP
    assert L.gdn_out_proj(D(), 0, 8, 0, FAKE, F1, None, F3, None) == SHAPE
    assert L.gdn_out_proj(D(), 0, 8, 2048, FAKE, None, None, F3, None) == NULL
    assert L.gdn_out_proj(D(), 0, 0, 2048, None, None, None, None, None) == OK


def test_binding_rejects_wrong_output_shapes():
    """The binding checks caller-provided outputs and optional inputs against
    the dimensions before any call (the kernels size every access from the
    dimensions, so a smaller buffer would be written past its end).  CPU
    tensors: each call must fail on the shape, before the device check."""
    import torch
    dims = gdn.Dims(16, 32, 128, 128, 4)
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    T, n, c = 10, 2, dims.c_ch
    conv, ssm = bf(4, c, 3), f32(4, 32, 128, 128)
    cases = [
        ("o", lambda: gdn.prefill(dims, bf(T, c), bf(c, 4), bf(T, 32), bf(T, 32), f32(32), f32(32), i32(n + 1),
                                  i32(n), conv, ssm, o=bf(T - 1, 32, 128))),
        ("z", lambda: gdn.prefill(dims, bf(T, c), bf(c, 4), bf(T, 32), bf(T, 32), f32(32), f32(32), i32(n + 1),
                                  i32(n), conv, ssm, z=bf(T, 32, 64))),
        ("o", lambda: gdn.decode(dims, bf(n, 1, c), bf(c, 4), bf(n, 1, 32), bf(n, 1, 32), f32(32), f32(32), i32(n),
                                 conv, ssm, o=bf(n, 1, 32, 127))),
        ("y", lambda: gdn.conv1d_fwd(dims, bf(T, c), bf(c, 4), i32(n + 1), i32(n), conv, y=bf(T, c - 8))),
        ("g", lambda: gdn.gating(bf(T, 32), bf(T, 32), f32(32), f32(32), g=f32(T, 16))),
        ("o", lambda: gdn.chunk_prefill(dims, bf(T, c), f32(T, 32), f32(T, 32), i32(n + 1), i32(n), ssm,
                                        o=bf(T, 32, 64))),
        ("o", lambda: gdn.recurrent_decode(dims, bf(n, 2, c), bf(n, 2, 32), bf(n, 2, 32), f32(32), f32(32), ssm,
                                           i32(n), i32(n, 2), o=bf(n, 1, 32, 128))),
        ("out", lambda: gdn.rmsnorm_gemma(bf(T, 64), bf(64), out=bf(T, 32))),
        ("z", lambda: gdn.in_proj(dims, bf(T, 64), bf(c + 4096, 64), bf(64, 64), z=bf(T, 32, 127))),
        ("y", lambda: gdn.out_proj(dims, bf(T, 4096), bf(64, 4096), y=bf(T - 2, 64))),
        ("dst", lambda: gdn.state_copy(dims, ssm, i32(3), i32(2))),
    ]
    for name, call in cases:
        with pytest.raises(gdn.GdnError, match=rf"\b{name} has shape"):
            call()

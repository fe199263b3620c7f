"""Thin Python binding over libgdn.so (the C ABI declared in include/gdn.h).

Argument marshalling only: every function checks tensor dtypes, devices,
shapes and contiguity, allocates outputs with torch when the caller passes
none, and calls the C entry point of the same name on torch's current HIP
stream.  All arithmetic runs in the HIP kernels behind the ABI.  If the
library is not built, import succeeds but the first call raises GdnError:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_BF16, GDN_F32 = 0, 1
_STATUS = {0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_DTYPE", -4: "GDN_ERR_UNSUPPORTED",
           -5: "GDN_ERR_WORKSPACE", -6: "GDN_ERR_HIP", -7: "GDN_ERR_ALIGN", -8: "GDN_ERR_TOO_LARGE"}

# Names and signatures of every exported entry point (mirrors include/gdn.h).
_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "gdn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gdn_version": (ctypes.c_char_p, []),
    "gdn_conv1d_fwd": (ctypes.c_int, [_P, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P]),
    "gdn_conv1d_update": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _P, _P, _P, _P]),
    "gdn_gating": (ctypes.c_int, [_I32, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_chunk_prefill_workspace_size": (_SZ, [_P, _I32, _I32, _I64, _I32]),
    "gdn_chunk_prefill": (ctypes.c_int, [_P, _I32, _I32, _I64, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P,
                                         _P, _F, _P, _SZ, _P]),
    "gdn_prefill_workspace_size": (_SZ, [_P, _I32, _I32, _I64, _I32]),
    "gdn_prefill": (ctypes.c_int, [_P, _I32, _I32, _I64, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _I32, _P, _P, _P, _F, _P, _SZ, _P]),
    "gdn_recurrent_decode": (ctypes.c_int, [_P, _I32, _I32, _I32, _F, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P,
                                            _P, _F, _P]),
    "gdn_prefill_noalloc_limit": (_SZ, []),
    "gdn_prefill_noalloc": (ctypes.c_int, [_P, _I32, _I32, _I64, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _I32, _P, _P, _P, _F, _P]),
    "gdn_decode": (ctypes.c_int, [_P, _I32, _I32, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P,
                                  _P, _P, _F, _P]),
    "gdn_state_copy": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _P, _P, _I32, _P]),
    "gdn_check_slots": (ctypes.c_int, [_I32, _P, _I32, _P, _I32, _P, _P]),
    "gdn_rmsnorm_gemma": (ctypes.c_int, [_I32, _I64, _I32, _P, _P, _F, _P, _P]),
    "gdn_in_proj": (ctypes.c_int, [_P, _I32, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_out_proj": (ctypes.c_int, [_P, _I32, _I64, _I32, _P, _P, _P, _P, _P]),
}


class GdnError(RuntimeError):
    pass


class Dims(NamedTuple):
    h_k: int = 16
    h_v: int = 32
    d_k: int = 128
    d_v: int = 128
    conv_w: int = 4

    @property
    def c_ch(self) -> int:
        return 2 * self.h_k * self.d_k + self.h_v * self.d_v


class _CDims(ctypes.Structure):
    _fields_ = [("h_k", ctypes.c_int32), ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("conv_w", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def lib(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libgdn.so (once per process) and attach the ABI signatures.  path:
    another build of the library to load instead (the launch-shape tuner
    times variant builds this way); only before the first load."""
    global _lib
    if _lib is None:
        path = path or LIB_PATH
        if not os.path.exists(path):
            raise GdnError(f"{path} is not built: run gated_deltanet_conv1d_amd.build.build() first")
        handle = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            if path != LIB_PATH and not hasattr(handle, name):
                continue        # an older variant build: only the calls it has
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def version() -> str:
    return lib().gdn_version().decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib().gdn_status_string(rc).decode()
        raise GdnError(f"{what} failed: {msg} ({rc})")


def _cdims(d: Dims) -> ctypes.Structure:
    return _CDims(*d)


def _act(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise GdnError(f"activation dtype must be bfloat16 or float32, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise GdnError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise GdnError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise GdnError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _shape(t: torch.Tensor, shape, name: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise GdnError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _opt_shape(t: Optional[torch.Tensor], shape, name: str) -> None:
    """Shape check of an optional argument (a caller-provided output buffer,
    an optional input): the kernels size every access from the dimensions,
    so a smaller buffer would be written or read past its end."""
    if t is not None:
        _shape(t, shape, name)


# ------------------------------------------------------------------ calls
def conv1d_fwd(dims: Dims, x, w, cu_seqlens, slots, conv_state, has_init=None, bias=None, y=None):
    """Causal conv1d + SiLU over a packed varlen batch; updates conv_state in place."""
    act = _act(x)
    t_total, n_seq = x.shape[0], slots.shape[0]
    _shape(x, (t_total, dims.c_ch), "x")
    _shape(w, (dims.c_ch, dims.conv_w), "w")
    _shape(cu_seqlens, (n_seq + 1,), "cu_seqlens")
    _shape(conv_state, (conv_state.shape[0], dims.c_ch, dims.conv_w - 1), "conv_state")
    _opt_shape(has_init, (n_seq,), "has_init")
    _opt_shape(bias, (dims.c_ch,), "bias")
    _opt_shape(y, (t_total, dims.c_ch), "y")
    if y is None:
        y = torch.empty_like(x)
    _check(lib().gdn_conv1d_fwd(ctypes.byref(_cdims(dims)), act, n_seq, t_total, _ptr(x, x.dtype, "x"),
                                _ptr(w, x.dtype, "w"), _ptr(bias, x.dtype, "bias"),
                                _ptr(cu_seqlens, torch.int32, "cu_seqlens"), _ptr(slots, torch.int32, "slots"),
                                _ptr(has_init, torch.uint8, "has_init"), _ptr(conv_state, x.dtype, "conv_state"),
                                conv_state.shape[0], _ptr(y, x.dtype, "y"), _stream()), "gdn_conv1d_fwd")
    return y


def conv1d_update(dims: Dims, x, w, conv_state, slots, out_slots=None, bias=None, y=None):
    """Conv for decode / MTP rows [n_seq, t_step, c_ch]; updates the conv pool."""
    act = _act(x)
    n_seq, t_step = x.shape[0], x.shape[1]
    _shape(x, (n_seq, t_step, dims.c_ch), "x")
    _shape(w, (dims.c_ch, dims.conv_w), "w")
    _shape(conv_state, (conv_state.shape[0], dims.c_ch, dims.conv_w - 1), "conv_state")
    _shape(slots, (n_seq,), "slots")
    _opt_shape(out_slots, (n_seq, t_step), "out_slots")
    _opt_shape(bias, (dims.c_ch,), "bias")
    _opt_shape(y, (n_seq, t_step, dims.c_ch), "y")
    if y is None:
        y = torch.empty_like(x)
    _check(lib().gdn_conv1d_update(ctypes.byref(_cdims(dims)), act, n_seq, t_step, _ptr(x, x.dtype, "x"),
                                   _ptr(w, x.dtype, "w"), _ptr(bias, x.dtype, "bias"),
                                   _ptr(conv_state, x.dtype, "conv_state"), conv_state.shape[0],
                                   _ptr(slots, torch.int32, "slots"), _ptr(out_slots, torch.int32, "out_slots"),
                                   _ptr(y, x.dtype, "y"), _stream()), "gdn_conv1d_update")
    return y


def gating(a, b, A_log, dt_bias, g=None, beta=None):
    """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b); a, b [..., h_v]."""
    act = _act(a)
    h_v = a.shape[-1]
    n = a.numel() // h_v
    _shape(b, a.shape, "b")
    _shape(A_log, (h_v,), "A_log")
    _shape(dt_bias, (h_v,), "dt_bias")
    _opt_shape(g, a.shape, "g")
    _opt_shape(beta, a.shape, "beta")
    if g is None:
        g = torch.empty(a.shape, dtype=torch.float32, device=a.device)
    if beta is None:
        beta = torch.empty(a.shape, dtype=torch.float32, device=a.device)
    _check(lib().gdn_gating(act, n, h_v, _ptr(a, a.dtype, "a"), _ptr(b, a.dtype, "b"),
                            _ptr(A_log, torch.float32, "A_log"), _ptr(dt_bias, torch.float32, "dt_bias"),
                            _ptr(g, torch.float32, "g"), _ptr(beta, torch.float32, "beta"), _stream()),
           "gdn_gating")
    return g, beta


def chunk_prefill_workspace_size(dims: Dims, act: int, n_seq: int, t_total: int, chunk: int) -> int:
    return int(lib().gdn_chunk_prefill_workspace_size(ctypes.byref(_cdims(dims)), act, n_seq, t_total, chunk))


def chunk_prefill(dims: Dims, qkv, g, beta, cu_seqlens, slots, state, has_init=None, chunk: int = 64,
                  scale: float = 1.0, z=None, norm_w=None, norm_eps: float = 1e-6, o=None, workspace=None):
    """Chunked gated delta rule over a packed varlen batch; updates state in place."""
    act = _act(qkv)
    t_total, n_seq = qkv.shape[0], slots.shape[0]
    _shape(qkv, (t_total, dims.c_ch), "qkv")
    _shape(g, (t_total, dims.h_v), "g")
    _shape(beta, (t_total, dims.h_v), "beta")
    _shape(cu_seqlens, (n_seq + 1,), "cu_seqlens")
    _shape(state, (state.shape[0], dims.h_v, dims.d_v, dims.d_k), "state")
    _opt_shape(has_init, (n_seq,), "has_init")
    _opt_shape(z, (t_total, dims.h_v, dims.d_v), "z")
    _opt_shape(norm_w, (dims.d_v,), "norm_w")
    _opt_shape(o, (t_total, dims.h_v, dims.d_v), "o")
    if o is None:
        o = torch.empty((t_total, dims.h_v, dims.d_v), dtype=qkv.dtype, device=qkv.device)
    ws = chunk_prefill_workspace_size(dims, act, n_seq, t_total, chunk)
    if ws and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=qkv.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_chunk_prefill(ctypes.byref(_cdims(dims)), act, n_seq, t_total, chunk, scale,
                                   _ptr(qkv, qkv.dtype, "qkv"), _ptr(g, torch.float32, "g"),
                                   _ptr(beta, torch.float32, "beta"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
                                   _ptr(slots, torch.int32, "slots"), _ptr(has_init, torch.uint8, "has_init"),
                                   _ptr(state, torch.float32, "state"), state.shape[0], _ptr(o, qkv.dtype, "o"),
                                   _ptr(z, qkv.dtype, "z"), _ptr(norm_w, qkv.dtype, "norm_w"), norm_eps,
                                   _ptr(workspace, None, "workspace"), ws_bytes, _stream()), "gdn_chunk_prefill")
    return o


def prefill_workspace_size(dims: Dims, act: int, n_seq: int, t_total: int, chunk: int) -> int:
    return int(lib().gdn_prefill_workspace_size(ctypes.byref(_cdims(dims)), act, n_seq, t_total, chunk))


def prefill(dims: Dims, x, conv_w, a, b, A_log, dt_bias, cu_seqlens, slots, conv_state, state, has_init=None,
            chunk: int = 64, scale: float = 1.0, z=None, norm_w=None, norm_eps: float = 1e-6, conv_b=None, o=None,
            workspace=None):
    """The whole prefill path in one call (conv1d + SiLU, gating, chunked rule,
    epilogue), with the conv output and gates kept inside the chunk kernels.
    Updates conv_state and state in place; returns out."""
    act = _act(x)
    t_total, n_seq = x.shape[0], slots.shape[0]
    _shape(x, (t_total, dims.c_ch), "x")
    _shape(a, (t_total, dims.h_v), "a")
    _shape(b, (t_total, dims.h_v), "b")
    _shape(conv_w, (dims.c_ch, dims.conv_w), "conv_w")
    _shape(A_log, (dims.h_v,), "A_log")
    _shape(dt_bias, (dims.h_v,), "dt_bias")
    _shape(cu_seqlens, (n_seq + 1,), "cu_seqlens")
    _shape(conv_state, (conv_state.shape[0], dims.c_ch, dims.conv_w - 1), "conv_state")
    _shape(state, (state.shape[0], dims.h_v, dims.d_v, dims.d_k), "state")
    _opt_shape(has_init, (n_seq,), "has_init")
    _opt_shape(conv_b, (dims.c_ch,), "conv_b")
    _opt_shape(z, (t_total, dims.h_v, dims.d_v), "z")
    _opt_shape(norm_w, (dims.d_v,), "norm_w")
    _opt_shape(o, (t_total, dims.h_v, dims.d_v), "o")
    if o is None:
        o = torch.empty((t_total, dims.h_v, dims.d_v), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(prefill_workspace_size(dims, act, n_seq, t_total, chunk), 1), dtype=torch.uint8,
                                device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().gdn_prefill(ctypes.byref(_cdims(dims)), act, n_seq, t_total, chunk, scale, _ptr(x, x.dtype, "x"),
                             _ptr(conv_w, x.dtype, "conv_w"), _ptr(conv_b, x.dtype, "conv_b"), _ptr(a, x.dtype, "a"),
                             _ptr(b, x.dtype, "b"), _ptr(A_log, torch.float32, "A_log"),
                             _ptr(dt_bias, torch.float32, "dt_bias"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
                             _ptr(slots, torch.int32, "slots"), _ptr(has_init, torch.uint8, "has_init"),
                             _ptr(conv_state, x.dtype, "conv_state"), _ptr(state, torch.float32, "state"),
                             state.shape[0], _ptr(o, x.dtype, "o"), _ptr(z, x.dtype, "z"),
                             _ptr(norm_w, x.dtype, "norm_w"), norm_eps, _ptr(workspace, None, "workspace"), ws_bytes,
                             _stream()), "gdn_prefill")
    return o


def recurrent_decode(dims: Dims, qkv, a, b, A_log, dt_bias, state, slots, out_slots=None, scale: float = 1.0,
                     z=None, norm_w=None, norm_eps: float = 1e-6, o=None):
    """Fused recurrent step over request-major rows [n_seq, t_step, ...]."""
    act = _act(qkv)
    n_seq, t_step = qkv.shape[0], qkv.shape[1]
    _shape(qkv, (n_seq, t_step, dims.c_ch), "qkv")
    _shape(a, (n_seq, t_step, dims.h_v), "a")
    _shape(b, (n_seq, t_step, dims.h_v), "b")
    _shape(A_log, (dims.h_v,), "A_log")
    _shape(dt_bias, (dims.h_v,), "dt_bias")
    _shape(state, (state.shape[0], dims.h_v, dims.d_v, dims.d_k), "state")
    _shape(slots, (n_seq,), "slots")
    _opt_shape(out_slots, (n_seq, t_step), "out_slots")
    _opt_shape(z, (n_seq, t_step, dims.h_v, dims.d_v), "z")
    _opt_shape(norm_w, (dims.d_v,), "norm_w")
    _opt_shape(o, (n_seq, t_step, dims.h_v, dims.d_v), "o")
    if o is None:
        o = torch.empty((n_seq, t_step, dims.h_v, dims.d_v), dtype=qkv.dtype, device=qkv.device)
    _check(lib().gdn_recurrent_decode(ctypes.byref(_cdims(dims)), act, n_seq, t_step, scale,
                                      _ptr(qkv, qkv.dtype, "qkv"), _ptr(a, qkv.dtype, "a"), _ptr(b, qkv.dtype, "b"),
                                      _ptr(A_log, torch.float32, "A_log"), _ptr(dt_bias, torch.float32, "dt_bias"),
                                      _ptr(state, torch.float32, "state"), state.shape[0],
                                      _ptr(slots, torch.int32, "slots"), _ptr(out_slots, torch.int32, "out_slots"),
                                      _ptr(o, qkv.dtype, "o"), _ptr(z, qkv.dtype, "z"),
                                      _ptr(norm_w, qkv.dtype, "norm_w"), norm_eps, _stream()),
           "gdn_recurrent_decode")
    return o


def decode(dims: Dims, x, conv_w, a, b, A_log, dt_bias, slots, conv_state, state, out_slots=None,
           scale: float = 1.0, z=None, norm_w=None, norm_eps: float = 1e-6, conv_b=None, o=None):
    """The whole decode / MTP step in one call (gdn_decode): conv window update,
    gating, the recurrent step and the epilogue over request-major rows
    [n_seq, t_step, ...].  Returns out [n_seq, t_step, h_v, d_v]."""
    act = _act(x)
    n_seq, t_step = x.shape[0], x.shape[1]
    _shape(x, (n_seq, t_step, dims.c_ch), "x")
    _shape(conv_w, (dims.c_ch, dims.conv_w), "conv_w")
    _shape(a, (n_seq, t_step, dims.h_v), "a")
    _shape(b, (n_seq, t_step, dims.h_v), "b")
    _shape(slots, (n_seq,), "slots")
    _shape(A_log, (dims.h_v,), "A_log")
    _shape(dt_bias, (dims.h_v,), "dt_bias")
    _shape(conv_state, (conv_state.shape[0], dims.c_ch, dims.conv_w - 1), "conv_state")
    _shape(state, (state.shape[0], dims.h_v, dims.d_v, dims.d_k), "state")
    _opt_shape(out_slots, (n_seq, t_step), "out_slots")
    _opt_shape(conv_b, (dims.c_ch,), "conv_b")
    _opt_shape(z, (n_seq, t_step, dims.h_v, dims.d_v), "z")
    _opt_shape(norm_w, (dims.d_v,), "norm_w")
    _opt_shape(o, (n_seq, t_step, dims.h_v, dims.d_v), "o")
    if o is None:
        o = torch.empty((n_seq, t_step, dims.h_v, dims.d_v), dtype=x.dtype, device=x.device)
    _check(lib().gdn_decode(ctypes.byref(_cdims(dims)), act, n_seq, t_step, scale, _ptr(x, x.dtype, "x"),
                            _ptr(conv_w, x.dtype, "conv_w"), _ptr(conv_b, x.dtype, "conv_b"), _ptr(a, x.dtype, "a"),
                            _ptr(b, x.dtype, "b"), _ptr(A_log, torch.float32, "A_log"),
                            _ptr(dt_bias, torch.float32, "dt_bias"), _ptr(conv_state, x.dtype, "conv_state"),
                            _ptr(state, torch.float32, "state"), state.shape[0], _ptr(slots, torch.int32, "slots"),
                            _ptr(out_slots, torch.int32, "out_slots"), _ptr(o, x.dtype, "o"), _ptr(z, x.dtype, "z"),
                            _ptr(norm_w, x.dtype, "norm_w"), norm_eps, _stream()), "gdn_decode")
    return o


def state_copy(dims: Dims, state, src, dst, conv_state=None):
    """Bitwise state[dst[i]] <- state[src[i]] (and the conv pool, when given)."""
    act = GDN_BF16 if conv_state is None else _act(conv_state)
    _shape(state, (state.shape[0], dims.h_v, dims.d_v, dims.d_k), "state")
    _shape(dst, tuple(src.shape), "dst")
    _opt_shape(conv_state, (state.shape[0], dims.c_ch, dims.conv_w - 1), "conv_state")
    _check(lib().gdn_state_copy(ctypes.byref(_cdims(dims)), act, _ptr(state, torch.float32, "state"),
                                _ptr(conv_state, None, "conv_state"), state.shape[0], _ptr(src, torch.int32, "src"),
                                _ptr(dst, torch.int32, "dst"), src.shape[0], _stream()), "gdn_state_copy")


def check_slots(n_slots: int, slots, out_slots=None) -> torch.Tensor:
    """Device check of slot tables (gdn_check_slots): int32 flags over
    slots.ravel() ++ out_slots.ravel(), 1 = padding other than -1,
    2 = an in-range slot equal to an earlier entry; all zero means valid."""
    s = slots.reshape(-1)
    o = None if out_slots is None else out_slots.reshape(-1)
    n, n_out = s.numel(), 0 if o is None else o.numel()
    flags = torch.empty(n + n_out, dtype=torch.int32, device=slots.device)
    _check(lib().gdn_check_slots(n_slots, _ptr(s, torch.int32, "slots"), n,
                                 _ptr(o, torch.int32, "out_slots") if n_out else None, n_out,
                                 _ptr(flags, torch.int32, "flags"), _stream()), "gdn_check_slots")
    return flags


def rmsnorm_gemma(x, w, eps: float = 1e-6, out=None):
    """Gemma-form RMSNorm over the last axis (gdn_rmsnorm_gemma): x / rms(x) * (1 + w)."""
    hidden = x.shape[-1]
    _shape(w, (hidden,), "w")
    _opt_shape(out, x.shape, "out")
    if out is None:
        out = torch.empty_like(x)
    _check(lib().gdn_rmsnorm_gemma(_act(x), x.numel() // hidden if hidden else 0, hidden, _ptr(x, x.dtype, "x"),
                                   _ptr(w, x.dtype, "w"), eps, _ptr(out, x.dtype, "out"), _stream()),
           "gdn_rmsnorm_gemma")
    return out


def in_proj(dims: Dims, xn, w_qkvz, w_ba, qkv=None, z=None, b=None, a=None):
    """The input projections (gdn_in_proj).  xn [T, hidden] bf16.  Returns
    (qkv [T, c_ch], z [T, h_v, d_v], b [T, h_v], a [T, h_v])."""
    T, hidden = xn.shape
    vd = dims.h_v * dims.d_v
    _shape(w_qkvz, (dims.c_ch + vd, hidden), "w_qkvz")
    _shape(w_ba, (2 * dims.h_v, hidden), "w_ba")
    _opt_shape(qkv, (T, dims.c_ch), "qkv")
    _opt_shape(z, (T, dims.h_v, dims.d_v), "z")
    _opt_shape(b, (T, dims.h_v), "b")
    _opt_shape(a, (T, dims.h_v), "a")
    mk = lambda *shape: torch.empty(shape, dtype=xn.dtype, device=xn.device)
    qkv = mk(T, dims.c_ch) if qkv is None else qkv
    z = mk(T, dims.h_v, dims.d_v) if z is None else z
    b = mk(T, dims.h_v) if b is None else b
    a = mk(T, dims.h_v) if a is None else a
    _check(lib().gdn_in_proj(ctypes.byref(_cdims(dims)), _act(xn), T, hidden, _ptr(xn, xn.dtype, "xn"),
                             _ptr(w_qkvz, xn.dtype, "w_qkvz"), _ptr(w_ba, xn.dtype, "w_ba"),
                             _ptr(qkv, xn.dtype, "qkv"), _ptr(z, xn.dtype, "z"), _ptr(b, xn.dtype, "b"),
                             _ptr(a, xn.dtype, "a"), _stream()), "gdn_in_proj")
    return qkv, z, b, a


def out_proj(dims: Dims, o, w_out, residual=None, y=None):
    """y = o w_out^T (+ residual) (gdn_out_proj).  o [T, h_v * d_v] (or
    [T, h_v, d_v]) bf16; returns y [T, hidden]."""
    T = o.shape[0]
    hidden = w_out.shape[0]
    _shape(w_out, (hidden, dims.h_v * dims.d_v), "w_out")
    if o.numel() != T * dims.h_v * dims.d_v:
        raise GdnError(f"o: expected {T} x {dims.h_v * dims.d_v} values, got shape {tuple(o.shape)}")
    _opt_shape(residual, (T, hidden), "residual")
    _opt_shape(y, (T, hidden), "y")
    if y is None:
        y = torch.empty((T, hidden), dtype=o.dtype, device=o.device)
    _check(lib().gdn_out_proj(ctypes.byref(_cdims(dims)), _act(o), T, hidden, _ptr(o, o.dtype, "o"),
                              _ptr(w_out, o.dtype, "w_out"), _ptr(residual, o.dtype, "residual"),
                              _ptr(y, o.dtype, "y"), _stream()), "gdn_out_proj")
    return y


# ------------------------------------------------------- layer sequences
def prefill_layer(dims: Dims, x, conv_w, A_log, dt_bias, a, b, cu_seqlens, slots, conv_state, state, has_init=None,
                  chunk: int = 64, scale: float = 1.0, z=None, norm_w=None, norm_eps: float = 1e-6, conv_b=None):
    """The prefill hot path as the pages order it: conv1d + SiLU, gating, then
    the chunked gated delta rule with fused q/k L2 norm and gated RMSNorm.
    Returns (out, y, g, beta)."""
    y = conv1d_fwd(dims, x, conv_w, cu_seqlens, slots, conv_state, has_init, conv_b)
    g, beta = gating(a, b, A_log, dt_bias)
    out = chunk_prefill(dims, y, g, beta, cu_seqlens, slots, state, has_init, chunk, scale, z, norm_w, norm_eps)
    return out, y, g, beta


def decode_layer(dims: Dims, x, conv_w, A_log, dt_bias, a, b, slots, conv_state, state, out_slots=None,
                 scale: float = 1.0, z=None, norm_w=None, norm_eps: float = 1e-6, conv_b=None):
    """The decode / MTP hot path: conv update, then the fused recurrent step.
    Returns (out, y)."""
    y = conv1d_update(dims, x, conv_w, conv_state, slots, out_slots, conv_b)
    out = recurrent_decode(dims, y, a, b, A_log, dt_bias, state, slots, out_slots, scale, z, norm_w, norm_eps)
    return out, y


class BlockWeights(NamedTuple):
    """Weights of the layer around the core (device tensors, bf16)."""
    norm_w: torch.Tensor   # [hidden] Gemma RMSNorm weight (the norm multiplies by 1 + w)
    w_qkvz: torch.Tensor   # [c_ch + h_v d_v, hidden]
    w_ba: torch.Tensor     # [2 h_v, hidden]
    w_out: torch.Tensor    # [hidden, h_v d_v]


def block_prefill(dims: Dims, X, wts: BlockWeights, conv_w, A_log, dt_bias, cu_seqlens, slots, conv_state, state,
                  has_init=None, chunk: int = 64, scale: float = 1.0, norm_w=None, norm_eps: float = 1e-6,
                  block_eps: float = 1e-6, residual: bool = True, conv_b=None, workspace=None,
                  intermediates: bool = False):
    """The whole layer over a packed varlen batch X [T, hidden]: Gemma RMSNorm,
    the input projections, the single-call prefill and out_proj (+ X).  Four
    ABI calls; returns y [T, hidden], and with intermediates also a dict of
    the activations handed between them (xn, qkv, z, b, a, o)."""
    xn = rmsnorm_gemma(X, wts.norm_w, block_eps)
    qkv, z, b, a = in_proj(dims, xn, wts.w_qkvz, wts.w_ba)
    o = prefill(dims, qkv, conv_w, a, b, A_log, dt_bias, cu_seqlens, slots, conv_state, state, has_init, chunk,
                scale, z, norm_w, norm_eps, conv_b=conv_b, workspace=workspace)
    y = out_proj(dims, o, wts.w_out, X if residual else None)
    return (y, dict(xn=xn, qkv=qkv, z=z, b=b, a=a, o=o)) if intermediates else y


def block_decode(dims: Dims, X, wts: BlockWeights, conv_w, A_log, dt_bias, slots, conv_state, state,
                 out_slots=None, scale: float = 1.0, norm_w=None, norm_eps: float = 1e-6, block_eps: float = 1e-6,
                 residual: bool = True, conv_b=None, intermediates: bool = False):
    """The whole layer for a decode / MTP step, X [n_seq, t_step, hidden]
    request-major: Gemma RMSNorm, the input projections, the single-call
    decode and out_proj (+ X).  Returns y [n_seq, t_step, hidden] (and the
    intermediates, as block_prefill)."""
    n_seq, t_step, hidden = X.shape
    X2 = X.reshape(n_seq * t_step, hidden)
    xn = rmsnorm_gemma(X2, wts.norm_w, block_eps)
    qkv, z, b, a = in_proj(dims, xn, wts.w_qkvz, wts.w_ba)
    o = decode(dims, qkv.view(n_seq, t_step, dims.c_ch), conv_w, a.view(n_seq, t_step, dims.h_v),
               b.view(n_seq, t_step, dims.h_v), A_log, dt_bias, slots, conv_state, state, out_slots, scale,
               z.view(n_seq, t_step, dims.h_v, dims.d_v), norm_w, norm_eps, conv_b)
    y = out_proj(dims, o.view(n_seq * t_step, dims.h_v * dims.d_v), wts.w_out,
                 X2 if residual else None).view(n_seq, t_step, hidden)
    return (y, dict(xn=xn, qkv=qkv, z=z, b=b, a=a, o=o)) if intermediates else y

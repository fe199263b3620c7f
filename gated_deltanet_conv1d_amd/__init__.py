"""Gated DeltaNet (GDN) layer hot path for MI355X (gfx950).

The computation lives in libgdn.so (hand-written HIP kernels behind the C ABI
of include/gdn.h); this package only builds it and binds it.
"""
from .binding import (Dims, GdnError, chunk_prefill, chunk_prefill_workspace_size, conv1d_fwd,  # noqa: F401
                      conv1d_update, decode, decode_layer, gating, lib, prefill, prefill_layer, prefill_workspace_size,
                      recurrent_decode, state_copy, version)

"""Gated DeltaNet (GDN) layer hot path for MI355X (gfx950).

The computation lives in libgdn.so (hand-written HIP kernels behind the C ABI
of include/gdn.h); this package only builds it and binds it.
"""
from .binding import (BlockWeights, Dims, GdnError, block_decode, block_prefill, check_slots, chunk_prefill,  # noqa: F401
                      chunk_prefill_workspace_size, conv1d_fwd, conv1d_update, decode, decode_layer, gating,
                      in_proj, lib, out_proj, prefill, prefill_layer, prefill_workspace_size, recurrent_decode,
                      rmsnorm_gemma, state_copy, version)

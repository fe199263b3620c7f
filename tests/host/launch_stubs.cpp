// Host-only stand-ins for the kernel launchers of libgdn, so that the C ABI's
// validation and argument marshalling (gdn_api.cpp) can be built and run on
// the CPU under the address and undefined-behaviour sanitizers.  Each stub
// records which launcher ran and a copy of its argument block; nothing here
// touches a device.
#include "launch_stubs.hpp"

namespace stub {
Record last;
hipError_t next_result = hipSuccess;
}  // namespace stub

namespace gdn {

#define GDN_STUB(fn, Args, field)                           \
  hipError_t fn(const Args& a, hipStream_t) {               \
    stub::last = stub::Record{};                            \
    stub::last.which = #fn;                                 \
    stub::last.field = a;                                   \
    return stub::next_result;                               \
  }
GDN_STUB(launch_conv1d_fwd, ConvFwdArgs, conv_fwd)
GDN_STUB(launch_conv1d_update, ConvUpdateArgs, conv_update)
GDN_STUB(launch_gating, GatingArgs, gating)
GDN_STUB(launch_state_copy, StateCopyArgs, state_copy)
GDN_STUB(launch_recurrent, RecurrentArgs, recurrent)
GDN_STUB(launch_decode, DecodeArgs, decode)
GDN_STUB(launch_chunk_split, ChunkArgs, chunk)
GDN_STUB(launch_prefill_fused, ChunkArgs, chunk)
GDN_STUB(launch_gemma_norm, GemmaNormArgs, norm)
GDN_STUB(launch_proj, ProjArgs, proj)
GDN_STUB(launch_slot_check, SlotCheckArgs, slot_check)
#undef GDN_STUB

bool decode_supported(const Shape& s) { return s.h_v == s.h_k || s.h_v == 2 * s.h_k; }

bool chunk_supported(int d, int chunk, bool) {
  return (d == 16 || d == 32 || d == 64 || d == 128) && (chunk == 16 || chunk == 32 || chunk == 64);
}

// a size that grows with the batch, as the real one does (its value is the
// library's business; the API only compares it with the caller's bytes)
size_t chunk_split_workspace_size(const Shape& s, bool bf16, int32_t n_seq, int64_t t_total, int32_t chunk) {
  if (!chunk_supported(s.d, chunk, bf16)) return 0;
  return (size_t)(t_total / chunk + n_seq) * (size_t)s.h_v * 99840u;
}

}  // namespace gdn

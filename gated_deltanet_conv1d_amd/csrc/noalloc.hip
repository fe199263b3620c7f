// gdn_prefill_noalloc: gdn_prefill for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The split path's workspace is a file-scope device array
// in this translation unit instead of a caller buffer.  Each device holds its
// own copy of the array (loaded with this code object, kept until the process
// ends); its address is taken once per device with hipGetSymbolAddress, and
// only that address -- never the array's host-side name -- reaches a kernel.
//
// Nothing in the workspace needs to start at zero: the chunk index is written
// by its own kernel before any read, and every unit a later pass reads is
// written first by the pass before it.  Calls that overlap on one device share
// the array and race; callers serialise them (one stream, or events).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)256 << 20;  // 256 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, or nullptr on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t gdn_prefill_noalloc_limit(void) { return kScratchBytes; }

int gdn_prefill_noalloc(const gdn_dims* dims, int32_t act, int32_t n_seq, int64_t t_total, int32_t chunk,
                        float scale, const void* x, const void* conv_w, const void* conv_b, const void* a,
                        const void* b, const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                        const int32_t* slots, const uint8_t* has_init, void* conv_state, float* state,
                        int32_t n_slots, void* o, const void* z, const void* norm_w, float norm_eps, void* stream) {
  if (gdn_prefill_workspace_size(dims, act, n_seq, t_total, chunk) > kScratchBytes) return GDN_ERR_TOO_LARGE;
  void* ws = scratch_ptr();
  if (!ws) return GDN_ERR_HIP;
  return gdn_prefill(dims, act, n_seq, t_total, chunk, scale, x, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens,
                     slots, has_init, conv_state, state, n_slots, o, z, norm_w, norm_eps, ws, kScratchBytes, stream);
}

}  // extern "C"

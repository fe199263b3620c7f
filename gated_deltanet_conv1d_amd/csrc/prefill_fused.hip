// The fused-input prefill on the split path: the prep and output kernels
// compute q, k, v as conv1d + SiLU of x in the chunk they work on (a W-1 row
// halo, the slot's conv state before a sequence start), and g, beta from a, b,
// so neither the conv output y nor g, beta ever reach HBM.  The chain kernel
// writes the final conv windows: the prep pass, which reads the old ones, is
// done by then, and it keeps the old q window of every sequence's first
// chunk in the workspace for the output pass.
// The conv1d arithmetic, the gate formulas and everything downstream match
// the separate gdn_conv1d_fwd + gdn_gating + gdn_chunk_prefill calls.
#include "chunk_split_kernels.hpp"

namespace gdn {
namespace {

template <typename T, int D, int W>
hipError_t by_chunk(const ChunkArgs& a, hipStream_t st) {
  switch (a.chunk) {
    case 16: return split::run<T, T, D, 16, true, W>(a, st);
    case 32: return split::run<T, T, D, 32, true, W>(a, st);
    case 64: return split::run<T, T, D, 64, true, W>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t by_width(const ChunkArgs& a, hipStream_t st) {
  switch (a.s.conv_w) {
    case 2: return by_chunk<T, D, 2>(a, st);
    case 3: return by_chunk<T, D, 3>(a, st);
    case 4: return by_chunk<T, D, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_fused(const ChunkArgs& a, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  switch (a.s.d) {
    case 16: e = a.bf16 ? by_width<bf16, 16>(a, st) : by_width<float, 16>(a, st); break;
    case 32: e = a.bf16 ? by_width<bf16, 32>(a, st) : by_width<float, 32>(a, st); break;
    case 64: e = a.bf16 ? by_width<bf16, 64>(a, st) : by_width<float, 64>(a, st); break;
    case 128: e = a.bf16 ? by_width<bf16, 128>(a, st) : by_width<float, 128>(a, st); break;
  }
  return e;
}

}  // namespace gdn

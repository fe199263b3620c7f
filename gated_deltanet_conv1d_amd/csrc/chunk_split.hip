// Launchers of the split chunked prefill (kernels in chunk_split_kernels.hpp):
// q, k, v from the conv1d output y and g, beta from the gating pass.
#include "chunk_split_kernels.hpp"

namespace gdn {
namespace split {

template <typename T, typename Op, int D>
hipError_t by_chunk(const ChunkArgs& a, hipStream_t st) {
  switch (a.chunk) {
    case 16: return run<T, Op, D, 16>(a, st);
    case 32: return run<T, Op, D, 32>(a, st);
    case 64: return run<T, Op, D, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename Op, int D>
size_t ws_by_chunk(int chunk, int32_t n_seq, int64_t t_total, int32_t h_v) {
  switch (chunk) {
    case 16: return ws_bytes<T, Op, D, 16>(n_seq, t_total, h_v);
    case 32: return ws_bytes<T, Op, D, 32>(n_seq, t_total, h_v);
    case 64: return ws_bytes<T, Op, D, 64>(n_seq, t_total, h_v);
  }
  return 0;
}

}  // namespace split

bool chunk_supported(int d, int chunk, bool) {
  return (d == 16 || d == 32 || d == 64 || d == 128) && (chunk == 16 || chunk == 32 || chunk == 64);
}

size_t chunk_split_workspace_size(const Shape& s, bool is_bf16, int32_t n_seq, int64_t t_total, int32_t chunk) {
  switch (s.d) {
    case 16: return is_bf16 ? split::ws_by_chunk<bf16, bf16, 16>(chunk, n_seq, t_total, s.h_v)
                         : split::ws_by_chunk<float, float, 16>(chunk, n_seq, t_total, s.h_v);
    case 32: return is_bf16 ? split::ws_by_chunk<bf16, bf16, 32>(chunk, n_seq, t_total, s.h_v)
                         : split::ws_by_chunk<float, float, 32>(chunk, n_seq, t_total, s.h_v);
    case 64: return is_bf16 ? split::ws_by_chunk<bf16, bf16, 64>(chunk, n_seq, t_total, s.h_v)
                         : split::ws_by_chunk<float, float, 64>(chunk, n_seq, t_total, s.h_v);
    case 128: return is_bf16 ? split::ws_by_chunk<bf16, bf16, 128>(chunk, n_seq, t_total, s.h_v)
                          : split::ws_by_chunk<float, float, 128>(chunk, n_seq, t_total, s.h_v);
  }
  return 0;
}

hipError_t launch_chunk_split(const ChunkArgs& a, hipStream_t st) {
  switch (a.s.d) {
    case 16: return a.bf16 ? split::by_chunk<bf16, bf16, 16>(a, st) : split::by_chunk<float, float, 16>(a, st);
    case 32: return a.bf16 ? split::by_chunk<bf16, bf16, 32>(a, st) : split::by_chunk<float, float, 32>(a, st);
    case 64: return a.bf16 ? split::by_chunk<bf16, bf16, 64>(a, st) : split::by_chunk<float, float, 64>(a, st);
    case 128: return a.bf16 ? split::by_chunk<bf16, bf16, 128>(a, st) : split::by_chunk<float, float, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

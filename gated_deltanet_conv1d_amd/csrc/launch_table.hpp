// Launch shapes of the chunked prefill's chain pass, by workload: written by
// gated_deltanet_conv1d_amd/tune.py from timings of every candidate shape on
// one MI355X (the table below is that script's output; rerun it to retune).
//
// A row applies to a call whose number of (sequence, V head) chains is at most
// max_chains and whose mean sequence length is at most max_len (the first
// matching row wins).  ntw: 16-wide d_v tiles per chain workgroup (they share
// each -W and K^T load), 8 = all of d_v in one workgroup, which then also
// computes the output (no output pass); pd: register stages of the
// chunk-operand prefetch.  The states do not depend on the shape (every
// accumulator sees the same MFMA order); the outputs of the whole-d_v chain
// can differ from the output pass's in the last bit (its products and norm
// sum run in another order).
#pragma once
#include <stdint.h>

namespace gdn {

struct ChainShape {
  int64_t max_chains;  // sequences x V heads
  int64_t max_len;     // mean tokens per sequence
  int ntw, pd;
};

constexpr ChainShape kChainTable[] = {
    {32, INT64_MAX, 1, 3},
    {64, INT64_MAX, 2, 3},
    {128, INT64_MAX, 4, 2},
    {INT64_MAX, INT64_MAX, 8, 2},
};

// The (ntw, pd) pairs the table uses, each instantiated once per kernel type.
#define GDN_CHAIN_SHAPES(X) X(1, 3) X(2, 3) X(4, 2) X(8, 2)

inline ChainShape chain_shape(int64_t chains, int64_t mean_len) {
  for (const ChainShape& s : kChainTable)
    if (chains <= s.max_chains && mean_len <= s.max_len) return s;
  return kChainTable[sizeof(kChainTable) / sizeof(kChainTable[0]) - 1];
}

}  // namespace gdn

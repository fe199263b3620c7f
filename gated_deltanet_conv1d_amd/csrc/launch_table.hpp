// Launch shapes of the chunked prefill's chain pass, by workload: written by
// gated_deltanet_conv1d_amd/tune.py from timings of every candidate shape on
// one MI355X (the table below is that script's output; rerun it to retune).
//
// A row applies to a call whose number of (sequence, V head) chains is at most
// max_chains and whose mean sequence length is at most max_len (the first
// matching row wins).  ntw: 16-wide d_v tiles per chain workgroup (they share
// each -W and K^T load); pd: register stages of the chunk-operand prefetch.
// Results do not depend on the shape: every accumulator sees the same MFMA
// order.
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
    {256, INT64_MAX, 4, 2},
    {512, INT64_MAX, 4, 3},
    {INT64_MAX, INT64_MAX, 4, 2},
};

// The (ntw, pd) pairs the table uses, each instantiated once per kernel type.
#define GDN_CHAIN_SHAPES(X) X(1, 3) X(2, 3) X(4, 2) X(4, 3)

inline ChainShape chain_shape(int64_t chains, int64_t mean_len) {
  for (const ChainShape& s : kChainTable)
    if (chains <= s.max_chains && mean_len <= s.max_len) return s;
  return kChainTable[sizeof(kChainTable) / sizeof(kChainTable[0]) - 1];
}

}  // namespace gdn

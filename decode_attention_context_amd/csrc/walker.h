// walker.h — ownership and block-table walk of a DCP shard (host and device).
//
// Token t of a sequence is stored by DCP rank (t / I) mod C, where I is the KV-cache
// interleave size and C the DCP size ("Context Parallel Guide", vLLM Ascend docs,
// "Usage -> Decode Context Parallel": --cp-kv-cache-interleave-size; blog "vLLM Decode
// Context Parallelism for long-context workloads", "How DCP works").  A rank's tokens,
// in ascending t, are numbered by a local index j: local chunk c = j / I is global chunk
// c * C + rank, so
//     t(j) = (j / I) * I * C + rank * I + j % I,
// and the rank holds  (L / (I C)) * I + clamp(L mod (I C) - rank * I, 0, I)  tokens of an
// L-token sequence.  Token t sits in cache page block_table[t / B], slot t % B.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DCP_HD __host__ __device__ __forceinline__
#else
#define DCP_HD inline
#endif

// Tokens of an L-token sequence stored by `rank` (L >= 0, I >= 1, 0 <= rank < C).
DCP_HD int64_t dcp_walk_local_count(int64_t L, int rank, int C, int I) {
  if (L <= 0) return 0;
  const int64_t ic = (int64_t)I * C;
  const int64_t full = L / ic;
  int64_t extra = L - full * ic - (int64_t)rank * I;
  extra = extra < 0 ? 0 : (extra > I ? I : extra);
  return full * I + extra;
}

// The same count in 32-bit arithmetic, for L and I * C below 2^31 (the library's bounds on
// sequence lengths and on I * C): one 32-bit division instead of a 64-bit one.
DCP_HD uint32_t dcp_walk_local_count32(uint32_t L, uint32_t rank, uint32_t C, uint32_t I) {
  const uint32_t ic = I * C;
  const uint32_t full = L / ic;
  const uint32_t rest = L - full * ic;   // < I * C
  const uint32_t lo = rank * I;
  const uint32_t extra = rest <= lo ? 0u : (rest - lo > I ? I : rest - lo);
  return full * I + extra;
}

// Global position of local token j of `rank` (32-bit: positions are below 2^31).
DCP_HD uint32_t dcp_walk_global_pos(uint32_t j, uint32_t rank, uint32_t C, uint32_t I) {
  const uint32_t c = j / I;
  return c * I * C + rank * I + (j - c * I);
}

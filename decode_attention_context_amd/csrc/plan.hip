// plan.hip — work planning of a shard call and the exported block-table walk.
//
// A shard call's work is split into items: contiguous ranges of a request's local tokens
// (the tokens its rank owns, in ascending position).  The planner runs as one wave:
//   1. local_b = tokens of request b on this rank (the walker's closed form); seq_len is
//      clamped to the block table's capacity (error bit DCP_DEVERR_SEQ_LEN otherwise);
//   2. chunk = the item size: total local tokens / target item count, rounded up to the
//      kernel's tile and clamped to [min_chunk, the longest request];
//   3. n_b = ceil(local_b / chunk) items per request; off = exclusive prefix sum;
//   4. item i of request b = (b, i * chunk, min((i + 1) * chunk, local_b), off_b + i), the
//      last field being the index of its partial output;
//   5. the items are stored in dispatch order, by descending tile count: the full-size
//      items of every request first (by request), then the shorter last items of the
//      requests by a counting sort over kBuckets buckets (longer ones sharing the top
//      bucket): workgroup slot k runs items[k].
// Since chunk >= total / target, the item count never exceeds target + batch, which is the
// bound the host sizes the workspace with.  A request's partials keep consecutive indices
// (the split combine reads them together); only the dispatch order changes.  Greedy
// dispatch of the longest items first keeps a ragged batch's long requests from starting
// in the last round: for 512 lognormal lengths around 67k tokens on 8 ranks it takes the
// simulated makespan from 1.54x to 1.04x the even share of one round.  The order of the
// shorter items within a bucket depends on atomics; no result does (each partial has its
// fixed index).
#include "launch.h"

namespace dcp {

namespace {

constexpr int kBuckets = 1024;   // tile-count buckets of the dispatch order
constexpr int kBucketsPerLane = kBuckets / 64;

// Inclusive scan across the 64 lanes of the wave (shuffles, no LDS).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// One wave plans the call: every reduction and scan is a shuffle, so no workgroup barrier
// is needed (the bucket histogram lives in LDS, written and read by this wave only).
__global__ __launch_bounds__(64) void plan_kernel(
    const int32_t* __restrict__ seq_lens, int batch, int rank, int cp, int interleave,
    int64_t len_cap, int64_t target, int tile, int min_chunk, int32_t* __restrict__ header,
    int32_t* __restrict__ off, int4* __restrict__ items) {
  __shared__ int s_hist[kBuckets];   // tail items per bucket, then next free position
  const int lane = threadIdx.x;
  const int per = (batch + 63) / 64;
  const int b0 = min(lane * per, batch);
  const int b1 = min(b0 + per, batch);
#pragma unroll
  for (int k = 0; k < kBucketsPerLane; ++k) s_hist[lane * kBucketsPerLane + k] = 0;

  // per-request arithmetic in 32 bits: lengths are clamped to len_cap and the host bounds
  // len_cap and interleave * cp below 2^31, so every local count, item size and item
  // boundary fits (64-bit divisions are long software sequences on the GPU)
  auto local_of = [&](int b, int& err) -> uint32_t {
    long long L = seq_lens[b];
    if (L < 0) { err |= kErrSeqLen; L = 0; }
    if (L > len_cap) { err |= kErrSeqLen; L = len_cap; }
    return dcp_walk_local_count32((uint32_t)L, (uint32_t)rank, (uint32_t)cp,
                                  (uint32_t)interleave);
  };

  // 1. total and longest local length, error bits
  long long sum = 0, mx = 0;
  int err = 0;
  for (int b = b0; b < b1; ++b) {
    const long long loc = local_of(b, err);
    sum += loc;
    mx = loc > mx ? loc : mx;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sum += __shfl_xor(sum, o, 64);
    const long long m2 = __shfl_xor(mx, o, 64);
    mx = m2 > mx ? m2 : mx;
    err |= __shfl_xor(err, o, 64);
  }

  // 2. item size (the call's one 64-bit division; the result is at most the longest
  // request rounded up to the tile)
  long long chunk64 = (sum + target - 1) / target;
  chunk64 = (chunk64 + tile - 1) / tile * tile;
  if (chunk64 < min_chunk) chunk64 = min_chunk;
  const long long cap = (mx + tile - 1) / tile * tile;
  if (chunk64 > cap) chunk64 = cap;
  if (chunk64 < tile) chunk64 = tile;
  const uint32_t chunk = (uint32_t)chunk64;
  const uint32_t utile = (uint32_t)tile;

  // 3. request b has n = ceil(loc / chunk) items: nf = loc / chunk full items of exactly
  // chunk tokens (all in the top bucket: no item is longer) and, when loc mod chunk != 0, a
  // tail item.  One scan of the packed pair (n, nf) gives the partial indices (off) and the
  // dispatch positions of the full items, which go first, by request; the tails follow,
  // ordered by bucket (one LDS atomic per request with a tail).  Item counts are at most
  // target + batch, so 32 bits hold them.
  auto items_of = [&](uint32_t loc) -> int { return (int)(loc / chunk + (loc % chunk != 0)); };
  auto bucket = [&](uint32_t len) -> int {   // kBuckets - 1 - (tile count, capped)
    const uint32_t nt = len / utile + (len % utile != 0);
    return kBuckets - 1 - (int)(nt < kBuckets - 1 ? nt : kBuckets - 1);
  };
  unsigned long long packed = 0;
  __syncthreads();   // the histogram is cleared
  for (int b = b0; b < b1; ++b) {
    int e = 0;
    const uint32_t loc = local_of(b, e);
    const uint32_t nf = loc / chunk;
    packed += ((unsigned long long)(uint32_t)items_of(loc) << 32) | nf;
    if (loc - nf * chunk != 0) atomicAdd(&s_hist[bucket(loc - nf * chunk)], 1);
  }
  const unsigned long long incl = wave_incl_scan(packed, lane);
  const unsigned long long total =
      __shfl(incl, 63, 64);
  const unsigned long long pre = incl - packed;
  const int n_items = (int)(total >> 32);
  const int n_full = (int)(total & 0xffffffffu);
  __syncthreads();   // the histogram is complete
  // 4. tail positions: n_full + exclusive scan of the tail counts (lane = 16 buckets)
  int cnt[kBucketsPerLane];
  int mine = 0;
#pragma unroll
  for (int k = 0; k < kBucketsPerLane; ++k) {
    cnt[k] = s_hist[lane * kBucketsPerLane + k];
    mine += cnt[k];
  }
  int run = n_full + wave_incl_scan(mine, lane) - mine;
#pragma unroll
  for (int k = 0; k < kBucketsPerLane; ++k) {
    s_hist[lane * kBucketsPerLane + k] = run;
    run += cnt[k];
  }
  __syncthreads();   // the positions are in place
  int base = (int)(pre >> 32);
  int fpos = (int)(pre & 0xffffffffu);
  for (int b = b0; b < b1; ++b) {
    int e = 0;
    const uint32_t loc = local_of(b, e);
    const int n = items_of(loc);
    const int nf = (int)(loc / chunk);
    off[b] = base;
    for (int i = 0; i < nf; ++i)
      items[fpos + i] = make_int4(b, (int)(i * chunk), (int)((i + 1) * chunk), base + i);
    if (nf < n)
      items[atomicAdd(&s_hist[bucket(loc - nf * chunk)], 1)] =
          make_int4(b, (int)(nf * chunk), (int)loc, base + nf);
    base += n;
    fpos += nf;
  }
  if (lane == 0) {
    off[batch] = n_items;
    header[1] = n_items;
    header[2] = (int32_t)chunk;
    header[0] = err;
  }
}

// One workgroup per request: every owned token's physical slot, in ascending position.
__global__ __launch_bounds__(256) void slots_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    int max_blocks, int block_size, int64_t num_blocks, int rank, int cp, int interleave,
    const int64_t* __restrict__ out_offsets, int64_t* __restrict__ slots_out,
    int32_t* __restrict__ err_word) {
  const int b = blockIdx.x;
  long long L = seq_lens[b];
  int err = 0;
  const long long cap = (long long)max_blocks * block_size;
  if (L < 0) { err |= kErrSeqLen; L = 0; }
  if (L > cap) { err |= kErrSeqLen; L = cap; }
  const long long n = dcp_walk_local_count(L, rank, cp, interleave);
  int64_t* dst = slots_out + out_offsets[b];
  const int32_t* bt = block_table + (size_t)b * max_blocks;
  for (long long j = threadIdx.x; j < n; j += blockDim.x) {
    const uint32_t t = dcp_walk_global_pos((uint32_t)j, rank, cp, interleave);
    const uint32_t lp = t / (uint32_t)block_size;
    const int32_t page = bt[lp];
    if (page < 0 || page >= num_blocks) {
      err |= kErrBlockId;
      dst[j] = -1;
    } else {
      dst[j] = (int64_t)page * block_size + (t - lp * (uint32_t)block_size);
    }
  }
  if (err) atomicOr(err_word, err);
}

__global__ void clear_word_kernel(int32_t* w) { *w = 0; }

}  // namespace

hipError_t launch_plan(const int32_t* seq_lens, int batch, int rank, int cp, int interleave,
                       int64_t len_cap, int64_t target_items, int tile, int min_chunk,
                       const WsPtrs& ws, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(64), 0, stream, seq_lens, batch,
                     rank, cp, interleave, len_cap, target_items, tile, min_chunk, ws.header,
                     ws.off, ws.items);
  return hipGetLastError();
}

hipError_t launch_shard_slots(const int32_t* block_table, const int32_t* seq_lens, int batch,
                              int max_blocks, int block_size, int64_t num_blocks, int rank,
                              int cp, int interleave, const int64_t* out_offsets,
                              int64_t* slots_out, int32_t* err_word, hipStream_t stream) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, err_word);
  hipLaunchKernelGGL(slots_kernel, dim3(batch), dim3(256), 0, stream, block_table, seq_lens,
                     max_blocks, block_size, num_blocks, rank, cp, interleave, out_offsets,
                     slots_out, err_word);
  return hipGetLastError();
}

}  // namespace dcp

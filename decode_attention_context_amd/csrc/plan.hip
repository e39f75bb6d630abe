// plan.hip — work planning of a shard call and the exported block-table walk.
//
// A shard call's work is split into items: contiguous ranges of a request's local tokens
// (the tokens its rank owns, in ascending position).  The planner runs as one workgroup:
//   1. local_b = tokens of request b on this rank (the walker's closed form); seq_len is
//      clamped to the block table's capacity (error bit DCP_DEVERR_SEQ_LEN otherwise);
//   2. chunk = the item size: total local tokens / target item count, rounded up to the
//      kernel's tile and clamped to [min_chunk, the longest request];
//   3. n_b = ceil(local_b / chunk) items per request; off = exclusive prefix sum;
//   4. item i of request b = (b, i * chunk, min((i + 1) * chunk, local_b), off_b + i), the
//      last field being the index of its partial output;
//   5. the items are stored in dispatch order, by descending tile count (a counting sort
//      over kBuckets buckets, longer items sharing the top bucket): workgroup slot k runs
//      items[k].
// Since chunk >= total / target, the item count never exceeds target + batch, which is the
// bound the host sizes the workspace with.  A request's partials keep consecutive indices
// (the split combine reads them together); only the dispatch order changes.  Greedy
// dispatch of the longest items first keeps a ragged batch's long requests from starting
// in the last round: for 512 lognormal lengths around 67k tokens on 8 ranks it takes the
// simulated makespan from 1.54x to 1.04x the even share of one round.  The order within a
// bucket depends on atomics; no result does (each partial has its fixed index).
#include "launch.h"

namespace dcp {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kBuckets = 1024;   // tile-count buckets of the dispatch order

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ seq_lens, int batch, int rank, int cp, int interleave,
    int64_t len_cap, int64_t target, int tile, int min_chunk, int32_t* __restrict__ header,
    int32_t* __restrict__ off, int4* __restrict__ items) {
  __shared__ long long s_a[kPlanThreads];
  __shared__ long long s_b[kPlanThreads];
  __shared__ int s_err[kPlanThreads];
  __shared__ int s_hist[kBuckets];   // items per bucket, then next free position per bucket
  const int tid = threadIdx.x;
  const int per = (batch + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(tid * per, batch);
  const int b1 = min(b0 + per, batch);

  auto local_of = [&](int b, int& err) -> long long {
    long long L = seq_lens[b];
    if (L < 0) { err |= kErrSeqLen; L = 0; }
    if (L > len_cap) { err |= kErrSeqLen; L = len_cap; }
    return dcp_walk_local_count(L, rank, cp, interleave);
  };

  long long sum = 0, mx = 0;
  int err = 0;
  for (int b = b0; b < b1; ++b) {
    const long long loc = local_of(b, err);
    sum += loc;
    mx = loc > mx ? loc : mx;
  }
  s_a[tid] = sum;
  s_b[tid] = mx;
  s_err[tid] = err;
  __syncthreads();
  for (int s = kPlanThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
      s_a[tid] += s_a[tid + s];
      s_b[tid] = s_b[tid] > s_b[tid + s] ? s_b[tid] : s_b[tid + s];
      s_err[tid] |= s_err[tid + s];
    }
    __syncthreads();
  }
  const long long total = s_a[0];
  const long long maxloc = s_b[0];
  const int err_all = s_err[0];
  __syncthreads();

  long long chunk = (total + target - 1) / target;
  chunk = (chunk + tile - 1) / tile * tile;
  if (chunk < min_chunk) chunk = min_chunk;
  const long long cap = (maxloc + tile - 1) / tile * tile;
  if (chunk > cap) chunk = cap;
  if (chunk < tile) chunk = tile;

  long long cnt = 0;
  for (int b = b0; b < b1; ++b) {
    int e = 0;
    cnt += (local_of(b, e) + chunk - 1) / chunk;
  }
  // inclusive scan of the per-thread counts (Hillis-Steele over the workgroup)
  s_a[tid] = cnt;
  __syncthreads();
  for (int s = 1; s < kPlanThreads; s <<= 1) {
    const long long v = tid >= s ? s_a[tid - s] : 0;
    __syncthreads();
    s_a[tid] += v;
    __syncthreads();
  }
  long long base = s_a[tid] - cnt;
  for (int k = tid; k < kBuckets; k += kPlanThreads) s_hist[k] = 0;
  __syncthreads();
  // bucket of an item: kBuckets - 1 - (tile count, capped): longest first
  auto bucket = [&](long long len) -> int {
    const long long nt = (len + tile - 1) / tile;
    return kBuckets - 1 - (int)(nt < kBuckets - 1 ? nt : kBuckets - 1);
  };
  for (int b = b0; b < b1; ++b) {
    int e = 0;
    const long long loc = local_of(b, e);
    const long long n = (loc + chunk - 1) / chunk;
    off[b] = (int32_t)base;
    for (long long i = 0; i < n; ++i) {
      const long long j0 = i * chunk;
      const long long j1 = j0 + chunk < loc ? j0 + chunk : loc;
      atomicAdd(&s_hist[bucket(j1 - j0)], 1);
    }
    base += n;
  }
  __syncthreads();
  // exclusive prefix sum of the bucket counts (Hillis-Steele over kBuckets entries)
  {
    const int mine = tid < kBuckets ? s_hist[tid] : 0;
    for (int s = 1; s < kBuckets; s <<= 1) {
      const int v = (tid < kBuckets && tid >= s) ? s_hist[tid - s] : 0;
      __syncthreads();
      if (tid < kBuckets) s_hist[tid] += v;
      __syncthreads();
    }
    const int incl = tid < kBuckets ? s_hist[tid] : 0;
    __syncthreads();
    if (tid < kBuckets) s_hist[tid] = incl - mine;
    __syncthreads();
  }
  base = s_a[tid] - cnt;
  for (int b = b0; b < b1; ++b) {
    int e = 0;
    const long long loc = local_of(b, e);
    const long long n = (loc + chunk - 1) / chunk;
    for (long long i = 0; i < n; ++i) {
      const long long j0 = i * chunk;
      const long long j1 = j0 + chunk < loc ? j0 + chunk : loc;
      items[atomicAdd(&s_hist[bucket(j1 - j0)], 1)] =
          make_int4(b, (int)j0, (int)j1, (int)(base + i));
    }
    base += n;
  }
  if (tid == kPlanThreads - 1) {
    off[batch] = (int32_t)s_a[kPlanThreads - 1];
    header[1] = (int32_t)s_a[kPlanThreads - 1];
    header[2] = (int32_t)chunk;
    header[0] = err_all;
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
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, batch,
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

// gqa_shard.hip — paged GQA decode attention over one DCP rank's KV shard (gfx950).
//
// What it computes ("vLLM Decode Context Parallelism for long-context workloads" blog,
// "DCP execution flow", step "Compute", and "GQA backend"): for every request b and query
// head h, the attention of the gathered query q[b][h] over the tokens t < seq_len[b] that
// this rank owns ((t / interleave) mod cp_size == rank), reading KV head h / G, together
// with the natural-log LSE of the scaled scores, so that the partials of all ranks merge
// into exact attention.
//
// The work is HBM-bound (per token and KV head: 2 * D * sizeof(T) bytes against
// 4 * G * D flops), so the design is about streaming K and V at full rate on the vector
// ALUs:
//   * One workgroup of NW = min(G, 4) waves per work item (request, KV head, local token
//     range); wave w owns G / NW of the query heads that share the KV head.
//   * 64-token tiles of K and V rows are copied HBM -> LDS with global_load_lds_dwordx4
//     (no register staging), double buffered so that tile i+1 streams in while tile i is
//     computed.  The block-table walk gives each lane the cache row of one token; when the
//     64 rows are consecutive in memory (the common case: interleave and block size are
//     multiples of the tile) the copy addresses are plain offsets, otherwise each row
//     index comes from the lane that walked it.  The 16-byte chunks of a K row are
//     XOR-swizzled by (row mod 16) so the transposed reads below are conflict free.
//   * Scores: lane = token.  The lane pulls its K row from LDS into registers once, and
//     each query head, being wave-uniform, arrives as whole-row scalar loads used as the
//     scalar operand of v_dot2_f32_bf16 (bf16) or v_fma_f32 (f32): no cross-lane
//     reduction.
//   * Online softmax in base 2 (scale * log2 e folded into the scores).  The tile max per
//     head is a DPP butterfly plus four lane reads (no LDS); running sums stay per lane and
//     are reduced once per item.
//   * P.V: lane = one dword of every V row (2 bf16 dims or 1 f32 dim).  For bf16 the V
//     values of token pairs (2k, 2k+1) are packed with v_perm_b32 and combined with the
//     bf16-rounded weight pairs by v_dot2_f32_bf16 into fp32 accumulators; the weights are
//     broadcast through LDS.
//   * An item that covers a request's whole shard writes (O, lse) directly; otherwise it
//     writes a normalized partial that the split combine merges.
#include "launch.h"

namespace dcp {

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(16))) uint32_t u32x16;
#define DCP_LDS __attribute__((address_space(3)))
#define DCP_CONST __attribute__((address_space(4)))

constexpr int kTile = kGqaTile;      // tokens per tile (= lanes)
constexpr int kRowBytes = 256;       // D * sizeof(T) for the supported shapes
constexpr int kChunks = kRowBytes / 16;
constexpr int kTileBytes = kTile * kRowBytes;   // 16 KiB
constexpr int kDmaPerTile = kTileBytes / 1024;  // 1 KiB per copy instruction

struct GqaKArgs {
  const void* q;
  const char* kp;
  const char* vp;
  const int32_t* bt;
  int hq, hkv, block_size, max_blocks;
  uint32_t num_blocks;
  int rank, cp, interleave;
  float sl2;  // scale * log2(e)
  float* o_out;
  float* lse_out;
  int32_t* header;
  const int32_t* off;
  const int4* items;
  float* plse;
  float* po;
};

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

constexpr int waves_for(int g) { return g >= 4 ? 4 : g; }

template <bool kBf16, int G>
__global__ __launch_bounds__(64 * waves_for(G), 2) void gqa_shard_kernel(GqaKArgs a) {
  constexpr int NW = waves_for(G);
  constexpr int HPW = G / NW;                   // query heads per wave
  constexpr int kElemBytes = kBf16 ? 2 : 4;
  constexpr int D = kRowBytes / kElemBytes;     // head dim
  constexpr int NA = kBf16 ? 2 : 1;             // accumulators per lane per head
  constexpr int kDmaPerWave = kDmaPerTile / NW;
  constexpr int kPWords = kBf16 ? kTile / 2 : kTile;  // weight slots per head per tile

  // [buffer][K, V][row * 16 + chunk]
  __shared__ u32x4 kv[2][2][kTile * kChunks];
  __shared__ uint32_t pbuf[NW][kPWords * HPW];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int item = blockIdx.x;
  if (item >= a.header[1]) return;
  const int4 it = a.items[item];
  const int b = it.x, j0 = it.y, j1 = it.z;
  const int kvh = blockIdx.y;
  const bool single = (a.off[b + 1] - a.off[b]) == 1;
  const int head0 = kvh * G + w * HPW;          // first query head of this wave
  // the wave's query heads: wave-uniform, read-only -> scalar loads
  const uint32_t DCP_CONST* qh = reinterpret_cast<const uint32_t DCP_CONST*>(
                                     reinterpret_cast<uintptr_t>(a.q)) +
                                 ((size_t)b * a.hq + head0) * (kRowBytes / 4);
  const int32_t* btb = a.bt + (size_t)b * a.max_blocks;
  const uint32_t B = (uint32_t)a.block_size;

  float m[HPW], ls[HPW], acc[HPW][NA];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m[h] = neg_inf();
    ls[h] = 0.f;
#pragma unroll
    for (int k = 0; k < NA; ++k) acc[h][k] = 0.f;
  }

  // ---- block-table walk: lane = local token tj + lane
  auto page_of = [&](int tj) -> int32_t {
    const int j = tj + lane;
    if (j >= j1) return 0;
    const uint32_t t = dcp_walk_global_pos((uint32_t)j, a.rank, a.cp, a.interleave);
    return btb[t / B];
  };
  // cache row (page * Hkv + kvh) * B + slot of the lane's token; ballot of valid tokens
  auto row_of = [&](int tj, int32_t pg, uint32_t& row) -> uint64_t {
    const int j = tj + lane;
    bool ok = j < j1;
    bool bad = false;
    row = 0;
    if (ok) {
      if (pg < 0 || (uint32_t)pg >= a.num_blocks) {
        ok = false;
        bad = true;
      } else {
        const uint32_t t = dcp_walk_global_pos((uint32_t)j, a.rank, a.cp, a.interleave);
        row = ((uint32_t)pg * a.hkv + kvh) * B + t % B;
      }
    }
    if (__ballot(bad) != 0 && threadIdx.x == 0) atomicOr(&a.header[0], kErrBlockId);
    return __ballot(ok);
  };
  // ---- HBM -> LDS copy of the K and V rows of one tile (this wave's share)
  char* lds_base = reinterpret_cast<char*>(&kv[0][0][0]);
  asm volatile("" : "+v"(lds_base));
  auto issue_tile = [&](int buf, uint32_t row) {
    const uint32_t row0 = __builtin_amdgcn_readfirstlane(row);
    const bool contig = __ballot(row == row0 + (uint32_t)lane) == ~0ull;
    const int pc = lane & (kChunks - 1);
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
      const int blk = w * kDmaPerWave + k;
      const int r = blk * (64 / kChunks) + lane / kChunks;  // tile row of this lane's slot
      const uint32_t rr = contig ? row0 + r : __shfl(row, r, 64);
      const size_t rb = (size_t)rr * kRowBytes;
      // K chunks XOR-swizzled (read transposed below), V rows stored as they are (read
      // row-wise: consecutive lanes hit consecutive banks)
      // the destination is formed from an opaque byte base so that the compiler does not
      // treat the copy as aliasing the tile being read (which would make every read wait
      // for the copy of the next tile); the loop's own wait + barrier order the buffers
      char* kd = lds_base + ((buf * 2 + 0) * kTileBytes + blk * 1024);
      char* vd = lds_base + ((buf * 2 + 1) * kTileBytes + blk * 1024);
      __builtin_amdgcn_global_load_lds(a.kp + rb + ((pc ^ (r & 15)) * 16), (void DCP_LDS*)kd, 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(a.vp + rb + pc * 16, (void DCP_LDS*)vd, 16, 0, 0);
    }
  };

  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  uint32_t row;
  uint64_t vm_cur = row_of(j0, page_of(j0), row);
  issue_tile(0, row);
  int32_t pg_next = ntiles > 1 ? page_of(j0 + kTile) : 0;

  for (int ti = 0; ti < ntiles; ++ti) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int tj = j0 + ti * kTile;
    uint64_t vm_next = 0;
    if (ti + 1 < ntiles) {
      vm_next = row_of(tj + kTile, pg_next, row);
      issue_tile((ti + 1) & 1, row);
      if (ti + 2 < ntiles) pg_next = page_of(tj + 2 * kTile);
    }
    const u32x4* kt = kv[ti & 1][0];
    const uint32_t* vt = reinterpret_cast<const uint32_t*>(kv[ti & 1][1]);

    // ---- scores: lane = token; the K row moves to registers once
    u32x4 krow[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) krow[c] = kt[lane * kChunks + (c ^ (lane & 15))];
    // 16 query dwords per scalar load, one load ahead of its use; each step is its own
    // scheduling region so that no more than two chunks (32 scalar registers) are live
    constexpr int kQSteps = HPW * (kChunks / 4);
    auto qload = [&](int st) -> u32x16 {
      uint64_t qa = reinterpret_cast<uint64_t>(qh + (st / (kChunks / 4)) * (kRowBytes / 4) +
                                               16 * (st % (kChunks / 4)));
      asm volatile("" : "+s"(qa));
      return *reinterpret_cast<const u32x16 DCP_CONST*>(qa);
    };
    float s[HPW];
    float sacc[HPW][2];
#pragma unroll
    for (int h = 0; h < HPW; ++h) sacc[h][0] = sacc[h][1] = 0.f;
    u32x16 qv[2];
    qv[0] = qload(0);
#pragma unroll
    for (int st = 0; st < kQSteps; ++st) {
      if (st + 1 < kQSteps) qv[(st + 1) & 1] = qload(st + 1);
      const int h = st / (kChunks / 4), qc = st % (kChunks / 4);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t kd = krow[4 * qc + e / 4][e % 4];
        float& dst = sacc[h][e & 1];
        if constexpr (kBf16) dst = dot2_bf16(qv[st & 1][e], kd, dst);
        else dst = fmaf(__uint_as_float(qv[st & 1][e]), __uint_as_float(kd), dst);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int h = 0; h < HPW; ++h) s[h] = sacc[h][0] + sacc[h][1];

    // ---- online softmax (base 2); weights to LDS for the P.V broadcast
    const bool valid = (vm_cur >> lane) & 1;
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const float x = valid ? s[h] * a.sl2 : neg_inf();
      const float mn = fmaxf(m[h], wave_max_dpp(x));
      float alpha = 1.f, p = 0.f;
      if (mn != neg_inf()) {
        alpha = __builtin_amdgcn_exp2f(m[h] - mn);
        p = __builtin_amdgcn_exp2f(x - mn);
      }
      m[h] = mn;
      ls[h] = fmaf(ls[h], alpha, p);
#pragma unroll
      for (int k = 0; k < NA; ++k) acc[h][k] *= alpha;
      if constexpr (kBf16) {
        // pair (2k, 2k+1) as one bf16x2 word, written by the even lane
        const uint32_t pb = f32_to_bf16_rne(p);
        const uint32_t pn = (uint32_t)__builtin_amdgcn_update_dpp((int)pb, (int)pb, kDppQuadXor1,
                                                                  0xF, 0xF, false);
        if (!(lane & 1)) pbuf[w][(lane >> 1) * HPW + h] = pb | (pn << 16);
      } else {
        pbuf[w][lane * HPW + h] = __float_as_uint(p);
      }
    }

    // ---- P.V: lane = one dword of every V row
    if constexpr (kBf16) {
#pragma unroll
      for (int k = 0; k < kTile / 2; ++k) {
        const uint32_t v0 = vt[(2 * k) * (kRowBytes / 4) + lane];
        const uint32_t v1 = vt[(2 * k + 1) * (kRowBytes / 4) + lane];
        const uint32_t lo = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
          const uint32_t pp = pbuf[w][k * HPW + h];
          acc[h][0] = dot2_bf16(pp, lo, acc[h][0]);
          acc[h][1] = dot2_bf16(pp, hi, acc[h][1]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kTile; ++t) {
        const float v = __uint_as_float(vt[t * (kRowBytes / 4) + lane]);
#pragma unroll
        for (int h = 0; h < HPW; ++h)
          acc[h][0] = fmaf(__uint_as_float(pbuf[w][t * HPW + h]), v, acc[h][0]);
      }
    }
    vm_cur = vm_next;
  }

  // ---- finalize: O = acc / l, lse = (m + log2 l) ln 2
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float lt = wave_sum_dpp(ls[h]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (m[h] + __log2f(lt)) * kLn2 : neg_inf();
    const int head = head0 + h;
    float* dst = single ? a.o_out + ((size_t)b * a.hq + head) * D
                        : a.po + ((size_t)item * a.hq + head) * D;
    if constexpr (kBf16) {
      *reinterpret_cast<float2*>(dst + 2 * lane) = make_float2(acc[h][0] * inv, acc[h][1] * inv);
    } else {
      dst[lane] = acc[h][0] * inv;
    }
    if (lane == 0) {
      if (single) a.lse_out[(size_t)b * a.hq + head] = lse;
      else a.plse[(size_t)item * a.hq + head] = lse;
    }
  }
}

template <bool kBf16>
hipError_t launch_g(const GqaKArgs& k, int group, dim3 grid, hipStream_t s) {
  switch (group) {
    case 1: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 1>), grid, dim3(64 * waves_for(1)), 0, s, k); break;
    case 2: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 2>), grid, dim3(64 * waves_for(2)), 0, s, k); break;
    case 4: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 4>), grid, dim3(64 * waves_for(4)), 0, s, k); break;
    case 8: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 8>), grid, dim3(64 * waves_for(8)), 0, s, k); break;
    case 16: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 16>), grid, dim3(64 * waves_for(16)), 0, s, k); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool gqa_supported(int dtype, int head_dim, int group) {
  const int elem = dtype == 1 ? 2 : 4;
  if (head_dim * elem != kRowBytes) return false;
  return group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
}

hipError_t launch_gqa_shard(const GqaArgs& a, int64_t max_items, const WsPtrs& ws,
                            float* o_out, float* lse_out, hipStream_t stream) {
  GqaKArgs k;
  k.q = a.q;
  k.kp = static_cast<const char*>(a.k_pages);
  k.vp = static_cast<const char*>(a.v_pages);
  k.bt = a.block_table;
  k.hq = a.hq;
  k.hkv = a.hkv;
  k.block_size = a.block_size;
  k.max_blocks = a.max_blocks;
  k.num_blocks = (uint32_t)a.num_blocks;
  k.rank = a.rank;
  k.cp = a.cp;
  k.interleave = a.interleave;
  k.sl2 = a.scale * kLog2e;
  k.o_out = o_out;
  k.lse_out = lse_out;
  k.header = ws.header;
  k.off = ws.off;
  k.items = ws.items;
  k.plse = ws.plse;
  k.po = ws.po;
  const dim3 grid((unsigned)max_items, (unsigned)a.hkv);
  const int group = a.hq / a.hkv;
  return a.dtype == 1 ? launch_g<true>(k, group, grid, stream)
                      : launch_g<false>(k, group, grid, stream);
}

}  // namespace dcp

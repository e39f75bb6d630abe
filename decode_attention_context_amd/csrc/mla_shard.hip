// mla_shard.hip — paged MLA decode attention over one DCP rank's shard, on bf16 MFMA.
//
// What it computes ("vLLM Decode Context Parallelism for long-context workloads" blog,
// "DCP execution flow", step "Compute", and "The memory wall in long-context inference",
// MLA item: all query heads share one low-rank latent KV row): for every request b and
// each of the 128 gathered query heads h, attention over the tokens this rank owns, with
// key = the token's 576-wide latent row and value = its first 512 columns, plus the
// natural-log LSE of the scaled scores.
//
// Per token this is 128 x (576 + 512) multiply-adds against 1152 bytes of cache: a dense
// contraction (about 242 flop/byte), so both products run on v_mfma_f32_16x16x32_bf16.
//
// Design:
//   * One workgroup of 8 waves per work item (request, local token range); wave w owns
//     query heads 16w .. 16w+15, so every cache byte is read from HBM once for all 128
//     heads.  The wave keeps its heads' query (18 k-steps x 8 bf16 per lane) and the fp32
//     output accumulator (32 tiles of 16 dims x 16 heads) in registers.
//   * 64-token tiles of latent rows are copied HBM -> LDS by global_load_lds_dwordx4
//     (no register staging), double buffered: tile i+1 streams in while tile i is
//     computed.  Rows are gathered through the block-table walk, so any interleave and
//     block size work; the 16-byte chunks of a row are XOR-swizzled by (row mod 8) so that
//     MFMA operand reads hit distinct banks.
//   * Scores as S^T = K . Q^T (M = 16 tokens, N = 16 heads, K = 32 latent dims): every
//     lane's four results belong to ONE head, so the online-softmax max needs only two
//     cross-lane steps and the weights never move between lanes.
//   * Output as O^T = V^T . P^T (M = 16 value dims, N = 16 heads, K = 32 tokens).  The
//     weight operand is the score registers rounded to bf16; the V^T operand is read with
//     ds_read_b64_tr_b16, which transposes 16-bit elements across each 16-lane group, in
//     the same token order as the score registers.  Accumulator lanes again hold one head,
//     so the online-softmax rescale is lane-local (and skipped when no max changed).
#include "launch.h"

namespace dcp {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
#define DCP_LDS __attribute__((address_space(3)))

constexpr int kHeads = 128;
constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kTile = kMlaTile;              // 64 tokens
constexpr int kRowBytes = kDk * 2;           // 1152
constexpr int kRowChunks = kRowBytes / 16;   // 72
constexpr int kTileBytes = kTile * kRowBytes;  // 73728
constexpr int kKSteps = kDk / 32;            // 18
constexpr int kDvTiles = kDv / 16;           // 32
// Query heads per wave = 16 * kHeadTiles; the workgroup has 128 / that many waves.
constexpr int kHeadTiles = 1;
constexpr int kWaves = kHeads / (16 * kHeadTiles);
constexpr int kDmaPerWave = kTileBytes / 1024 / kWaves;

struct MlaKArgs {
  const uint16_t* q;
  const char* lat;
  const int32_t* bt;
  int block_size, max_blocks;
  uint32_t num_blocks;
  int rank, cp, interleave;
  float sl2;
  float* o_out;
  float* lse_out;
  int32_t* header;
  const int32_t* off;
  const int4* items;
  float* plse;
  float* po;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ u32x2 lds_tr16(const char DCP_LDS* p) {
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 DCP_LDS*)p);
  return __builtin_bit_cast(u32x2, v);
}

__global__ __launch_bounds__(kWaves * 64, 1) void mla_shard_kernel(MlaKArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileBytes];

  const int item = blockIdx.x;
  if (item >= a.header[1]) return;
  const int4 it = a.items[item];
  const int b = it.x, j0 = it.y, j1 = it.z;
  const bool single = (a.off[b + 1] - a.off[b]) == 1;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;      // 16-lane group
  const int i16 = lane & 15;
  const int head0 = 16 * kHeadTiles * w + i16;   // head of head tile ht: head0 + 16 ht
  const uint32_t B = (uint32_t)a.block_size;
  const int32_t* btb = a.bt + (size_t)b * a.max_blocks;

  // ---- block-table walk: cache row of local token tj + lane
  auto page_of = [&](int tj) -> int32_t {
    const int j = tj + lane;
    if (j >= j1) return 0;
    const uint32_t t = dcp_walk_global_pos((uint32_t)j, a.rank, a.cp, a.interleave);
    return btb[t / B];
  };
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
        row = (uint32_t)pg * B + t % B;
      }
    }
    if (__ballot(bad) != 0 && threadIdx.x == 0) atomicOr(&a.header[0], kErrBlockId);
    return __ballot(ok);
  };
  // ---- HBM -> LDS copy of one tile (1 KiB per instruction, kDmaPerWave per wave)
  auto issue_tile = [&](char* buf, uint32_t row) {
    // An opaque copy of the lane id keeps the slot arithmetic below from being hoisted out
    // of the tile loop (it is cheap to redo, and hoisted it would pin 2 * kDmaPerWave
    // registers for the whole kernel).
    int lane_o;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_o) : "v"(lane));
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
      const int blk = w * kDmaPerWave + k;
      const int s = blk * 64 + lane_o;          // 16-B slot in the tile
      const int r = s / kRowChunks;
      const int c = (s - r * kRowChunks) ^ (r & 7);
      const uint32_t rr = __shfl(row, r, 64);
      const char* src = a.lat + (size_t)rr * kRowBytes + c * 16;
      __builtin_amdgcn_global_load_lds(src, (void DCP_LDS*)(buf + blk * 1024), 16, 0, 0);
    }
  };

  // ---- query (B operand of S^T = K Q^T): dims 32 ks + 8 g .. + 8 of each head tile
  bf16x8 qreg[kHeadTiles][kKSteps];
#pragma unroll
  for (int ht = 0; ht < kHeadTiles; ++ht) {
    const uint16_t* qrow = a.q + ((size_t)b * kHeads + head0 + 16 * ht) * kDk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[ht][ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }

  f4 acc[kHeadTiles][kDvTiles];
#pragma unroll
  for (int ht = 0; ht < kHeadTiles; ++ht)
#pragma unroll
    for (int i = 0; i < kDvTiles; ++i) acc[ht][i] = f4{0.f, 0.f, 0.f, 0.f};
  float m[kHeadTiles], ls[kHeadTiles];
#pragma unroll
  for (int ht = 0; ht < kHeadTiles; ++ht) {
    m[ht] = neg_inf();
    ls[ht] = 0.f;
  }

  // per-lane LDS offsets (chunk c of row r sits at byte 16 * (72 r + (c ^ (r & 7))))
  const int xk = i16 & 7;
  const int offk0 = i16 * kRowBytes + 16 * (g ^ xk);
  const int offk1 = i16 * kRowBytes + 16 * ((4 + g) ^ xk);
  const int rv = 4 * g + (i16 >> 2);
  const int xv = rv & 7;
  const int qv = (i16 >> 1) & 1;
  int offv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) offv[u] = rv * kRowBytes + 16 * ((2 * u + qv) ^ xv) + (i16 & 1) * 8;

  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  uint32_t row;
  uint64_t vm_cur = row_of(j0, page_of(j0), row);
  issue_tile(smem, row);
  int32_t pg_next = ntiles > 1 ? page_of(j0 + kTile) : 0;

  for (int ti = 0; ti < ntiles; ++ti) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int tj = j0 + ti * kTile;
    uint64_t vm_next = 0;
    if (ti + 1 < ntiles) {
      vm_next = row_of(tj + kTile, pg_next, row);
      issue_tile(smem + ((ti + 1) & 1) * kTileBytes, row);
      if (ti + 2 < ntiles) pg_next = page_of(tj + 2 * kTile);
    }
    const char* buf = smem + (ti & 1) * kTileBytes;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // scores of tokens 32 kb + [0, 16) (s[ht][0]) and 32 kb + [16, 32) (s[ht][1])
      f4 s[kHeadTiles][2];
#pragma unroll
      for (int ht = 0; ht < kHeadTiles; ++ht) s[ht][0] = s[ht][1] = f4{0.f, 0.f, 0.f, 0.f};
      const char* bk0 = buf + (2 * kb) * 16 * kRowBytes;
      const char* bk1 = bk0 + 16 * kRowBytes;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const int o = ((ks & 1) ? offk1 : offk0) + 128 * (ks >> 1);
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(bk0 + o);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(bk1 + o);
#pragma unroll
        for (int ht = 0; ht < kHeadTiles; ++ht) {
          s[ht][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[ht][ks], s[ht][0], 0, 0, 0);
          s[ht][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[ht][ks], s[ht][1], 0, 0, 0);
        }
        // keep the scheduler from hoisting every operand read (register pressure)
        if (ks % 3 == 2) __builtin_amdgcn_sched_barrier(0);
      }
      // lane holds one head per tile; s[.][0][i] is token 32 kb + 4 g + i, s[.][1][i] is
      // token 32 kb + 16 + 4 g + i
      bf16x8 pb[kHeadTiles];
#pragma unroll
      for (int ht = 0; ht < kHeadTiles; ++ht) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = s[ht][0][i] * a.sl2;
          x[4 + i] = s[ht][1][i] * a.sl2;
        }
        if (vm_cur != ~0ull) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (!((vm_cur >> (32 * kb + 4 * g + i)) & 1)) x[i] = neg_inf();
            if (!((vm_cur >> (32 * kb + 16 + 4 * g + i)) & 1)) x[4 + i] = neg_inf();
          }
        }
        float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(m[ht], tmax);
        if (__ballot(mn > m[ht]) != 0) {
          const float alpha = mn > m[ht] ? __builtin_amdgcn_exp2f(m[ht] - mn) : 1.f;
          ls[ht] *= alpha;
#pragma unroll
          for (int i = 0; i < kDvTiles; ++i) acc[ht][i] *= alpha;
        }
        m[ht] = mn;
        const float msafe = mn == neg_inf() ? 0.f : mn;
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = __builtin_amdgcn_exp2f(x[i] - msafe);
          ls[ht] += p[i];
        }
        u32x4 pw;
        pw.x = pack_bf16x2(p[0], p[1]);
        pw.y = pack_bf16x2(p[2], p[3]);
        pw.z = pack_bf16x2(p[4], p[5]);
        pw.w = pack_bf16x2(p[6], p[7]);
        pb[ht] = __builtin_bit_cast(bf16x8, pw);
      }

      const char* bv0 = buf + (32 * kb) * kRowBytes;
      const char* bv1 = bv0 + 16 * kRowBytes;
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) {
        const int o = offv[dt & 3] + 128 * (dt >> 2);
        const u32x2 v0 = lds_tr16((const char DCP_LDS*)(bv0 + o));
        const u32x2 v1 = lds_tr16((const char DCP_LDS*)(bv1 + o));
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
#pragma unroll
        for (int ht = 0; ht < kHeadTiles; ++ht)
          acc[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ht], acc[ht][dt], 0, 0, 0);
        if (dt % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    vm_cur = vm_next;
  }

  // ---- finalize: lane holds dims 16 dt + 4 g + [0, 4) of head head0 + 16 ht
#pragma unroll
  for (int ht = 0; ht < kHeadTiles; ++ht) {
    float lt = ls[ht] + __shfl_xor(ls[ht], 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (m[ht] + __log2f(lt)) * kLn2 : neg_inf();
    const int head = head0 + 16 * ht;
    float* dst = single ? a.o_out + ((size_t)b * kHeads + head) * kDv
                        : a.po + ((size_t)item * kHeads + head) * kDv;
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt) {
      const f4 v = acc[ht][dt] * inv;
      *reinterpret_cast<f4*>(dst + 16 * dt + 4 * g) = v;
    }
    if (g == 0) {
      if (single) a.lse_out[(size_t)b * kHeads + head] = lse;
      else a.plse[(size_t)item * kHeads + head] = lse;
    }
  }
}

}  // namespace

hipError_t launch_mla_shard(const MlaArgs& a, int64_t max_items, const WsPtrs& ws,
                            float* o_out, float* lse_out, hipStream_t stream) {
  MlaKArgs k;
  k.q = static_cast<const uint16_t*>(a.q);
  k.lat = static_cast<const char*>(a.latent);
  k.bt = a.block_table;
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
  hipLaunchKernelGGL(mla_shard_kernel, dim3((unsigned)max_items), dim3(kWaves * 64), 0, stream, k);
  return hipGetLastError();
}

}  // namespace dcp

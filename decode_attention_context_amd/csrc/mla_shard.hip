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

#ifndef MLA_HT
#define MLA_HT 1
#endif
#ifndef MLA_NW
#define MLA_NW 4
#endif

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
constexpr int kXcds = 8;                     // MI355X: 8 XCDs, workgroups dealt round-robin

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

// HT = 16-head tiles per wave, NW = waves per workgroup.  A workgroup covers
// 16 * HT * NW query heads; the 128 heads form kGroups = 128 / (16 HT NW) head groups,
// each a workgroup of its own.  Workgroup ids are laid out so that every head group of one
// work item lands on the same XCD (ids congruent mod 8) and is dispatched close in time, so
// the groups' reads of the same latent tiles meet in that XCD's L2.
template <int HT, int NW>
__global__ __launch_bounds__(NW * 64, 1) void mla_shard_kernel(MlaKArgs a) {
  constexpr int kGroups = kHeads / (16 * HT * NW);
  constexpr int kDmaPerWave = kTileBytes / 1024 / NW;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileBytes];

  const int blk = blockIdx.x;
  const int hg = (blk / kXcds) % kGroups;
  const int item = (blk / (kXcds * kGroups)) * kXcds + blk % kXcds;
  if (item >= a.header[1]) return;
  const int4 it = a.items[item];
  const int b = it.x, j0 = it.y, j1 = it.z;
  const bool single = (a.off[b + 1] - a.off[b]) == 1;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4;      // 16-lane group
  const int i16 = lane & 15;
  // head of head tile ht: head0 + 16 ht
  const int head0 = 16 * HT * (NW * hg + w) + i16;
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
    // of the tile loop (cheap to redo; hoisted it would pin 2 * kDmaPerWave registers).
    int lane_o;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_o) : "v"(lane));
    uint32_t rr[kDmaPerWave];
    int cc[kDmaPerWave];
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {   // every row-index shuffle first ...
      const int s = (w * kDmaPerWave + k) * 64 + lane_o;   // 16-B slot in the tile
      const int r = s / kRowChunks;
      cc[k] = (s - r * kRowChunks) ^ (r & 7);
      rr[k] = __shfl(row, r, 64);
    }
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {   // ... then the copies back to back
      const char* src = a.lat + (size_t)rr[k] * kRowBytes + cc[k] * 16;
      __builtin_amdgcn_global_load_lds(src, (void DCP_LDS*)(buf + (w * kDmaPerWave + k) * 1024),
                                       16, 0, 0);
    }
  };

  // ---- query (B operand of S^T = K Q^T): dims 32 ks + 8 g .. + 8 of each head tile
  bf16x8 qreg[HT][kKSteps];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint16_t* qrow = a.q + ((size_t)b * kHeads + head0 + 16 * ht) * kDk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[ht][ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }

  f4 acc[HT][kDvTiles];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < kDvTiles; ++i) acc[ht][i] = f4{0.f, 0.f, 0.f, 0.f};
  float m[HT], ls[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
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

    // ---- scores of the whole tile: s[ht][nt][i] is token 16 nt + 4 g + i of head tile ht
    f4 s[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) s[ht][nt] = f4{0.f, 0.f, 0.f, 0.f};
    // K operands are read two k-steps ahead of the MFMAs that use them (3-slot ring), so
    // every read has a full step of MFMAs to hide behind
    bf16x8 kop[3][4];
    auto kread = [&](int ks) {
      const int o = ((ks & 1) ? offk1 : offk0) + 128 * (ks >> 1);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        kop[ks % 3][nt] = *reinterpret_cast<const bf16x8*>(buf + nt * 16 * kRowBytes + o);
    };
    kread(0);
    kread(1);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + 2 < kKSteps) kread(ks + 2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          s[ht][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks % 3][nt], qreg[ht][ks],
                                                               s[ht][nt], 0, 0, 0);
      // one scheduling region per k-step
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax over the tile; P as the bf16 B operand of O^T += V^T P^T
    // k-block kb covers tokens 32 kb + [0, 32): lane slots 8 g .. 8 g + 7 hold tokens
    // 32 kb + 4 g + [0, 4) and 32 kb + 16 + 4 g + [0, 4), the order of the V^T reads below.
    bf16x8 pb[HT][2];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float x[16];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * nt + i] = s[ht][nt][i] * a.sl2;
      if (vm_cur != ~0ull) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((vm_cur >> (16 * nt + 4 * g + i)) & 1)) x[4 * nt + i] = neg_inf();
      }
      float tmax = x[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, x[i]);
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
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(x[i] - msafe);
        ls[ht] += p[i];
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float* p0 = p + 8 * kb;        // token tile 2 kb
        const float* p1 = p + 8 * kb + 4;    // token tile 2 kb + 1
        u32x4 pw;
        pw.x = pack_bf16x2(p0[0], p0[1]);
        pw.y = pack_bf16x2(p0[2], p0[3]);
        pw.z = pack_bf16x2(p1[0], p1[1]);
        pw.w = pack_bf16x2(p1[2], p1[3]);
        pb[ht][kb] = __builtin_bit_cast(bf16x8, pw);
      }
    }

    // ---- O^T += V^T P^T (V^T operands of dim tile dt+1 read during the MFMAs of dt)
    auto vop = [&](int dt, int kb) -> bf16x8 {
      const int o = offv[dt & 3] + 128 * (dt >> 2);
      const char* bv = buf + (32 * kb) * kRowBytes;
      const u32x2 v0 = lds_tr16((const char DCP_LDS*)(bv + o));
      const u32x2 v1 = lds_tr16((const char DCP_LDS*)(bv + 16 * kRowBytes + o));
      return __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
    };
    bf16x8 va[2][2];
    va[0][0] = vop(0, 0);
    va[0][1] = vop(0, 1);
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt) {
      if (dt + 1 < kDvTiles) {
        va[(dt + 1) & 1][0] = vop(dt + 1, 0);
        va[(dt + 1) & 1][1] = vop(dt + 1, 1);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          acc[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt & 1][kb], pb[ht][kb],
                                                                acc[ht][dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    vm_cur = vm_next;
  }

  // ---- finalize: lane holds dims 16 dt + 4 g + [0, 4) of head head0 + 16 ht
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
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

constexpr int kHT = MLA_HT;
constexpr int kNW = MLA_NW;
constexpr int kGroupsUsed = kHeads / (16 * kHT * kNW);

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
  const int64_t groups8 = (max_items + kXcds - 1) / kXcds;
  hipLaunchKernelGGL((mla_shard_kernel<kHT, kNW>), dim3((unsigned)(groups8 * kXcds * kGroupsUsed)),
                     dim3(kNW * 64), 0, stream, k);
  return hipGetLastError();
}

}  // namespace dcp

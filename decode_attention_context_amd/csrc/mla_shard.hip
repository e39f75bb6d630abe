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
#define DCP_CONST __attribute__((address_space(4)))

constexpr int kHeads = 128;
constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kTile = kMlaTile;              // 32 tokens per tile
constexpr int kNBuf = 4;                     // LDS tile ring: one computed, three in flight
constexpr int kRowBytes = kDk * 2;           // 1152
constexpr int kRowChunks = kRowBytes / 16;   // 72
constexpr int kTileBytes = kTile * kRowBytes;  // 36 KiB
constexpr int kKSteps = kDk / 32;            // 18
constexpr int kDvTiles = kDv / 16;           // 32
constexpr int kXcds = 8;                     // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr float kRescaleSlack = 8.f;          // see the online softmax below
constexpr int kAhead = 6;                    // LDS operand prefetch distance (MFMA steps)

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

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int kVm>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((kVm & 0xF) | ((kVm >> 4) << 14) | (0x7 << 4) | (0xF << 8));
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
  __shared__ __attribute__((aligned(1024))) char smem[kNBuf * kTileBytes];

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
  // Contiguous tiles: when the interleave and the block size are multiples of the tile, the
  // 32 tokens of a tile are consecutive positions inside one cache page, so one scalar
  // block-table read locates the whole tile.  Otherwise every token is walked by a lane.
  const bool fast = (a.interleave % kTile) == 0 && (a.block_size % kTile) == 0;

  // The copies write through an opaque base, the tile reads go through the array itself:
  // otherwise the compiler takes every read as aliasing the copies still in flight and
  // waits for all of them (the ring's own counter waits and barriers order the buffers).
  char DCP_LDS* lds_dma = (char DCP_LDS*)smem;
  asm volatile("" : "+v"(lds_dma));
  const char DCP_LDS* lds = (const char DCP_LDS*)smem;
  // the block table through the constant address space: scalar loads, which do not count
  // against the vector-memory counter the copy ring is paced with
  const int32_t DCP_CONST* btc = reinterpret_cast<const int32_t DCP_CONST*>(
      reinterpret_cast<uintptr_t>(btb));

  // Per-lane copy slots (loop invariant): 16-B slot (w * kDmaPerWave + k) * 64 + lane of a
  // tile holds chunk (s mod 72) ^ (row & 7) of tile row s / 72.
  uint32_t slot_off[kDmaPerWave], slot_col[kDmaPerWave];
  int slot_row[kDmaPerWave];
#pragma unroll
  for (int k = 0; k < kDmaPerWave; ++k) {
    const int sl = (w * kDmaPerWave + k) * 64 + lane;
    const int r = sl / kRowChunks;
    slot_row[k] = r;
    slot_col[k] = (uint32_t)(((sl - r * kRowChunks) ^ (r & 7)) * 16);
    slot_off[k] = (uint32_t)r * kRowBytes + slot_col[k];
  }

  // ---- one tile's HBM -> LDS copy (kDmaPerWave instructions of 1 KiB per wave); returns
  // the ballot of valid rows.  Chunk c of row r lands at byte 16 * (72 r + (c ^ (r & 7))).
  auto issue_tile = [&](int ti) -> uint64_t {
    const int tj = j0 + ti * kTile;
    char DCP_LDS* buf = lds_dma + (ti % kNBuf) * kTileBytes;
    uint32_t row0 = 0;
    uint32_t lrow = 0;              // slow path: this lane's row (lane < 32)
    uint64_t vm;
    if (fast) {
      const uint32_t t0 = dcp_walk_global_pos((uint32_t)tj, a.rank, a.cp, a.interleave);
      const uint32_t lp = t0 / B;
      const int32_t pg = btc[lp];
      const int nvalid = min(kTile, j1 - tj);
      const bool ok = pg >= 0 && (uint32_t)pg < a.num_blocks;
      if (!ok && threadIdx.x == 0) atomicOr(&a.header[0], kErrBlockId);
      row0 = ok ? (uint32_t)pg * B + (t0 - lp * B) : 0u;
      vm = ok ? (nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1)) : 0ull;
    } else {
      const int j = tj + lane;
      bool ok = lane < kTile && j < j1;
      bool bad = false;
      if (ok) {
        const uint32_t t = dcp_walk_global_pos((uint32_t)j, a.rank, a.cp, a.interleave);
        const uint32_t lp = t / B;
        const int32_t pg = btb[lp];
        if (pg < 0 || (uint32_t)pg >= a.num_blocks) {
          ok = false;
          bad = true;
        } else {
          lrow = (uint32_t)pg * B + (t - lp * B);
        }
      }
      if (__ballot(bad) != 0 && threadIdx.x == 0) atomicOr(&a.header[0], kErrBlockId);
      vm = __ballot(ok);
    }
    if (fast) {
      // rows row0 .. row0 + nrows - 1 are consecutive: one uniform base plus the lane's
      // precomputed slot offset; slots of rows past the valid prefix re-read row 0 (masked)
      const int nrows = vm ? 64 - __builtin_clzll(vm) : 0;   // valid rows form a prefix
      const char* base = a.lat + (size_t)row0 * kRowBytes;
      const uint32_t lim = (uint32_t)nrows * kRowBytes;
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k) {
        const uint32_t o = slot_off[k] < lim ? slot_off[k] : slot_col[k];
        __builtin_amdgcn_global_load_lds(base + o,
                                         (void DCP_LDS*)(buf + (w * kDmaPerWave + k) * 1024), 16,
                                         0, 0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k) {
        const uint32_t rr = __shfl(lrow, slot_row[k], 64);
        const char* src = a.lat + (size_t)rr * kRowBytes + slot_col[k];
        __builtin_amdgcn_global_load_lds(src, (void DCP_LDS*)(buf + (w * kDmaPerWave + k) * 1024),
                                         16, 0, 0);
      }
    }
    return vm;
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
  // the query must have landed before the copy ring starts: inside the ring the vector
  // memory counter only paces tile copies
  wait_vmcnt<0>();

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

  // per-lane LDS offsets inside a tile
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
  // prologue: three tiles in flight
  uint64_t vm0 = issue_tile(0);
  uint64_t vm1 = ntiles > 1 ? issue_tile(1) : 0ull;
  uint64_t vm2 = ntiles > 2 ? issue_tile(2) : 0ull;

  for (int ti = 0; ti < ntiles; ++ti) {
    // wait for this wave's copies of tile ti (those of tiles ti+1, ti+2 may stay in flight)
    const int pend = min(2, ntiles - 1 - ti);
    if (!fast || pend == 0) wait_vmcnt<0>();
    else if (pend == 1) wait_vmcnt<kDmaPerWave>();
    else wait_vmcnt<2 * kDmaPerWave>();
    // Every wave's copies of tile ti have landed and tile ti-1 is free.  A bare barrier:
    // the fence of __syncthreads would also wait for the copies still in flight.
    asm volatile("s_barrier" ::: "memory");
    uint64_t vm3 = 0ull;
    if (ti + 3 < ntiles) vm3 = issue_tile(ti + 3);
    const char DCP_LDS* buf = lds + (ti % kNBuf) * kTileBytes;

    // ---- scores: s[ht][nt][i] is token 16 nt + 4 g + i of head tile ht
    f4 s[HT][2];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) s[ht][0] = s[ht][1] = f4{0.f, 0.f, 0.f, 0.f};
    // K operands are read kAhead k-steps before the MFMAs that use them: with one wave per
    // SIMD, a step's two MFMAs (32 cycles) cannot cover one LDS round trip by themselves
    bf16x8 kop[kAhead + 1][2];
    auto kread = [&](int ks) {
      const int o = ((ks & 1) ? offk1 : offk0) + 128 * (ks >> 1);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        kop[ks % (kAhead + 1)][nt] =
            *reinterpret_cast<const bf16x8 DCP_LDS*>(buf + nt * 16 * kRowBytes + o);
    };
#pragma unroll
    for (int ks = 0; ks < kAhead; ++ks) kread(ks);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kAhead < kKSteps) kread(ks + kAhead);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          s[ht][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks % (kAhead + 1)][nt],
                                                               qreg[ht][ks], s[ht][nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);   // one scheduling region per k-step
    }

    // ---- online softmax; P (bf16) as the B operand of O^T += V^T P^T, whose k slots
    // 8 g .. 8 g + 7 are tokens 4 g + [0, 4) and 16 + 4 g + [0, 4)
    bf16x8 pb[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = s[ht][0][i] * a.sl2;
        x[4 + i] = s[ht][1][i] * a.sl2;
      }
      if (vm0 != 0xffffffffull) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!((vm0 >> (4 * g + i)) & 1)) x[i] = neg_inf();
          if (!((vm0 >> (16 + 4 * g + i)) & 1)) x[4 + i] = neg_inf();
        }
      }
      float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      // The reference max moves only when a head's tile max exceeds it by more than
      // kRescaleSlack (log2 units): weights stay below 2^kRescaleSlack, exactly
      // representable in bf16/fp32, and the 128-register rescale of the accumulator runs a
      // handful of times per item instead of on most tiles.
      const bool up = tmax > m[ht] + kRescaleSlack;
      const float mn = up ? tmax : m[ht];
      if (__ballot(up) != 0) {
        const float alpha = up ? __builtin_amdgcn_exp2f(m[ht] - mn) : 1.f;
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

    // ---- O^T += V^T P^T (V^T operands read kAhead dim tiles ahead)
    auto vop = [&](int dt) -> bf16x8 {
      const int o = offv[dt & 3] + 128 * (dt >> 2);
      const u32x2 v0 = lds_tr16(buf + o);
      const u32x2 v1 = lds_tr16(buf + 16 * kRowBytes + o);
      return __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
    };
    bf16x8 va[kAhead + 1];
#pragma unroll
    for (int dt = 0; dt < kAhead; ++dt) va[dt] = vop(dt);
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt) {
      if (dt + kAhead < kDvTiles) va[(dt + kAhead) % (kAhead + 1)] = vop(dt + kAhead);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        acc[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt % (kAhead + 1)], pb[ht],
                                                              acc[ht][dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    vm0 = vm1;
    vm1 = vm2;
    vm2 = vm3;
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

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
//   * Two workgroups of 12 waves per work item (request, local token range), each owning 64
//     of the 128 heads (two pairs of 16-head tiles).  The two groups of an item get
//     workgroup ids congruent mod 8, so they run on the same XCD and read each latent tile
//     from HBM once between them (the second read hits that XCD's L2).
//   * Warp specialisation.  Four score waves = (head pair, half of the 576 dims) compute the
//     partial S^T = K . Q^T of both 16-head tiles of their pair (M = 16 tokens, N = 16
//     heads, K = 32 latent dims per MFMA; every K operand read feeds two MFMAs), swap the
//     partial scores of one head tile through LDS and finish the online softmax of the
//     other.  Eight output waves = (head pair, quarter of the 512 value dims) keep O^T in
//     AGPRs and, one tile behind, accumulate O^T += V^T . P^T (M = 16 value dims, N = 16
//     heads, K = 32 tokens), the V^T operand read with ds_read_b64_tr_b16 in the token
//     order of the score registers.  In both products every lane's results belong to one
//     head, so the softmax max needs two cross-lane steps and the weights never move
//     between lanes.
//   * 32-token tiles of latent rows are copied HBM -> LDS by global_load_lds_dwordx4 (no
//     register staging) into a 4-deep ring: two tiles in flight while the score waves work
//     on one and the output waves on the previous one.  The copies are issued from inline
//     assembly and paced by explicit vector-memory counter waits plus a bare s_barrier;
//     the compiler, which does not see them, then has no reason to drain them before LDS
//     reads.  The 16-byte chunks of a row are XOR-swizzled by (row mod 8), which spreads
//     the operand reads over the LDS banks.
//   * When the interleave and the block size are multiples of 32, every tile is one run of
//     consecutive slots in one page, located by one readlane from a per-wave table of tile
//     sources.  Otherwise (the general kernel, down to interleave 1) the cache row of every
//     token of a window of 12 tiles sits in an LDS table that the score waves, which have
//     no copies in flight, build a few tiles ahead; the output waves' copies then read their
//     rows from LDS and stay paced exactly as for page-contiguous tiles.
//   * The running max only moves when a tile's max exceeds it by more than 8 (log2 units);
//     the output waves rescale their accumulators only on such tiles.
//   * Multi-token decode (q_len query positions per request, the last q_len cache tokens
//     being the request's own draft tokens): each work item gets two workgroups per query
//     position, all on one XCD.  Position i sees the positions up to seq_len - q_len + i,
//     a prefix of the shard's local tokens, so its workgroups simply end the item there
//     (possibly before its first tile: an empty partial, lse = -inf).
#include "launch.h"

namespace dcp {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(2))) float f2;
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
constexpr int kHeadTiles = 4;                // 16-head tiles per workgroup (64 heads)
constexpr int kGroups = kHeads / (16 * kHeadTiles);      // head groups (workgroups) per item
constexpr int kQkWaves = 4;                  // score waves: (head pair, half of the 576 dims)
constexpr int kPvWaves = 8;                  // output waves: (head pair, quarter of the 512 dims)
constexpr int kWaves = kQkWaves + kPvWaves;  // 12 waves, three per SIMD
constexpr int kHalfSteps = kKSteps / 2;      // 9 k-steps of 32 dims per score wave
constexpr int kQuarterTiles = kDvTiles / 4;  // 8 dv tiles of 16 dims per output wave
constexpr int kSlotsHi = 5;                  // 1-KiB tile copies per tile: output waves 0..3
constexpr int kSlotsLo = 4;                  // output waves 4..7 (4 x 5 + 4 x 4 = 36 slots)
constexpr int kPhase1Tiles = 2;              // dv tiles of an output wave before the mid barrier
constexpr int kXcds = 8;                     // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr float kRescaleSlack = 8.f;          // see the online softmax below
constexpr int kAheadK = 4;                   // K operand prefetch distance (k-steps)
constexpr int kAheadV = 3;                   // V^T operand prefetch distance (dv tiles)
// LDS: the tile ring; the partial-score exchange [pair][head tile][lane][8 floats]; the
// weights P [head tile][lane][16 B]; the rescale factors and the final normalisation
// [head tile][16] floats
constexpr int kRingBytes = kNBuf * kTileBytes;                  // 147456
constexpr int kXOff = kRingBytes;
constexpr int kPOff = kXOff + kHeadTiles * 64 * 32;             // + 8192
constexpr int kAOff = kPOff + kHeadTiles * 1024;                // + 4096
constexpr int kFOff = kAOff + kHeadTiles * 16 * 4;              // + 256
constexpr int kTOff = kFOff + kHeadTiles * 16 * 4;              // + 256
// general tiles: the cache rows of the tokens of kTWin tiles, built ahead by the score waves
constexpr int kTWin = 12;
constexpr int kLdsBytes = kTOff + kTWin * kTile * 4;            // + 1536 = 161792

struct MlaKArgs {
  const uint16_t* q;
  const char* lat;
  const int32_t* bt;
  int block_size, max_blocks;
  uint32_t num_blocks;
  int rank, cp, interleave;
  float sl2;
  const int32_t* seq_lens;
  int64_t len_cap;
  int q_len;
  int o_bf16;    // O written in bf16 (requests with a single item; others via the combine)
  void* o_out;
  float* lse_out;
  int32_t* header;
  const int32_t* off;
  const int4* items;
  float* plse;
  float* po;
};

// Two floats to a packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x2 lds_tr16(const char DCP_LDS* p) {
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 DCP_LDS*)p);
  return __builtin_bit_cast(u32x2, v);
}


// O^T tile += V^T P^T with the accumulator pinned to AGPRs.  kNop inserts wait states
// first, for an operand written by a VALU op just before (the weights, or a rescaled
// accumulator).  The compiler does not see this as an MFMA, so code that reads an
// accumulator after the last one issues its own wait states (settle_acc).
template <bool kNop>
__device__ __forceinline__ void mfma_acc(f4& acc, const bf16x8& va, const bf16x8& pb) {
  if constexpr (kNop)
    asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(va), "v"(pb));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(va), "v"(pb));
}

__device__ __forceinline__ void wait_lgkm0() {
  // lgkmcnt(0), vector-memory and export counters unconstrained (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// kFast: the interleave and the block size are multiples of the tile, so the 32 tokens of a
// tile are consecutive slots of one cache page.
//
// Warp-specialised workgroup of 12 waves for 64 heads (two pairs of 16-head tiles).  Every
// K / V operand read from LDS feeds two MFMAs (both head tiles of a pair):
//   * score waves 0..3 = (head pair hp = w / 2, half kh = w % 2 of the 576 dims): for tile
//     t, the partial S^T = K Q^T of both head tiles of the pair over their 288 dims
//     (18 K reads, 36 MFMAs).  The two halves swap the partial scores of one head tile
//     through LDS, so each finishes the online softmax of one head tile: running max,
//     bf16 weights P and the factor that rescales the output accumulated so far, handed
//     to the output waves through LDS;
//   * output waves 4..11 = (head pair hp = (w - 4) / 4, quarter dq of the 512 value dims):
//     O^T in AGPRs (both head tiles, 128 dims), one tile behind the score waves,
//     O^T += V^T P^T (16 transposed V reads, 16 MFMAs per tile).
// Waves are dealt round-robin over the SIMDs: each SIMD runs one score wave and two output
// waves (68 MFMAs per tile).  Two barriers per tile: at barrier A of iteration t, tile t
// has landed (copies paced by each wave's own vector-memory counter), P of tile t-1 is in
// LDS and every read of tile t-2 is done, so its buffer takes the copy of tile t+2; at
// barrier B the partial scores of tile t have been swapped.  The output waves split their
// MFMAs over both phases, so the matrix cores stay busy while the softmax runs.
template <bool kFast>
__global__ __launch_bounds__(kWaves * 64, 1) void mla_shard_kernel(MlaKArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  // Workgroup ids: the q_len * kGroups (query position, head group) workgroups of one work
  // item are congruent mod 8 (same XCD) and adjacent in dispatch order.
  const int blk = blockIdx.x;
  const int ngroups = kGroups * a.q_len;
  const int hgq = (blk / kXcds) % ngroups;
  const int qi = hgq / kGroups, hg = hgq - qi * kGroups;
  const int slot = (blk / (kXcds * ngroups)) * kXcds + blk % kXcds;
  if (slot >= a.header[1]) return;
  const int4 it = a.items[slot];   // in dispatch order, longest first
  const int b = it.x, j0 = it.y;
  const int item = it.w;           // index of the item's partial
  // query position qi sees a prefix of the shard's tokens
  const int j1 = a.q_len == 1 ? it.z
                              : min(it.z, row_local_end(a.seq_lens, b, a.len_cap, a.q_len, qi,
                                                        a.rank, a.cp, a.interleave));
  const bool single = (a.off[b + 1] - a.off[b]) == 1;
  // rows of (request b, position qi) and of (item, position qi) in the outputs
  const size_t orow = ((size_t)b * a.q_len + qi) * kHeads;
  const size_t prow = ((size_t)item * a.q_len + qi) * kHeads;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4;      // 16-lane group
  const int i16 = lane & 15;
  const uint32_t B = (uint32_t)a.block_size;
  const int32_t* btb = a.bt + (size_t)b * a.max_blocks;
  const char DCP_LDS* lds = (const char DCP_LDS*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  const bool is_qk = w < kQkWaves;
  const int ntiles = j1 > j0 ? (j1 - j0 + kTile - 1) / kTile : 0;

  // Page-contiguous tiles: a per-wave table of tile sources, lane k holding the first cache
  // row of tile 64 * window + k (or ~0 for a bad page).  It is built by a lane-parallel walk
  // and one gather of block-table entries, once per 64 tiles (the gather's vector-memory
  // wait then drains the copies in flight, once per window), so locating a tile is one
  // readlane: no scalar memory load inside the tile loop, whose counter the LDS operand
  // waits share.
  struct TileSrc {
    const char* base;   // global address of the tile's first row
    uint32_t lim;       // bytes of valid rows (slots past them re-read row 0, masked)
    bool full;          // all 32 rows valid
  };
  uint32_t row_tab = 0;
  auto build_table = [&](int win) {
    const int tt = win * 64 + lane;
    bool bad = false;
    uint32_t row = ~0u;
    if (tt < ntiles) {
      const uint32_t t = dcp_walk_global_pos((uint32_t)(j0 + tt * kTile), a.rank, a.cp,
                                             a.interleave);
      const uint32_t lp = t / B;
      const int32_t pg = btb[lp];
      if (pg < 0 || (uint32_t)pg >= a.num_blocks) bad = true;
      else row = (uint32_t)pg * B + (t - lp * B);
    }
    if (__ballot(bad) != 0 && threadIdx.x == 0) atomicOr(&a.header[0], kErrBlockId);
    row_tab = row;
  };
  if constexpr (kFast) build_table(0);
  uint64_t vm_new = 0;
  // source of tile ti
  auto tile_src = [&](int ti) -> TileSrc {
    if ((ti & 63) == 0 && ti > 0) build_table(ti >> 6);
    const int nvalid = min(kTile, j1 - (j0 + ti * kTile));
    const uint32_t row0 = __builtin_amdgcn_readlane(row_tab, ti & 63);
    const bool ok = row0 != ~0u;
    TileSrc ts;
    ts.base = a.lat + (size_t)(ok ? row0 : 0u) * kRowBytes;
    ts.full = ok && nvalid == kTile;
    ts.lim = ok ? (uint32_t)nvalid * kRowBytes : 0u;
    vm_new = ts.full ? 0xffffffffull : (ok ? ((1ull << nvalid) - 1) : 0ull);
    return ts;
  };
  // mask of valid rows of tile ti (page-contiguous tiles: from the source table)
  // General tiles: the cache row of every token of a window of kTWin tiles sits in LDS
  // (~0 for no token or a bad page).  The score waves, which have no copies in flight,
  // walk the tokens and load the block-table entries (gen_load) and store the rows
  // (gen_store) a few tiles before the window is first used, so no block-table load ever
  // waits inside the output waves, whose copies stay paced by the counter alone.
  uint32_t DCP_LDS* const rowtab = (uint32_t DCP_LDS*)(smem + kTOff);
  uint32_t gen_t[2];
  int32_t gen_pg[2];
  bool gen_ok[2];
  auto gen_load = [&](int win) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int e = pass * (kQkWaves * 64) + w * 64 + lane;   // entry of the window
      const int j = j0 + win * kTWin * kTile + e;
      gen_ok[pass] = e < kTWin * kTile && j < j1;
      gen_t[pass] = 0;
      gen_pg[pass] = 0;
      if (gen_ok[pass]) {
        gen_t[pass] = dcp_walk_global_pos((uint32_t)j, a.rank, a.cp, a.interleave);
        gen_pg[pass] = btb[gen_t[pass] / B];
      }
    }
  };
  auto gen_store = [&]() {
    bool bad = false;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int e = pass * (kQkWaves * 64) + w * 64 + lane;
      if (e < kTWin * kTile) {
        uint32_t row = ~0u;
        if (gen_ok[pass]) {
          const uint32_t lp = gen_t[pass] / B;
          if (gen_pg[pass] < 0 || (uint32_t)gen_pg[pass] >= a.num_blocks) bad = true;
          else row = (uint32_t)gen_pg[pass] * B + (gen_t[pass] - lp * B);
        }
        rowtab[e] = row;
      }
    }
    if (__ballot(bad) != 0 && lane == 0) atomicOr(&a.header[0], kErrBlockId);
  };
  // mask of valid rows of tile ti
  auto tile_mask = [&](int ti) -> uint64_t {
    if constexpr (kFast) {
      (void)tile_src(ti);
      return vm_new;
    } else {
      const bool ok = lane < kTile && rowtab[(ti % kTWin) * kTile + (lane & (kTile - 1))] != ~0u;
      return __ballot(ok);
    }
  };
  if constexpr (!kFast) {
    // window 0 before any copy
    if (is_qk) {
      gen_load(0);
      gen_store();
    }
    wait_lgkm0();
    asm volatile("s_barrier" ::: "memory");
  }

  if (is_qk) {
    // ================= score wave: head pair hp, dims 288 kh .. + 288 =================
    const int hp = w >> 1, kh = w & 1;
    const int own = 2 * hp + kh;   // local head tile whose softmax this wave finishes
    // Barrier A of iteration t (both roles run ntiles + 1 iterations; the output waves'
    // copies of tile t have landed).  Bare barriers: the fence of __syncthreads would also
    // wait for the copies still in flight.
    uint64_t vm0 = tile_mask(0);
    uint64_t vm1 = ntiles > 1 ? tile_mask(1) : 0ull;
    uint64_t vm2 = 0ull;
    auto barrier_a = [&](int t) {
      asm volatile("s_barrier" ::: "memory");
      vm2 = t + 2 < ntiles ? tile_mask(t + 2) : 0ull;
    };

    const int head_p = 16 * (kHeadTiles * hg + 2 * hp) + i16;   // lane's head, tile 2 hp
    // query (B operand of S^T = K Q^T): qreg[hh][j] = dims 32 (9 kh + j) + 8 g .. + 8 of
    // head tile 2 hp + hh
    bf16x8 qreg[2][kHalfSteps];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint16_t* qrow =
          a.q + (orow + head_p + 16 * hh) * kDk + 8 * g + 32 * kHalfSteps * kh;
#pragma unroll
      for (int j = 0; j < kHalfSteps; ++j)
        qreg[hh][j] = *reinterpret_cast<const bf16x8*>(qrow + 32 * j);
    }
    // the query must have landed before the copy ring is paced by the counter alone
    wait_vmcnt<0>();
    // The query lives in AGPRs (the MFMAs read their B operand from there), leaving the
    // VGPRs to the operand ring: both roles then fit three waves per SIMD.
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int j = 0; j < kHalfSteps; ++j) asm volatile("" : "+a"(qreg[hh][j]));
    float m = neg_inf();   // running max (log2 units) of this lane's head of tile `own`
    float negm = 0.f;      // -m, or 0 while m is -inf
    float ls = 0.f;        // this lane's share of the running sum of weights
    const int xk = i16 & 7;
    const int offk0 = i16 * kRowBytes + 16 * (g ^ xk);
    const int offk1 = i16 * kRowBytes + 16 * ((4 + g) ^ xk);
    // partial scores: written for the partner's head tile, read for the own one
    f4 DCP_LDS* xdst = (f4 DCP_LDS*)(smem + kXOff) + ((2 * hp + 1 - kh) * 64 + lane) * 2;
    const f4 DCP_LDS* xsrc = (const f4 DCP_LDS*)(smem + kXOff) + (own * 64 + lane) * 2;
    u32x4 DCP_LDS* pdst = (u32x4 DCP_LDS*)(smem + kPOff) + own * 64 + lane;
    float DCP_LDS* adst = (float DCP_LDS*)(smem + kAOff) + own * 16 + i16;

    // Iteration t: phase 1 = tile t's partial scores (MFMAs) and the swap; phase 2 (after
    // barrier B) = the online softmax of the own head tile and the hand-over of P.
    for (int t = 0; t <= ntiles; ++t) {
      wait_lgkm0();   // the previous tile's weights are in LDS before the barrier
      barrier_a(t);
      // general tiles: the window of tiles t+3 .. is built in this iteration (its first
      // tile is first read at barrier A of the next one)
      const bool gen_now = !kFast && (t + 3) % kTWin == 0 && t + 3 < ntiles;
      if (gen_now) gen_load((t + 3) / kTWin);
      f4 sm0 = {0.f, 0.f, 0.f, 0.f}, sm1 = {0.f, 0.f, 0.f, 0.f};   // own head tile
      if (t < ntiles) {
        const char DCP_LDS* tb = lds + (t % kNBuf) * kTileBytes;
        // s[tt][hh]: token half tt, head tile 2 hp + hh (four independent MFMA chains)
        f4 s[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) s[tt][hh] = f4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kop[kAheadK + 1][2];
        auto kread = [&](int j) {
          const int ks = kHalfSteps * kh + j;
          const int o = ((ks & 1) ? offk1 : offk0) + 128 * (ks >> 1);
          kop[j % (kAheadK + 1)][0] = *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + o);
          kop[j % (kAheadK + 1)][1] =
              *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + 16 * kRowBytes + o);
        };
#pragma unroll
        for (int j = 0; j < kAheadK; ++j) kread(j);
#pragma unroll
        for (int j = 0; j < kHalfSteps; ++j) {
          if (j + kAheadK < kHalfSteps) kread(j + kAheadK);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              s[tt][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j % (kAheadK + 1)][tt],
                                                                  qreg[hh][j], s[tt][hh], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // hand the partner's head tile over; keep the own one
        xdst[0] = kh ? s[0][0] : s[0][1];
        xdst[1] = kh ? s[1][0] : s[1][1];
        sm0 = kh ? s[0][1] : s[0][0];
        sm1 = kh ? s[1][1] : s[1][0];
      }
      wait_lgkm0();   // the partial scores are in LDS before the mid barrier
      asm volatile("s_barrier" ::: "memory");   // barrier B
      // every wave has read the table entries of tile t+2 (at barrier A): the old window is
      // done with
      if (gen_now) gen_store();
      if (t < ntiles) {
        const f4 s0 = sm0 + xsrc[0];
        const f4 s1 = sm1 + xsrc[1];
        // scores: x[i] is token 4 g + i, x[4 + i] token 16 + 4 g + i; masked rows -> -inf
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = s0[i];
          x[4 + i] = s1[i];
        }
        if ((uint32_t)vm0 != 0xffffffffu) {   // partial tile (uniform); the empty asm keeps
          asm volatile("");                   // the masking a branch
          const uint32_t lo = (uint32_t)(vm0 >> (4 * g)) & 0xFu;
          const uint32_t hi = (uint32_t)(vm0 >> (16 + 4 * g)) & 0xFu;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = ((lo >> i) & 1u) ? x[i] : neg_inf();
            x[4 + i] = ((hi >> i) & 1u) ? x[4 + i] : neg_inf();
          }
        }
        // tile max of this lane's head: within the lane, then across the four 16-lane
        // rows (which hold the same head) with two swaps
        float tm = max_f(max_f(max_f(x[0], x[1]), max_f(x[2], x[3])),
                         max_f(max_f(x[4], x[5]), max_f(x[6], x[7])));
        {
          const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tm),
                                                             __float_as_uint(tm), false, false);
          tm = max_f(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
          const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm),
                                                             __float_as_uint(tm), false, false);
          tm = max_f(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
        }
        const float tmax = tm * a.sl2;
        // The running max only moves when a head's tile max exceeds it by more than
        // kRescaleSlack (always on the first tile with valid tokens).  Between raises the
        // weights stay below 2^kRescaleSlack, exactly representable in bf16 / fp32, and
        // the final normalisation by the running sum is exact either way.
        const bool up = tmax > m + kRescaleSlack;
        const float alpha = up ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;   // m = -inf -> 0
        if (up) {
          m = tmax;
          negm = -tmax;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(fmaf(x[i], a.sl2, negm));
        ls = ls * alpha + (((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7])));
        // B operand of O^T += V^T P^T: k slots 8 g .. 8 g + 7 = tokens 4 g + [0, 4) and
        // 16 + 4 g + [0, 4); the output lanes with the same index read these 16 bytes
        *pdst = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
        if (g == 0) *adst = alpha;
      }
      vm0 = vm1;
      vm1 = vm2;
    }
    // ---- per-head normalisation for the output waves, and the lse
    float lt = ls;
    {
      const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lt), __float_as_uint(lt),
                                                         false, false);
      lt = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
      const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt),
                                                         false, false);
      lt = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : neg_inf();
    if (g == 0) {
      const int head = head_p + 16 * kh;
      ((float DCP_LDS*)(smem + kFOff))[own * 16 + i16] = inv;
      if (single) a.lse_out[orow + head] = lse;
      else a.plse[prow + head] = lse;
    }
    wait_lgkm0();
    asm volatile("s_barrier" ::: "memory");
  } else {
    // ============ output wave: head pair hp, value dims 128 dq .. + 128 ============
    const int pv = w - kQkWaves;
    const int hp = pv >> 2, dq = pv & 3;
    // ---- HBM -> LDS tile copies, all issued by the output waves.  A tile is 36 slots of
    // 1 KiB (64 lanes x 16 B); slot s, lane l holds chunk (q mod 72) ^ (row & 7) of tile row
    // q / 72, q = 64 s + l.  Output wave p copies 5 slots from 5p (p < 4) or 4 slots from
    // 20 + 4 (p - 4).
    const int pvw = w - kQkWaves;
    const int slot0 = pvw < 4 ? kSlotsHi * pvw : 4 * kSlotsHi + kSlotsLo * (pvw - 4);
    const int nslots = is_qk ? 0 : (pvw < 4 ? kSlotsHi : kSlotsLo);
    uint32_t slot_off[kSlotsHi], slot_col[kSlotsHi];
    int slot_row[kSlotsHi];
#pragma unroll
    for (int k = 0; k < kSlotsHi; ++k) {
      const int sl = max(slot0 + k, 0) * 64 + lane;
      const int r = min(sl / kRowChunks, kTile - 1);   // slots a wave does not copy: unused
      slot_row[k] = r;
      slot_col[k] = (uint32_t)(((sl - r * kRowChunks) ^ (r & 7)) * 16);
      slot_off[k] = (uint32_t)r * kRowBytes + slot_col[k];
    }
    // all of this wave's copies of tile ti; returns the mask of valid rows
    auto issue_tile = [&](int ti) -> uint64_t {
      const uint32_t dst = lds_addr + (uint32_t)((ti % kNBuf) * kTileBytes + slot0 * 1024);
      if constexpr (kFast) {
        const TileSrc ts = tile_src(ti);
#pragma unroll
        for (int k = 0; k < kSlotsHi; ++k) {
          if (k < nslots) {
            const uint32_t voff =
                ts.full ? slot_off[k] : (slot_off[k] < ts.lim ? slot_off[k] : slot_col[k]);
            copy16_sbase<false>(dst + k * 1024, voff, ts.base);
          }
        }
        return vm_new;
      } else {
        // general tiles: each copy takes the row of its token from the LDS table (rows
        // without a valid token re-read row 0; their tokens are masked)
        const uint32_t DCP_LDS* tr = rowtab + (ti % kTWin) * kTile;
#pragma unroll
        for (int k = 0; k < kSlotsHi; ++k) {
          if (k < nslots) {
            const uint32_t r = tr[slot_row[k]];
            const uint32_t rr = r == ~0u ? 0u : r;
            copy16_vaddr<false>(dst + k * 1024, a.lat + (size_t)rr * kRowBytes + slot_col[k]);
          }
        }
        return 0ull;
      }
    };

    // prologue: tiles 0 and 1 in flight
    if (ntiles > 0) (void)issue_tile(0);
    if (ntiles > 1) (void)issue_tile(1);

    // Barrier A of iteration t: this wave's copies of tile t have landed (those of tile t+1
    // may still fly), then every wave's have; tile t+2 starts.  Bare barriers: the fence of
    // __syncthreads would also wait for the copies still in flight.
    auto barrier_a = [&](int t) {
      if (t < ntiles) {
        if (t + 1 < ntiles) {
          if (nslots == kSlotsHi) wait_vmcnt<kSlotsHi>();
          else wait_vmcnt<kSlotsLo>();
        } else {
          wait_vmcnt<0>();
        }
      }
      asm volatile("s_barrier" ::: "memory");
      if (t + 2 < ntiles) (void)issue_tile(t + 2);
    };


    const int head_p = 16 * (kHeadTiles * hg + 2 * hp) + i16;   // lane's head, tile 2 hp
    // Every definition of an accumulator comes out of an AGPR-constrained asm statement,
    // so the register allocator keeps the loop-carried accumulators in AGPRs.
    f4 acc[2][kQuarterTiles];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < kQuarterTiles; ++i) {
        acc[hh][i] = f4{0.f, 0.f, 0.f, 0.f};
        asm volatile("" : "+a"(acc[hh][i]));
      }
    // Wait states between the last accumulator MFMAs and VALU reads of the accumulators;
    // every accumulator passes through an AGPR-constrained statement here, so the reads
    // cannot be hoisted above it.
    auto settle_acc = [&]() {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+a"(acc[0][4]), "+a"(acc[0][5]), "+a"(acc[0][6]), "+a"(acc[0][7]),
                     "+a"(acc[1][4]), "+a"(acc[1][5]), "+a"(acc[1][6]), "+a"(acc[1][7]));
      asm volatile(""
                   : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]),
                     "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]));
    };
    // V^T operand (A of O^T = V^T P^T) for value-dim tile dt of this wave's quarter
    const int rv = 4 * g + (i16 >> 2);
    const int xv = rv & 7;
    const int qv = (i16 >> 1) & 1;
    int offv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      offv[u] = rv * kRowBytes + 16 * ((2 * u + qv) ^ xv) + (i16 & 1) * 8 + dq * 256;
    const u32x4 DCP_LDS* psrc = (const u32x4 DCP_LDS*)(smem + kPOff) + 2 * hp * 64 + lane;
    const float DCP_LDS* asrc = (const float DCP_LDS*)(smem + kAOff) + 2 * hp * 16 + i16;

    // Iteration t: phase 1 = P of tile t-1 (written by the score waves in phase 2 of the
    // previous iteration), the rescale, and the first kPhase1Tiles dv tiles; phase 2 = the
    // other dv tiles, while the score waves run the softmax.
    for (int t = 0; t <= ntiles; ++t) {
      barrier_a(t);
      const int u = t - 1;
      const char DCP_LDS* tb = lds + ((u + kNBuf) % kNBuf) * kTileBytes;
      auto vop = [&](int dt) -> bf16x8 {
        const int o = offv[dt & 3] + 128 * (dt >> 2);
        const u32x2 v0 = lds_tr16(tb + o);
        const u32x2 v1 = lds_tr16(tb + 16 * kRowBytes + o);
        return __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
      };
      bf16x8 pb0, pb1;
      bf16x8 va[kAheadV + 1];
      if (t >= 1) {
        pb0 = __builtin_bit_cast(bf16x8, psrc[0]);
        pb1 = __builtin_bit_cast(bf16x8, psrc[64]);
        const float alpha0 = asrc[0], alpha1 = asrc[16];
#pragma unroll
        for (int dt = 0; dt < kAheadV; ++dt) va[dt] = vop(dt);
        if (__ballot(alpha0 != 1.f || alpha1 != 1.f) != 0) {
          settle_acc();
#pragma unroll
          for (int i = 0; i < kQuarterTiles; ++i) {
            acc[0][i] *= alpha0;
            acc[1][i] *= alpha1;
            asm volatile("" : "+a"(acc[0][i]), "+a"(acc[1][i]));
          }
        }
#pragma unroll
        for (int dt = 0; dt < kPhase1Tiles; ++dt) {
          if (dt + kAheadV < kQuarterTiles) va[(dt + kAheadV) % (kAheadV + 1)] = vop(dt + kAheadV);
          if (dt == 0) mfma_acc<true>(acc[0][dt], va[dt % (kAheadV + 1)], pb0);
          else mfma_acc<false>(acc[0][dt], va[dt % (kAheadV + 1)], pb0);
          mfma_acc<false>(acc[1][dt], va[dt % (kAheadV + 1)], pb1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      asm volatile("s_barrier" ::: "memory");   // barrier B
      if (t >= 1) {
#pragma unroll
        for (int dt = kPhase1Tiles; dt < kQuarterTiles; ++dt) {
          if (dt + kAheadV < kQuarterTiles) va[(dt + kAheadV) % (kAheadV + 1)] = vop(dt + kAheadV);
          mfma_acc<false>(acc[0][dt], va[dt % (kAheadV + 1)], pb0);
          mfma_acc<false>(acc[1][dt], va[dt % (kAheadV + 1)], pb1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    asm volatile("s_barrier" ::: "memory");
    // ---- finalize: lane holds dims 128 dq + 16 dt + 4 g + [0, 4) of its heads
    const float inv0 = ((const float DCP_LDS*)(smem + kFOff))[2 * hp * 16 + i16];
    const float inv1 = ((const float DCP_LDS*)(smem + kFOff))[(2 * hp + 1) * 16 + i16];
    settle_acc();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int head = head_p + 16 * hh;
      float* dst = (single ? static_cast<float*>(a.o_out) + (orow + head) * kDv
                           : a.po + (prow + head) * kDv) +
                   dq * 128;
      uint16_t* dstb = static_cast<uint16_t*>(a.o_out) + (orow + head) * kDv + dq * 128;
      const float inv = hh ? inv1 : inv0;
      if (single && a.o_bf16) {   // uniform
#pragma unroll
        for (int dt = 0; dt < kQuarterTiles; ++dt) {
          const f4 v = acc[hh][dt] * inv;
          *reinterpret_cast<uint2*>(dstb + 16 * dt + 4 * g) =
              make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                         f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < kQuarterTiles; ++dt) {
          const f4 v = acc[hh][dt] * inv;
          *reinterpret_cast<f4*>(dst + 16 * dt + 4 * g) = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_mla_shard(const MlaArgs& a, int64_t max_items, const WsPtrs& ws,
                            void* o_out, float* lse_out, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1) {
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
  k.seq_lens = a.rows.seq_lens;
  k.len_cap = a.rows.len_cap;
  k.q_len = a.rows.q_len;
  k.o_bf16 = a.o_bf16;
  k.o_out = o_out;
  k.lse_out = lse_out;
  k.header = ws.header;
  k.off = ws.off;
  k.items = ws.items;
  k.plse = ws.plse;
  k.po = ws.po;
  const int64_t groups8 = (max_items + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(groups8 * kXcds * kGroups * a.rows.q_len));
  const bool fast = (a.interleave % kTile) == 0 && (a.block_size % kTile) == 0;
  if (fast)
    hipExtLaunchKernelGGL(mla_shard_kernel<true>, grid, dim3(kWaves * 64), 0, stream, ev0, ev1, 0,
                          k);
  else
    hipExtLaunchKernelGGL(mla_shard_kernel<false>, grid, dim3(kWaves * 64), 0, stream, ev0, ev1,
                          0, k);
  return hipGetLastError();
}

}  // namespace dcp

// mla_shard.hip — paged MLA decode attention over one DCP rank's shard, on bf16 MFMA.
//
// What it computes ("vLLM Decode Context Parallelism for long-context workloads" blog,
// "DCP execution flow", step "Compute", and "The memory wall in long-context inference",
// MLA item: all query heads share one low-rank latent KV row): for every request b and
// each of the H gathered query heads h (H = 128, or 64, 32, 16 for smaller DCP groups),
// attention over the tokens this rank owns, with key = the token's 576-wide latent row and
// value = its first 512 columns, plus the natural-log LSE of the scaled scores.
//
// Per token at 128 heads this is 128 x (576 + 512) multiply-adds against 1152 bytes of
// cache: a dense contraction (about 242 flop/byte, just below the bf16 ridge of MI355X), so
// both products run on v_mfma_f32_16x16x32_bf16 and the kernel has to keep the HBM stream
// and the matrix cores busy at the same time.
//
// Design (described at 128 heads; fewer heads give each wave one 16-head tile, H / 4 of its
// columns real):
//   * One workgroup of four waves (one per SIMD) per work item (request, local token range)
//     and query position, holding all heads, so each latent tile is copied from HBM into
//     LDS exactly once.  Wave w owns heads 32 w .. 32 w + 31 (two 16-head tiles) from end
//     to end: its query lives in 144 VGPRs and its O^T accumulators (32 heads x 512 dims,
//     float32) in all 256 AGPRs, so no score, weight or rescale factor ever moves between
//     waves.
//   * S^T = K Q^T per 16 tokens x 16 heads on v_mfma_f32_16x16x32_bf16 (K operand: one
//     16-byte LDS read per lane feeding the MFMAs of both head tiles); the lane holding
//     head i16 and tokens 4 g .. 4 g + 3 of each 16-token half then holds, packed to bf16,
//     exactly the P^T operand of O^T += V^T P^T on the same instruction (32 tokens per
//     MFMA), whose V^T operand is two ds_read_b64_tr_b16 per 16 value dims, again feeding
//     both head tiles.  Per 32-token tile a wave issues 72 + 64 MFMAs against 36 + 64 LDS
//     operand reads.
//   * Software pipeline: iteration t runs the MFMAs of S^T for tile t + 1 while the online
//     softmax of tile t (already in registers) runs on the vector ALUs between them, then
//     O^T += V^T P^T of tile t.  The running max moves only when a tile's max exceeds it by
//     more than 8 (log2 units); the accumulators are rescaled (a rare branch) only then.
//   * 32-token tiles of latent rows (36 KiB) are copied HBM -> LDS by
//     global_load_lds_dwordx4 (no register staging) into a 4-deep ring: tiles t and t + 1
//     are read while t + 2 and t + 3 are in flight.  The copies are issued from inline
//     assembly between the O^T MFMAs (all four waves, 9 KiB each per tile), paced by the
//     waves' vector-memory counters and a bare s_barrier per tile, so the compiler never
//     drains them before LDS reads.  The 16-byte chunks of a row are XOR-swizzled by
//     (row mod 8), which spreads the operand reads over the LDS banks.
//   * Where each tile comes from is read from a table in LDS, built a window ahead.  When
//     the interleave and the block size are multiples of 32, a tile is one run of
//     consecutive slots of one page and the table holds its first cache row (64 tiles per
//     window, one pass built by wave 3); otherwise (down to interleave 1) it holds the cache
//     row of every token (12 tiles per window, six passes spread over the four waves and
//     six iterations).  A wave stages its block-table entries just before its own copies of
//     the next tile, so the per-tile counter wait covers them (no drain).
//   * Multi-token decode (q_len query positions per request, the last q_len cache tokens
//     being the request's own draft tokens): each work item gets one workgroup per query
//     position, all on one XCD (the later ones read the tiles from L2).  Position i sees
//     the positions up to seq_len - q_len + i, a prefix of the shard's local tokens, so its
//     workgroup ends the item there (possibly before its first tile: an empty partial).
//   * A request whose shard is one work item gets (O, lse) written directly; otherwise
//     each item writes its normalized partial output in bf16 (rounded to nearest even)
//     with its float32 LSE, and the split combine merges them.
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

constexpr int kMaxHeads = 128;                 // 4 waves x 2 head tiles of 16
constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kTile = kMlaTile;                // 32 tokens per tile
constexpr int kNBuf = 4;                       // LDS tile ring
constexpr int kRowBytes = kDk * 2;             // 1152
constexpr int kRowChunks = kRowBytes / 16;     // 72
constexpr int kTileBytes = kTile * kRowBytes;  // 36 KiB
constexpr int kKSteps = kDk / 32;              // 18 k-steps of S^T = K Q^T
constexpr int kDvTiles = kDv / 16;             // 32 value-dim tiles of O^T
constexpr int kWaves = 4;                      // H / 4 heads each (32 at 128 heads)
constexpr int kBuilder = 3;                    // wave 3 builds window 0 and page-run tables
constexpr int kSlots = kTileBytes / 1024;      // 36 one-KiB copies per tile
// All four waves copy every tile (9 one-KiB copies each), the table builders included: a
// wave's block-table entries are staged before its copies of the next tile and
// vector-memory loads complete in order, so the wait that lets the next tile's copies stay
// in flight also covers the staged entries (no drain at a window build).  Against one
// builder wave that copied nothing on fine interleaves (waves 0..2 taking 12 copies each)
// and drained its copies at every window build, measured on MI355X: 197.1 -> 180.1 us at
// interleave 1 and 169.3 -> 161.7 us at interleave 64 (MLA decode shape, median of 40
// interleaved launches); spreading the per-token window build over the four waves and
// reading each copy's row one copy ahead then took interleave 1 from 191.0 to 183.2 us
// (5626 -> 5076 cycles per tile and wave).
constexpr int kCopyWaves = kWaves;
constexpr int kXcds = 8;                       // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr float kRescaleSlack = 8.f;
// K operand prefetch distance (k-steps): 3 where the registers allow it (the page-contiguous
// path); the general path keeps more table state live and stays at 2 to avoid spills
template <bool kFast> constexpr int ahead_k() { return kFast ? 3 : 2; }
// V^T operand prefetch distance (dv tiles): up to 14 transposed LDS reads in flight per wave
// (the counter's limit is 15).  Measured on MI355X at the MLA decode shape, 60 interleaved
// launches each: 171.5 -> 166.1 us against 3 tiles ahead (175.0 -> 170.6 us on another box);
// K prefetch beyond 3 k-steps spills and gains nothing.
constexpr int kAheadV = 7;
// tile tables: two windows; page-contiguous tiles keep one entry (first row) per tile and
// 64 tiles per window, general tiles one entry (row) per token and 12 tiles per window
constexpr int kFastWin = 64;
constexpr int kGenWin = 12;
constexpr int kWinEntries = kGenWin * kTile;   // 384 >= kFastWin
constexpr int kRingBytes = kNBuf * kTileBytes;  // 147456
constexpr int kTabOff = kRingBytes;
constexpr int kStageOff = kTabOff + 2 * kWinEntries * 4;   // + 3072: block-table entries
constexpr int kSlotOff = kStageOff + kWinEntries * 4;      // + 1536: copy offsets per thread
constexpr int kLdsBytes = kSlotOff + kWaves * 64 * 32;     // + 8192 = 160256
static_assert(kSlots % kCopyWaves == 0, "copy slots");
static_assert(kGenWin > 4 && kFastWin > 4, "a window is built before its first copy");

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
  int heads;     // query heads H (rows per position): 16, 32, 64 or 128
  int hpw;       // heads per wave, H / 4
  int o_bf16;    // O written in bf16 (requests with a single item; others via the combine)
  void* o_out;
  float* lse_out;
  int32_t* header;
  const int32_t* off;
  const int4* items;
  float* plse;
  uint16_t* po;  // bf16 split partials
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
// first, for an accumulator a VALU op may have just rewritten (the rescale).  The compiler
// does not see this as an MFMA, so code that reads an accumulator after the last one
// issues its own wait states (settle below).
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
// tile are consecutive slots of one cache page.  kNt: the tile copies take the non-temporal
// cache policy (one workgroup per item reads each tile: q_len = 1).
//
// One wave issues its MFMAs in order, and a 16x16x32 MFMA leaves room for about two simple
// vector instructions (or one exp2) beside it without slowing the matrix core (measured on
// MI355X).  So the softmax of a tile is cut into 18 pieces of that size, one per k-step of
// the next tile's S^T, and the tile copies are issued between the O^T MFMAs.
//
// HT: 16-head tiles per wave (2 for 128 heads, 1 for 64 or fewer; a wave with fewer than 16
// heads pads its tile: the padding columns load a valid head's query and are never written).
template <bool kFast, bool kNt, int HT>
__global__ __launch_bounds__(kWaves * 64, 1) void mla_shard_kernel(MlaKArgs a) {
  static_assert(HT == 1 || HT == 2, "head tiles per wave");
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  // Workgroup ids (dealt round-robin over the 8 XCDs): the q_len workgroups (query
  // positions) of one work item are congruent mod 8, and so are four consecutive work items
  // (in dispatch order the full items of one request are consecutive): they share one XCD's
  // L2 for the tiles and the query.  blk = 32 q_len a + 8 (4 qi + c) + x runs item
  // 32 a + 4 x + c, position qi.
  const int blk = blockIdx.x;
  const int x8 = blk % kXcds;
  const int grp = (blk / kXcds) % (4 * a.q_len);
  const int qi = grp / 4;
  const int slot = (blk / (kXcds * 4 * a.q_len)) * (kXcds * 4) + 4 * x8 + grp % 4;
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
  const size_t orow = ((size_t)b * a.q_len + qi) * a.heads;
  const size_t prow = ((size_t)item * a.q_len + qi) * a.heads;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4;      // 16-lane group
  const int i16 = lane & 15;
  const uint32_t B = (uint32_t)a.block_size;
  const int32_t* btb = a.bt + (size_t)b * a.max_blocks;
  const char DCP_LDS* lds = (const char DCP_LDS*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  const int ntiles = j1 > j0 ? (j1 - j0 + kTile - 1) / kTile : 0;
  constexpr int kSlotsPerWave = kSlots / kCopyWaves;
  const bool copier = w < kCopyWaves;

  // ---- tile tables: window W in half W & 1 of the table.  stage_pass(W, p) copies the
  // block-table entries of 64 of window W's tokens (page-contiguous: of each tile's first
  // token) into LDS by global_load_lds_dword; commit_pass(W, p), one iteration later and by
  // the same wave, turns them into cache rows (~0 for no token or a bad page).  In the tile
  // loop the staged entries go out at the top of an iteration, before that wave's copies of
  // tile t + 3, so the next iteration's wait (everything but those copies) covers them.
  constexpr int kWin = kFast ? kFastWin : kGenWin;
  constexpr int kPasses = kFast ? 1 : kWinEntries / 64;   // 64 entries per pass
  uint32_t DCP_LDS* const tab = (uint32_t DCP_LDS*)(smem + kTabOff);
  const int32_t DCP_LDS* const stage = (const int32_t DCP_LDS*)(smem + kStageOff);
  auto tab_entry = [&](int k, int i) -> uint32_t DCP_LDS* {
    return tab + ((k / kWin) & 1) * kWinEntries + (k % kWin) * (kFast ? 1 : kTile) + i;
  };
  // entry e of window W: its tile and token, whether it exists, its global position t
  auto entry_pos = [&](int W, int e, uint32_t& t) -> bool {
    const int tile = W * kWin + (kFast ? e : e / kTile);
    const int j = j0 + tile * kTile + (kFast ? 0 : e % kTile);
    const bool valid = (!kFast || e < kWin) && tile < ntiles && j < j1;
    t = valid ? dcp_walk_global_pos((uint32_t)j, a.rank, a.cp, a.interleave) : 0u;
    return valid;
  };
  // (the passes stay a loop: unrolled, their walks would be scheduled together and need
  // registers the tile loop does not have)
  auto stage_pass = [&](int W, int p) {
    uint32_t t;
    const bool valid = entry_pos(W, p * 64 + lane, t);
    const int32_t* src = btb + (valid ? t / B : 0u);
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "{m0}"(lds_addr + kStageOff + p * 256)
                 : "memory");
  };
  auto commit_pass = [&](int W, int p) {   // the staged entries have landed (see the callers)
    const int e = p * 64 + lane;
    uint32_t t;
    uint32_t row = ~0u;
    bool bad = false;
    if (entry_pos(W, e, t)) {
      const int32_t pg = stage[e];
      if (pg < 0 || (uint32_t)pg >= a.num_blocks) bad = true;
      else row = (uint32_t)pg * B + (t - (t / B) * B);
    }
    if (!kFast || e < kWin)
      *tab_entry(W * kWin + (kFast ? e : e / kTile), kFast ? 0 : e % kTile) = row;
    if (__ballot(bad) != 0 && lane == 0) atomicOr(&a.header[0], kErrBlockId);
  };

  // ---- copies (the copier waves): slot s = kSlotsPerWave w + k of a tile, lane l holds LDS
  // bytes 16 (64 s + l) of the tile = row r = (64 s + l) / 72, position c = (64 s + l) mod
  // 72, which receives the row's chunk c ^ (r & 7).  The byte offset of slot k's source
  // chunk within the tile (< 2^16) is a 16-bit entry of a per-thread LDS record (the tile
  // loop has no registers to spare for them).
  uint16_t DCP_LDS* const slot_rec = (uint16_t DCP_LDS*)(smem + kSlotOff) + threadIdx.x * 16;
  if (copier) {
#pragma unroll
    for (int k = 0; k < kSlotsPerWave; ++k) {
      const int q = (kSlotsPerWave * w + k) * 64 + lane;
      const int r = q / kRowChunks;
      slot_rec[k] = (uint16_t)(r * kRowBytes + ((q - r * kRowChunks) ^ (r & 7)) * 16);
    }
  }
  // The copies of one tile: plan() reads where the tile comes from (and this thread's slot
  // offsets), copy(k) issues slot k.
  struct TileCopy {
    uint32_t so[(kSlotsPerWave + 1) / 2];   // slot offsets, two per register
    const char* base;                 // page-contiguous tiles: the tile's first row
    uint32_t dst;                     // LDS address of this wave's first slot
    int nvalid;                       // page-contiguous tiles: rows holding tokens
    int ti;                           // the tile (general tiles: its rows are in the table)
    uint32_t row;                     // general tiles: the row of the next copy's token
    __device__ uint32_t off(int k) const { return (k & 1) ? so[k / 2] >> 16 : so[k / 2] & 0xffffu; }
  };
  auto plan_copy = [&](int ti) -> TileCopy {
    TileCopy c;
    const u32x4 lo = *(const u32x4 DCP_LDS*)slot_rec;
    const u32x2 hi = *(const u32x2 DCP_LDS*)(slot_rec + 8);
    const uint32_t all[6] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y};
#pragma unroll
    for (int i = 0; i < (kSlotsPerWave + 1) / 2; ++i) c.so[i] = all[i];
    c.dst = lds_addr + (uint32_t)((ti % kNBuf) * kTileBytes + kSlotsPerWave * w * 1024);
    c.ti = ti;
    if constexpr (!kFast) c.row = *tab_entry(ti, (int)(c.off(0) / kRowBytes));
    if constexpr (kFast) {
      const uint32_t row0 = __builtin_amdgcn_readfirstlane(*tab_entry(ti, 0));
      const bool ok = row0 != ~0u;
      c.nvalid = ok ? min(kTile, j1 - (j0 + ti * kTile)) : 0;
      c.base = a.lat + (size_t)(ok ? row0 : 0u) * kRowBytes;
    }
    return c;
  };
  auto copy_slot = [&](TileCopy& c, int k) {
    if constexpr (kFast) {
      // rows past the valid ones re-read row 0 (their tokens are masked)
      uint32_t voff = c.off(k);
      if (c.nvalid != kTile) {   // uniform
        const uint32_t r = voff / kRowBytes;
        voff = (int)r < c.nvalid ? voff : voff - r * kRowBytes;
      }
      copy16_sbase<kNt>(c.dst + k * 1024, voff, c.base);
    } else {
      // each copy takes the row of its token from the table (tokens without a valid row
      // re-read row 0); the next copy's row is read from the table one copy ahead
      const uint32_t r = c.off(k) / kRowBytes;
      const uint32_t row = c.row;
      if (k + 1 < kSlotsPerWave) c.row = *tab_entry(c.ti, (int)(c.off(k + 1) / kRowBytes));
      const char* src = a.lat + (size_t)(row == ~0u ? 0u : row) * kRowBytes + (c.off(k) - r * kRowBytes);
      copy16_vaddr<kNt>(c.dst + k * 1024, src);
    }
  };
  auto issue_tile = [&](int ti) {
    TileCopy c = plan_copy(ti);
#pragma unroll
    for (int k = 0; k < kSlotsPerWave; ++k) copy_slot(c, k);
  };
  // mask of the valid tokens of tile ti (bit i = token i), wave-uniform
  auto tile_mask = [&](int ti) -> uint32_t {
    if constexpr (kFast) {
      const uint32_t row0 = __builtin_amdgcn_readfirstlane(*tab_entry(ti, 0));
      const int nvalid = row0 != ~0u ? min(kTile, j1 - (j0 + ti * kTile)) : 0;
      return nvalid >= kTile ? 0xffffffffu : ((1u << nvalid) - 1u);
    } else {
      const bool ok = lane < kTile && *tab_entry(ti, lane & (kTile - 1)) != ~0u;
      return (uint32_t)__ballot(ok);
    }
  };

  // ---- the query of this wave's heads (B operand of S^T = K Q^T):
  // qreg[hh][ks] = dims 32 ks + 8 g .. + 8 of head hpw w + 16 hh + i16.  Its loads overlap
  // the table build and the first tile copies; the tile-0 wait below covers them (they
  // were issued first).
  const int head0 = a.hpw * w + i16;
  bf16x8 qreg[HT][kKSteps];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) {
    // padding columns (i16 + 16 hh >= hpw) read the wave's last head
    const int hq = a.hpw * w + min(i16 + 16 * hh, a.hpw - 1);
    const uint16_t* qrow = a.q + (orow + hq) * kDk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[hh][ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }
  // window 0 of the tile table before the first copy
  if (w == kBuilder && ntiles > 0) {
#pragma unroll 1
    for (int p = 0; p < kPasses; ++p) stage_pass(0, p);
    wait_vmcnt<0>();
#pragma unroll 1
    for (int p = 0; p < kPasses; ++p) commit_pass(0, p);
  }
  wait_lgkm0();
  asm volatile("s_barrier" ::: "memory");
  // prologue: tiles 0..2 in flight
  if (copier) {
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k < ntiles) issue_tile(k);
  }

  // O^T accumulators in AGPRs: every definition comes out of an AGPR-constrained asm
  // statement, so the register allocator keeps the loop-carried accumulators there
  f4 acc[HT][kDvTiles];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int i = 0; i < kDvTiles; ++i) {
      acc[hh][i] = f4{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[hh][i]));
    }
  // Wait states between the last accumulator MFMAs and VALU reads of the accumulators;
  // every accumulator passes through an AGPR-constrained statement after them, so the
  // reads cannot be hoisted above.
  auto settle = [&]() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int hh = 0; hh < HT; ++hh)
#pragma unroll
      for (int i = 0; i < kDvTiles; i += 4)
        asm volatile("" : "+a"(acc[hh][i]), "+a"(acc[hh][i + 1]), "+a"(acc[hh][i + 2]),
                     "+a"(acc[hh][i + 3]));
  };

  // K operand (A of S^T): tile row 16 tt + i16, chunk 4 ks + g (position ^ (row & 7))
  // (k-steps 2 m + 1 read chunk position ((4 + g) ^ xk) = (g ^ xk) ^ 4: offk0 ^ 64, the row
  // offset being a multiple of 128)
  const int xk = i16 & 7;
  const int offk0 = i16 * kRowBytes + 16 * (g ^ xk);
  // V^T operand (A of O^T): this lane addresses tile row 4 g + i16 / 4 (+ 16), bytes
  // 8 (i16 mod 4) of the 32 value bytes of dims 16 dt .. 16 dt + 15
  const int rv = 4 * g + (i16 >> 2);
  const int xv = rv & 7;
  const int qv = (i16 >> 1) & 1;
  // dims 16 dt.. sit at chunk position (2 (dt mod 4) + qv) ^ xv = ((qv ^ xv) ^ 2 (dt mod 4))
  // of 8-chunk group dt / 4: offv0 ^ 32 (dt mod 4), plus 128 (dt / 4)
  const int offv0 = rv * kRowBytes + 16 * (qv ^ xv) + (i16 & 1) * 8;

  auto kread = [&](const char DCP_LDS* tb, int ks, bf16x8 (&k2)[2]) {
    const int o = ((ks & 1) ? (offk0 ^ 64) : offk0) + 128 * (ks >> 1);
    k2[0] = *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + o);
    k2[1] = *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + 16 * kRowBytes + o);
  };
  // S^T MFMAs: compiler builtins, so that the hazard recognizer keeps every later write of
  // their operand registers clear of the matrix core's reads.  Their accumulators stay in
  // VGPRs (the file is built with -amdgpu-mfma-vgpr-form; the AGPRs all hold O^T).
  auto qk_step = [&](const bf16x8 (&k2)[2], int ks, f4 (&s)[2][HT]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) {
        s[tt][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            k2[tt], qreg[hh][ks], ks == 0 ? f4{0.f, 0.f, 0.f, 0.f} : s[tt][hh], 0, 0, 0);
      }
  };

  float m[HT], negm[HT], ls[HT];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) {
    m[hh] = neg_inf();   // running max (log2 units) of this lane's heads
    negm[hh] = 0.f;      // -m, or 0 while m is -inf
    ls[hh] = 0.f;        // this lane's share of the running sums
  }

  f4 sc[2][HT];   // S^T of the tile whose softmax runs next: [token half][head tile]
  // tile 0 (and the query, loaded before it) has landed in every wave's copies
  if (ntiles > 2) wait_vmcnt<2 * kSlotsPerWave>();
  else if (ntiles > 1) wait_vmcnt<kSlotsPerWave>();
  else wait_vmcnt<0>();
  asm volatile("s_barrier" ::: "memory");
  uint32_t vmask_next = 0;
  if (ntiles > 0) {
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      bf16x8 k2[2];
      kread(lds, ks, k2);
      qk_step(k2, ks, sc);
    }
    vmask_next = tile_mask(0);
  }

  for (int t = 0; t < ntiles; ++t) {
    // tile t + 1 has landed (only tile t + 2 may still be in flight); after the barrier
    // every wave is past iteration t - 1, so buffer (t - 1) mod 4 takes tile t + 3
    // (the builder's entries staged at iteration t - 1 went out before its copies of tile
    // t + 2, so this wait covers them too)
    const bool staged = w == kBuilder && t > 0 && (t - 1) % kWin == 0 &&
                        ((t - 1) / kWin + 1) * kWin < ntiles;
    if (t + 2 < ntiles) wait_vmcnt<kSlotsPerWave>();
    else wait_vmcnt<0>();
    wait_lgkm0();
    asm volatile("s_barrier" ::: "memory");
    // tables: page-contiguous tiles: window W + 1 (one pass) is staged by wave 3 at
    // iteration W kWin and committed one iteration later; per-token tables: pass p of window
    // W + 1 is staged at iteration W kWin + p by wave p mod 4 and committed one iteration
    // later by the same wave, so the build is spread over the waves and the iterations
    if constexpr (kFast) {
      if (staged) commit_pass((t - 1) / kWin + 1, 0);
      if (w == kBuilder && t % kWin == 0 && (t / kWin + 1) * kWin < ntiles)
        stage_pass(t / kWin + 1, 0);
    } else {
      const int tw = t % kWin;
      if ((t / kWin + 1) * kWin < ntiles) {
        if (tw >= 1 && tw <= kPasses && (tw - 1) % kWaves == w) commit_pass(t / kWin + 1, tw - 1);
        if (tw < kPasses && tw % kWaves == w) stage_pass(t / kWin + 1, tw);
      }
    }
    // tokens of tile t that do not exist (a partial tile, a bad page): scores -inf (a
    // uniform branch, taken on few tiles)
    const uint32_t vmask = vmask_next;
    if (vmask != 0xffffffffu) {
      const uint32_t mb = vmask >> (4 * g);   // bit e: token 4 g + e, bit 16 + e: 16 + 4 g + e
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          sc[0][hh][e] = ((mb >> e) & 1u) ? sc[0][hh][e] : neg_inf();
          sc[1][hh][e] = ((mb >> (16 + e)) & 1u) ? sc[1][hh][e] : neg_inf();
        }
    }

    // ---- S^T of tile t + 1 (computed also after the last tile, on a buffer of stale data,
    // and then unused: the loop body stays one block) with the online softmax of tile t
    // (base 2) cut into one piece per k-step.  Scores stay unscaled until the exp2:
    // scale * log2(e) > 0 keeps the maxima.
    f4 sn[2][HT];
    const char DCP_LDS* tbn = lds + ((t + 1) % kNBuf) * kTileBytes;
    constexpr int kAheadK = ahead_k<kFast>();
    bf16x8 kop[kAheadK + 1][2];
#pragma unroll
    for (int ks = 0; ks < kAheadK; ++ks) kread(tbn, ks, kop[ks]);
    float tm[HT], alpha[HT], p[HT][8];
    bool grow = false;   // this lane's accumulators need rescaling
    bf16x8 pb[HT];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kAheadK < kKSteps) kread(tbn, ks + kAheadK, kop[(ks + kAheadK) % (kAheadK + 1)]);
      qk_step(kop[ks % (kAheadK + 1)], ks, sn);
      if (ks <= 1) {
        // the lane's max of head tile hh over its 8 tokens
        const int hh = ks < HT ? ks : 0;   // (HT = 1: k-step 1 has no piece)
        if (ks < HT) {
        const f4 u = sc[0][hh], v = sc[1][hh];
        tm[hh] = max_f(max_f(max_f(u[0], u[1]), max_f(u[2], u[3])),
                       max_f(max_f(v[0], v[1]), max_f(v[2], v[3])));
        }
      } else if (ks <= 3) {
        const int hh = ks - 2 < HT ? ks - 2 : 0;
        if (ks - 2 < HT)
          tm[hh] = rows_max(tm[hh]) * a.sl2;   // the head's max over the tile (log2 units)
      } else if (ks <= 5) {
        // The running max only moves when the tile's max exceeds it by more than
        // kRescaleSlack (always on the first tile with a valid token).  In between the
        // weights stay below 2^kRescaleSlack and the final normalisation by the running sum
        // is exact for any reference max.
        const int hh = ks - 4 < HT ? ks - 4 : 0;
        if (ks - 4 < HT) {
          const bool up = tm[hh] > m[hh] + kRescaleSlack;
          alpha[hh] = up ? __builtin_amdgcn_exp2f(m[hh] - tm[hh]) : 1.f;   // m = -inf -> 0
          grow = grow || (up && m[hh] != neg_inf());   // accumulators are 0 while m = -inf
          m[hh] = up ? tm[hh] : m[hh];
          negm[hh] = up ? -tm[hh] : negm[hh];
        }
      } else if (ks <= 13) {
        // two weights per k-step: p = exp2(scale log2e s - m); masked tokens give 0
        const int i = 2 * (ks - 6);           // 0 .. 14 over [hh][tt][e]
        const int hh = (i >> 3) < HT ? (i >> 3) : 0, tt = (i >> 2) & 1, e = i & 3;
        if ((i >> 3) < HT) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            p[hh][4 * tt + e + u] =
                __builtin_amdgcn_exp2f(fmaf(sc[tt][hh][e + u], a.sl2, negm[hh]));
        }
      } else if (ks <= 15) {
        const int hh = ks - 14 < HT ? ks - 14 : 0;
        if (ks - 14 < HT) {
          const float* q = p[hh];
          ls[hh] = fmaf(ls[hh], alpha[hh],
                        ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7])));
        }
      } else if (ks - 16 < HT) {
        // B operand of O^T += V^T P^T: k slots 8 g .. 8 g + 7 = tokens 4 g + [0, 4) and
        // 16 + 4 g + [0, 4)
        const int hh = ks - 16;
        const float* q = p[hh];
        pb[hh] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(q[0], q[1]), pack_bf16x2(q[2], q[3]),
                                                  pack_bf16x2(q[4], q[5]), pack_bf16x2(q[6], q[7])});
        // computed here, between the MFMAs, not sunk past the rescale branch
        asm volatile("" : "+v"(pb[hh]), "+v"(ls[hh]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__ballot(grow) != 0) {   // uniform, rare: rescale the accumulators
      settle();
#pragma unroll
      for (int i = 0; i < kDvTiles; ++i) {
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          acc[hh][i] *= alpha[hh];
          asm volatile("" : "+a"(acc[hh][i]));
        }
      }
    }

    // ---- O^T += V^T P^T of tile t, 16 value dims per MFMA pair; the copies of tile t + 3
    // go out between them, one per two or three value tiles
    {
      const char DCP_LDS* tb = lds + (t % kNBuf) * kTileBytes;
      auto vop = [&](int dt) -> bf16x8 {
        const int o = (offv0 ^ (32 * (dt & 3))) + 128 * (dt >> 2);
        const u32x2 v0 = lds_tr16(tb + o);
        const u32x2 v1 = lds_tr16(tb + 16 * kRowBytes + o);
        return __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
      };
      const bool copies = copier && t + 3 < ntiles;
      TileCopy cp;
      if (copies) cp = plan_copy(t + 3);
      if (t + 1 < ntiles) vmask_next = tile_mask(t + 1);
      bf16x8 va[kAheadV + 1];
#pragma unroll
      for (int dt = 0; dt < kAheadV; ++dt) va[dt] = vop(dt);
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) {
        if (dt + kAheadV < kDvTiles) va[(dt + kAheadV) % (kAheadV + 1)] = vop(dt + kAheadV);
        if (dt == 0) mfma_acc<true>(acc[0][dt], va[dt % (kAheadV + 1)], pb[0]);
        else mfma_acc<false>(acc[0][dt], va[dt % (kAheadV + 1)], pb[0]);
        if constexpr (HT == 2) mfma_acc<false>(acc[1][dt], va[dt % (kAheadV + 1)], pb[1]);
#pragma unroll
        for (int k = 0; k < kSlotsPerWave; ++k)
          if (dt == 1 + (k * 30) / kSlotsPerWave && copies) copy_slot(cp, k);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) sc[tt][hh] = sn[tt][hh];
  }

  // ---- finalize: O = acc / l per head, lse = (m + log2 l) ln 2
  settle();
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) {
    const float lt = rows_sum(ls[hh]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (m[hh] + __log2f(lt)) * kLn2 : neg_inf();
    const int head = head0 + 16 * hh;
    if (i16 + 16 * hh >= a.hpw) continue;   // a padding column (fewer than 16 heads a wave)
    if (g == 0) {
      if (single) a.lse_out[orow + head] = lse;
      else a.plse[prow + head] = lse;
    }
    // lane holds dims 16 dt + 4 g + [0, 4) of its head
    if (single && !a.o_bf16) {   // uniform
      float* dst = static_cast<float*>(a.o_out) + (orow + head) * kDv + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt)
        *reinterpret_cast<f4*>(dst + 16 * dt) = acc[hh][dt] * inv;
    } else {
      uint16_t* dst = (single ? static_cast<uint16_t*>(a.o_out) + (orow + head) * kDv
                              : a.po + (prow + head) * kDv) + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) {
        const f4 v = acc[hh][dt] * inv;
        *reinterpret_cast<uint2*>(dst + 16 * dt) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
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
  k.heads = a.heads;
  k.hpw = a.heads / kWaves;
  k.o_bf16 = a.o_bf16;
  k.o_out = o_out;
  k.lse_out = lse_out;
  k.header = ws.header;
  k.off = ws.off;
  k.items = ws.items;
  k.plse = ws.plse;
  k.po = static_cast<uint16_t*>(ws.po);
  const int64_t groups32 = (max_items + 4 * kXcds - 1) / (4 * kXcds);
  const dim3 grid((unsigned)(groups32 * 4 * kXcds * a.rows.q_len));
  const bool fast = (a.interleave % kTile) == 0 && (a.block_size % kTile) == 0;
  const bool nt = a.rows.q_len == 1;
  if (a.heads < kWaves || a.heads > kMaxHeads || a.heads % kWaves != 0)
    return hipErrorInvalidValue;
#define DCP_MLA_LAUNCH(F, N, H)                                                              \
  hipExtLaunchKernelGGL((mla_shard_kernel<F, N, H>), grid, dim3(kWaves * 64), 0, stream, ev0, \
                        ev1, 0, k)
#define DCP_MLA_LAUNCH_H(F, N)                  \
  if (k.hpw > 16) DCP_MLA_LAUNCH(F, N, 2);      \
  else DCP_MLA_LAUNCH(F, N, 1)
  if (fast) {
    if (nt) { DCP_MLA_LAUNCH_H(true, true); } else { DCP_MLA_LAUNCH_H(true, false); }
  } else {
    if (nt) { DCP_MLA_LAUNCH_H(false, true); } else { DCP_MLA_LAUNCH_H(false, false); }
  }
#undef DCP_MLA_LAUNCH_H
#undef DCP_MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace dcp

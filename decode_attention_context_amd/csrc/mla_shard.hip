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
//   * Two workgroups of 4 waves per work item (request, local token range), each owning 64
//     of the 128 heads; wave w of a group owns 16 heads.  A wave keeps its heads' query
//     (18 k-steps x 8 bf16 per lane) and the fp32 output accumulator (32 tiles of 16 dims x
//     16 heads, in AGPRs) in registers.  The two groups of an item get workgroup ids
//     congruent mod 8, so they run on the same XCD and read each latent tile from HBM once
//     between them (the second read hits that XCD's L2).
//   * 32-token tiles of latent rows are copied HBM -> LDS by global_load_lds_dwordx4 (no
//     register staging) into a 4-deep ring: three tiles in flight while one is computed.
//     The copies are issued from inline assembly and paced by explicit vector-memory
//     counter waits plus a bare s_barrier; the compiler, which does not see them, then has
//     no reason to drain them before LDS reads of the other ring buffers.  The 16-byte
//     chunks of a row are XOR-swizzled by (row mod 8) so that operand reads spread over
//     the LDS banks.
//   * When the interleave and the block size are multiples of 32, every tile is one run of
//     consecutive slots in one page: one scalar block-table read locates it and each lane
//     copies from precomputed offsets off that base.  Otherwise each lane walks its own
//     token (the general kernel).
//   * Scores as S^T = K . Q^T (M = 16 tokens, N = 16 heads, K = 32 latent dims): every
//     lane's results belong to ONE head, so the online-softmax max needs only two
//     cross-lane steps and the weights never move between lanes.
//   * Output as O^T = V^T . P^T (M = 16 value dims, N = 16 heads, K = 32 tokens).  The
//     weight operand is the scores' exponentials rounded to bf16; the V^T operand is read
//     with ds_read_b64_tr_b16, which transposes 16-bit elements across each 16-lane group,
//     in the same token order as the score registers.  Accumulator lanes again hold one
//     head, so the online-softmax rescale is lane-local.
//   * The running max only moves when a tile's max exceeds it by more than 8 (log2
//     units).  That rare event leaves the steady tile loop, rescales the accumulator and
//     re-enters it, so inside the loop the accumulator is only ever touched by MFMAs.
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
constexpr int kQkWaves = kHeadTiles;         // score waves: one per head tile
constexpr int kPvWaves = 2 * kHeadTiles;     // output waves: one per (head tile, dv half)
constexpr int kWaves = kQkWaves + kPvWaves;  // 12 waves, three per SIMD
constexpr int kDmaPerWave = kTileBytes / 1024 / kWaves;  // 16-B copies per lane per tile
constexpr int kDvHalfTiles = kDvTiles / 2;   // dv tiles of one output wave
constexpr int kXcds = 8;                     // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr float kRescaleSlack = 8.f;          // see the online softmax below
constexpr int kAheadK = 4;                   // K operand prefetch distance (k-steps)
constexpr int kAheadV = 6;                   // V^T operand prefetch distance (dv tiles)
// LDS: the tile ring, then the weight exchange (two slots: tile parity), the rescale
// factors, and the final per-head normalisation
constexpr int kRingBytes = kNBuf * kTileBytes;                  // 147456
constexpr int kPOff = kRingBytes;                               // [2][4][64 lanes][16 B]
constexpr int kAOff = kPOff + 2 * kHeadTiles * 1024;            // [2][4][16] float
constexpr int kFOff = kAOff + 2 * kHeadTiles * 16 * 4;          // [4][16] float
constexpr int kLdsBytes = kFOff + kHeadTiles * 16 * 4;          // 156416

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

// Two floats to a packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
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

// One 16-byte-per-lane HBM -> LDS copy: LDS bytes [lds + 16 lane, + 16) <- global
// sbase + voff (scalar base, 32-bit lane offset).  M0 carries the LDS address; one wait
// state separates its write from the copy that reads it.
__device__ __forceinline__ void copy16_sbase(uint32_t lds, uint32_t voff, const char* sbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
// The same from a per-lane 64-bit address.
__device__ __forceinline__ void copy16_vaddr(uint32_t lds, const char* src) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
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
// Warp-specialised workgroup of 12 waves for 64 heads (four 16-head tiles):
//   * score waves 0..3 (one per head tile) hold the head tile's query and compute, for tile
//     t, S^T = K Q^T, the online-softmax state and the bf16 weights P, which they hand over
//     through LDS together with the factor that rescales the output accumulated so far;
//   * output waves 4..11 (one per head tile and half of the 512 value dims) hold O^T in
//     AGPRs and, one tile behind, accumulate O^T += V^T P^T.
// Waves are dealt round-robin over the SIMDs, so each SIMD runs one score wave and two
// output waves (68 MFMAs per tile), and every wave issues only 33-36 LDS reads per tile.
// One barrier per tile: at barrier t, tile t has landed (copies paced by each wave's own
// vector-memory counter), the weights of tile t-1 are in LDS, and every read of tile t-2
// is done, so its buffer takes the copy of tile t+2.
template <bool kFast>
__global__ __launch_bounds__(kWaves * 64, 1) void mla_shard_kernel(MlaKArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  // Workgroup ids: the kGroups head groups of one work item are congruent mod 8 (same XCD)
  // and adjacent in dispatch order.
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
  const uint32_t B = (uint32_t)a.block_size;
  const int32_t* btb = a.bt + (size_t)b * a.max_blocks;
  // the block table through the constant address space: scalar loads, which do not count
  // against the vector-memory counter the copy ring is paced with
  const int32_t DCP_CONST* btc = reinterpret_cast<const int32_t DCP_CONST*>(
      reinterpret_cast<uintptr_t>(btb));
  const char DCP_LDS* lds = (const char DCP_LDS*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;

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

  // ---- one tile's HBM -> LDS copy (kDmaPerWave copies of 1 KiB per wave); returns the
  // mask of valid rows.  Chunk c of row r lands at byte 16 * (72 r + (c ^ (r & 7))).
  auto issue_tile = [&](int ti) -> uint64_t {
    const int tj = j0 + ti * kTile;
    const uint32_t dst = lds_addr + (uint32_t)((ti % kNBuf) * kTileBytes + w * kDmaPerWave * 1024);
    if constexpr (kFast) {
      const uint32_t t0 = dcp_walk_global_pos((uint32_t)tj, a.rank, a.cp, a.interleave);
      const uint32_t lp = t0 / B;
      const int32_t pg = btc[lp];
      const int nvalid = min(kTile, j1 - tj);
      const bool ok = pg >= 0 && (uint32_t)pg < a.num_blocks;
      if (!ok && threadIdx.x == 0) atomicOr(&a.header[0], kErrBlockId);
      const uint32_t row0 = ok ? (uint32_t)pg * B + (t0 - lp * B) : 0u;
      const char* base = a.lat + (size_t)row0 * kRowBytes;
      if (ok && nvalid == kTile) {
#pragma unroll
        for (int k = 0; k < kDmaPerWave; ++k) copy16_sbase(dst + k * 1024, slot_off[k], base);
        return 0xffffffffull;
      }
      // partial (last) tile or a bad page: slots of rows past the valid prefix re-read row
      // 0 of the tile (their scores are masked)
      const uint32_t lim = ok ? (uint32_t)nvalid * kRowBytes : 0u;
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k)
        copy16_sbase(dst + k * 1024, slot_off[k] < lim ? slot_off[k] : slot_col[k], base);
      return ok ? ((1ull << nvalid) - 1) : 0ull;
    } else {
      const int j = tj + lane;
      bool ok = lane < kTile && j < j1;
      bool bad = false;
      uint32_t lrow = 0;
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
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k) {
        const uint32_t rr = __shfl(lrow, slot_row[k], 64);
        copy16_vaddr(dst + k * 1024, a.lat + (size_t)rr * kRowBytes + slot_col[k]);
      }
      return __ballot(ok);
    }
  };

  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  // prologue: tiles 0 and 1 in flight
  uint64_t vm0 = issue_tile(0);
  uint64_t vm1 = ntiles > 1 ? issue_tile(1) : 0ull;
  uint64_t vm2 = 0ull;

  // Iteration t of the tile loop, common part: tile t has landed for every wave, tile t+2
  // starts.  Both roles run exactly ntiles + 1 of these.
  auto sync_tile = [&](int t) {
    if (t < ntiles) {
      if (kFast && t + 1 < ntiles) wait_vmcnt<kDmaPerWave>();
      else wait_vmcnt<0>();
    }
    asm volatile("s_barrier" ::: "memory");
    vm2 = t + 2 < ntiles ? issue_tile(t + 2) : 0ull;
  };

  if (w < kQkWaves) {
    // ================= score wave: head tile w =================
    const int head = 16 * (kHeadTiles * hg + w) + i16;
    // query (B operand of S^T = K Q^T): dims 32 ks + 8 g .. + 8
    bf16x8 qreg[kKSteps];
    {
      const uint16_t* qrow = a.q + ((size_t)b * kHeads + head) * kDk + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    }
    // the query must have landed before the copy ring is paced by the counter alone
    wait_vmcnt<0>();
    // The query lives in AGPRs (the MFMAs read their B operand from there), leaving the
    // VGPRs to the operand ring: both roles then fit three waves per SIMD.
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+a"(qreg[ks]));
    float m = neg_inf();   // running max (log2 units) of this lane's head
    float negm = 0.f;      // -m, or 0 while m is -inf
    float ls = 0.f;        // this lane's share of the running sum of weights
    const int xk = i16 & 7;
    const int offk0 = i16 * kRowBytes + 16 * (g ^ xk);
    const int offk1 = i16 * kRowBytes + 16 * ((4 + g) ^ xk);
    char DCP_LDS* pdst = (char DCP_LDS*)smem + kPOff + w * 1024 + lane * 16;
    float DCP_LDS* adst = (float DCP_LDS*)(smem + kAOff) + w * 16 + i16;

    for (int t = 0; t <= ntiles; ++t) {
      wait_lgkm0();   // the previous tile's weights are in LDS before the barrier
      sync_tile(t);
      if (t < ntiles) {
        const char DCP_LDS* tb = lds + (t % kNBuf) * kTileBytes;
        f4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        bf16x8 kop[kAheadK + 1][2];
        auto kread = [&](int ks) {
          const int o = ((ks & 1) ? offk1 : offk0) + 128 * (ks >> 1);
          kop[ks % (kAheadK + 1)][0] = *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + o);
          kop[ks % (kAheadK + 1)][1] =
              *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + 16 * kRowBytes + o);
        };
#pragma unroll
        for (int ks = 0; ks < kAheadK; ++ks) kread(ks);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          if (ks + kAheadK < kKSteps) kread(ks + kAheadK);
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks % (kAheadK + 1)][0], qreg[ks], s0,
                                                       0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks % (kAheadK + 1)][1], qreg[ks], s1,
                                                       0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // scores: x[i] is token 4 g + i, x[4 + i] token 16 + 4 g + i; masked rows -> -inf
        float x[8];
        {
          const uint32_t lo = (uint32_t)(vm0 >> (4 * g)) & 0xFu;
          const uint32_t hi = (uint32_t)(vm0 >> (16 + 4 * g)) & 0xFu;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = ((lo >> i) & 1u) ? s0[i] : neg_inf();
            x[4 + i] = ((hi >> i) & 1u) ? s1[i] : neg_inf();
          }
        }
        // tile max of this lane's head: within the lane, then across the four 16-lane
        // rows (which hold the same head) with two swaps
        float tm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        {
          const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tm),
                                                             __float_as_uint(tm), false, false);
          tm = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
          const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm),
                                                             __float_as_uint(tm), false, false);
          tm = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
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
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(x[i], a.sl2, negm));
        ls = ls * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
        // B operand of O^T += V^T P^T: k slots 8 g .. 8 g + 7 = tokens 4 g + [0, 4) and
        // 16 + 4 g + [0, 4); the output lane with the same index reads these 16 bytes
        const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        *reinterpret_cast<u32x4 DCP_LDS*>(pdst + (t & 1) * (kHeadTiles * 1024)) = pw;
        if (g == 0) adst[(t & 1) * (kHeadTiles * 16)] = alpha;
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
      ((float DCP_LDS*)(smem + kFOff))[w * 16 + i16] = inv;
      if (single) a.lse_out[(size_t)b * kHeads + head] = lse;
      else a.plse[(size_t)item * kHeads + head] = lse;
    }
    wait_lgkm0();
    asm volatile("s_barrier" ::: "memory");
  } else {
    // ================= output wave: head tile ht, value dims 256 half .. + 256 ==========
    const int pv = w - kQkWaves;
    const int ht = pv >> 1;
    const int half = pv & 1;
    const int head = 16 * (kHeadTiles * hg + ht) + i16;
    // Every definition of an accumulator comes out of an AGPR-constrained asm statement,
    // so the register allocator keeps the loop-carried accumulators in AGPRs.
    f4 acc[kDvHalfTiles];
#pragma unroll
    for (int i = 0; i < kDvHalfTiles; ++i) {
      acc[i] = f4{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[i]));
    }
    // Wait states between the last accumulator MFMAs and VALU reads of the accumulators;
    // every accumulator passes through an AGPR-constrained statement here, so the reads
    // cannot be hoisted above it.
    auto settle_acc = [&]() {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+a"(acc[8]), "+a"(acc[9]), "+a"(acc[10]), "+a"(acc[11]),
                     "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]), "+a"(acc[15]));
      asm volatile(""
                   : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                     "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]));
    };
    // V^T operand (A of O^T = V^T P^T) for value-dim tile dt of this wave's half
    const int rv = 4 * g + (i16 >> 2);
    const int xv = rv & 7;
    const int qv = (i16 >> 1) & 1;
    int offv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      offv[u] = rv * kRowBytes + 16 * ((2 * u + qv) ^ xv) + (i16 & 1) * 8 + half * 512;
    const char DCP_LDS* psrc = lds + kPOff + ht * 1024 + lane * 16;
    const float DCP_LDS* asrc = (const float DCP_LDS*)(smem + kAOff) + ht * 16 + i16;

    for (int t = 0; t <= ntiles; ++t) {
      sync_tile(t);
      if (t >= 1) {
        const int u = t - 1;   // the tile whose weights the score waves wrote last
        const char DCP_LDS* tb = lds + (u % kNBuf) * kTileBytes;
        auto vop = [&](int dt) -> bf16x8 {
          const int o = offv[dt & 3] + 128 * (dt >> 2);
          const u32x2 v0 = lds_tr16(tb + o);
          const u32x2 v1 = lds_tr16(tb + 16 * kRowBytes + o);
          return __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
        };
        const bf16x8 pb =
            *reinterpret_cast<const bf16x8 DCP_LDS*>(psrc + (u & 1) * (kHeadTiles * 1024));
        const float alpha = asrc[(u & 1) * (kHeadTiles * 16)];
        bf16x8 va[kAheadV + 1];
#pragma unroll
        for (int dt = 0; dt < kAheadV; ++dt) va[dt] = vop(dt);
        if (__ballot(alpha != 1.f) != 0) {
          settle_acc();
#pragma unroll
          for (int i = 0; i < kDvHalfTiles; ++i) {
            acc[i] *= alpha;
            asm volatile("" : "+a"(acc[i]));
          }
        }
#pragma unroll
        for (int dt = 0; dt < kDvHalfTiles; ++dt) {
          if (dt + kAheadV < kDvHalfTiles) va[(dt + kAheadV) % (kAheadV + 1)] = vop(dt + kAheadV);
          if (dt == 0) mfma_acc<true>(acc[dt], va[dt % (kAheadV + 1)], pb);
          else mfma_acc<false>(acc[dt], va[dt % (kAheadV + 1)], pb);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    asm volatile("s_barrier" ::: "memory");
    // ---- finalize: lane holds dims 256 half + 16 dt + 4 g + [0, 4) of its head
    const float inv = ((const float DCP_LDS*)(smem + kFOff))[ht * 16 + i16];
    settle_acc();
    float* dst = (single ? a.o_out + ((size_t)b * kHeads + head) * kDv
                         : a.po + ((size_t)item * kHeads + head) * kDv) +
                 half * 256;
#pragma unroll
    for (int dt = 0; dt < kDvHalfTiles; ++dt) {
      const f4 v = acc[dt] * inv;
      *reinterpret_cast<f4*>(dst + 16 * dt + 4 * g) = v;
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
  const int64_t groups8 = (max_items + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(groups8 * kXcds * kGroups));
  const bool fast = (a.interleave % kTile) == 0 && (a.block_size % kTile) == 0;
  if (fast)
    hipLaunchKernelGGL(mla_shard_kernel<true>, grid, dim3(kWaves * 64), 0, stream, k);
  else
    hipLaunchKernelGGL(mla_shard_kernel<false>, grid, dim3(kWaves * 64), 0, stream, k);
  return hipGetLastError();
}

}  // namespace dcp

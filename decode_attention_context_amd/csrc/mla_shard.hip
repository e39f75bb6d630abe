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
constexpr int kWaves = 4;                    // waves per workgroup, 16 heads each
constexpr int kGroups = kHeads / (16 * kWaves);          // head groups (workgroups) per item
constexpr int kDmaPerWave = kTileBytes / 1024 / kWaves;  // 16-B copies per lane per tile
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

// kFast: the interleave and the block size are multiples of the tile, so the 32 tokens of a
// tile are consecutive slots of one cache page.
template <bool kFast>
__global__ __launch_bounds__(kWaves * 64, 1) void mla_shard_kernel(MlaKArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kNBuf * kTileBytes];

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
  const int head = 16 * (kWaves * hg + w) + i16;
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

  // ---- query (B operand of S^T = K Q^T): dims 32 ks + 8 g .. + 8
  bf16x8 qreg[kKSteps];
  {
    const uint16_t* qrow = a.q + ((size_t)b * kHeads + head) * kDk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }
  // the query must have landed before the copy ring starts: inside the ring the vector
  // memory counter only paces tile copies
  wait_vmcnt<0>();

  // Every definition of an accumulator comes out of an AGPR-constrained asm statement, so
  // the register allocator keeps the loop-carried accumulators in AGPRs instead of copying
  // them to VGPRs around every tile.
  f4 acc[kDvTiles];
#pragma unroll
  for (int i = 0; i < kDvTiles; ++i) {
    acc[i] = f4{0.f, 0.f, 0.f, 0.f};
    asm volatile("" : "+a"(acc[i]));
  }
  float m = neg_inf();   // running max (log2 units) of this lane's head
  float negm = 0.f;      // -m, or 0 while m is -inf
  float ls = 0.f;        // this lane's share of the running sum of weights

  // Wait states between the last accumulator MFMAs and VALU reads of the accumulators.
  // Every accumulator passes through an AGPR-constrained statement here, so the reads
  // cannot be hoisted above it (out of the rare rescale branch, into the tile loop).
  auto settle_acc = [&]() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[24]), "+a"(acc[25]), "+a"(acc[26]), "+a"(acc[27]),
                   "+a"(acc[28]), "+a"(acc[29]), "+a"(acc[30]), "+a"(acc[31]));
#pragma unroll
    for (int i0 = 0; i0 < 24; i0 += 8)
      asm volatile(""
                   : "+a"(acc[i0]), "+a"(acc[i0 + 1]), "+a"(acc[i0 + 2]), "+a"(acc[i0 + 3]),
                     "+a"(acc[i0 + 4]), "+a"(acc[i0 + 5]), "+a"(acc[i0 + 6]),
                     "+a"(acc[i0 + 7]));
  };

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

  // K operands (A of S^T = K Q^T) for k-step ks of a tile: tokens i16 and 16 + i16
  auto kread = [&](const char DCP_LDS* tb, int ks, bf16x8 (&dst)[2]) {
    const int o = ((ks & 1) ? offk1 : offk0) + 128 * (ks >> 1);
    dst[0] = *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + o);
    dst[1] = *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + 16 * kRowBytes + o);
  };
  // V^T operand (A of O^T = V^T P^T) for value-dim tile dt
  auto vop = [&](const char DCP_LDS* tb, int dt) -> bf16x8 {
    const int o = offv[dt & 3] + 128 * (dt >> 2);
    const u32x2 v0 = lds_tr16(tb + o);
    const u32x2 v1 = lds_tr16(tb + 16 * kRowBytes + o);
    return __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
  };
  // Score masking: x[i] is token 4 g + i, x[4 + i] token 16 + 4 g + i of the tile; rows
  // outside the mask get -inf (branch-free: it runs in the shadow of MFMAs).
  auto mask_scores = [&](const f4& s0, const f4& s1, uint64_t vm, float (&xo)[8]) {
    const uint32_t lo = (uint32_t)(vm >> (4 * g)) & 0xFu;
    const uint32_t hi = (uint32_t)(vm >> (16 + 4 * g)) & 0xFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xo[i] = ((lo >> i) & 1u) ? s0[i] : neg_inf();
      xo[4 + i] = ((hi >> i) & 1u) ? s1[i] : neg_inf();
    }
  };
  // max over the 32 tokens of the tile for this lane's head (lanes i16, 16+i16, 32+i16,
  // 48+i16 hold one head): within the lane, then across the 16-lane rows with two swaps
  auto lane_max = [&](const float (&xi)[8]) -> float {
    return fmaxf(fmaxf(fmaxf(xi[0], xi[1]), fmaxf(xi[2], xi[3])),
                 fmaxf(fmaxf(xi[4], xi[5]), fmaxf(xi[6], xi[7])));
  };
  auto row_max = [&](float t) -> float {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t),
                                                       false, false);
    t = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t),
                                                       false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
  };

  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  // prologue: tiles 0, 1, 2 in flight
  uint64_t vm0 = issue_tile(0);
  uint64_t vm1 = ntiles > 1 ? issue_tile(1) : 0ull;
  uint64_t vm2 = ntiles > 2 ? issue_tile(2) : 0ull;
  uint64_t vm3 = 0ull;

  // scores of tile 0
  float x[8];               // scores of the tile whose weights come next
  float tmax;               // their max (log2 units) for this lane's head
  {
    if (!kFast || ntiles < 2) wait_vmcnt<0>();
    else if (ntiles == 2) wait_vmcnt<kDmaPerWave>();
    else wait_vmcnt<2 * kDmaPerWave>();
    asm volatile("s_barrier" ::: "memory");
    f4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    bf16x8 kop[kAhead + 1][2];
#pragma unroll
    for (int ks = 0; ks < kAhead; ++ks) kread(lds, ks, kop[ks]);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kAhead < kKSteps) kread(lds, ks + kAhead, kop[(ks + kAhead) % (kAhead + 1)]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks % (kAhead + 1)][0], qreg[ks], s0, 0,
                                                   0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks % (kAhead + 1)][1], qreg[ks], s1, 0,
                                                   0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask_scores(s0, s1, vm0, x);
    tmax = row_max(lane_max(x)) * a.sl2;
  }

  // Software pipeline, iteration ti: (1) the running-max check for tile ti, (2) wait for
  // tile ti+1 and start tile ti+3, (3) the MFMAs of tile ti+1's scores with tile ti's
  // weights computed between them, (4) the MFMAs of tile ti's O^T += V^T P^T with tile
  // ti+1's masking and max computed between them.  The ring holds tiles ti (read by (4)),
  // ti+1 (read by (3)), ti+2 and ti+3 (landing).  On the last tile, (3) reads a stale
  // buffer whose scores are never used.
  for (int ti = 0; ti < ntiles; ++ti) {
    // (1) Some head's tile max exceeds its running max by more than kRescaleSlack (always
    // on the first tile with valid tokens): move those maxima to the tile max and
    // rescale.  Between raises the weights stay below 2^kRescaleSlack, exactly
    // representable in bf16 / fp32, and the final normalisation by the running sum is
    // exact either way.
    {
      const bool up = tmax > m + kRescaleSlack;
      if (__ballot(up) != 0) {
        const float alpha = up ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;   // m = -inf -> 0
        if (up) {
          m = tmax;
          negm = -tmax;
        }
        ls *= alpha;
        settle_acc();
#pragma unroll
        for (int i = 0; i < kDvTiles; ++i) {
          acc[i] *= alpha;
          asm volatile("" : "+a"(acc[i]));
        }
      }
    }
    // (2) this wave's copies of tile ti+1 have landed (those of ti+2 may still fly); after
    // the barrier every wave's have, and every wave is done with tile ti-1, whose buffer
    // tile ti+3 now takes.  A bare barrier: the fence of __syncthreads would also wait for
    // the copies still in flight.
    if (kFast && ti + 2 < ntiles) wait_vmcnt<kDmaPerWave>();
    else wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
    vm3 = ti + 3 < ntiles ? issue_tile(ti + 3) : 0ull;
    const char DCP_LDS* bq = lds + ((ti + 1) % kNBuf) * kTileBytes;
    const char DCP_LDS* bv = lds + (ti % kNBuf) * kTileBytes;

    // (3) scores of tile ti+1; weights of tile ti
    f4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = {0.f, 0.f, 0.f, 0.f};
    float p[8];
    bf16x8 pb;
    {
      bf16x8 kop[kAhead + 1][2];
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) kread(bq, ks, kop[ks]);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + kAhead < kKSteps) kread(bq, ks + kAhead, kop[(ks + kAhead) % (kAhead + 1)]);
        n0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks % (kAhead + 1)][0], qreg[ks], n0,
                                                     0, 0, 0);
        n1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks % (kAhead + 1)][1], qreg[ks], n1,
                                                     0, 0, 0);
        if (ks < 8) p[ks] = __builtin_amdgcn_exp2f(fmaf(x[ks], a.sl2, negm));
        if (ks == 9)
          pb = __builtin_bit_cast(
              bf16x8, u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
        if (ks == 10) ls += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        __builtin_amdgcn_sched_barrier(0);   // one scheduling region per k-step
      }
    }

    // (4) O^T += V^T P^T of tile ti (V^T operands read kAhead dim tiles ahead); masking and
    // max of tile ti+1
    {
      float xn[8];
      float tn = 0.f;
      bf16x8 va[kAhead + 1];
#pragma unroll
      for (int dt = 0; dt < kAhead; ++dt) va[dt] = vop(bv, dt);
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) {
        if (dt + kAhead < kDvTiles) va[(dt + kAhead) % (kAhead + 1)] = vop(bv, dt + kAhead);
        if (dt == 0) mfma_acc<true>(acc[dt], va[dt % (kAhead + 1)], pb);
        else mfma_acc<false>(acc[dt], va[dt % (kAhead + 1)], pb);
        if (dt == 1) mask_scores(n0, n1, vm1, xn);
        if (dt == 3) tn = lane_max(xn);
        if (dt == 5) tn = row_max(tn);
        if (dt == 7) tn *= a.sl2;
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = xn[i];
      tmax = tn;
    }
    vm0 = vm1;
    vm1 = vm2;
    vm2 = vm3;
  }

  // ---- finalize: lane holds dims 16 dt + 4 g + [0, 4) of its head
  settle_acc();
  float lt = ls + __shfl_xor(ls, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : neg_inf();
  float* dst = single ? a.o_out + ((size_t)b * kHeads + head) * kDv
                      : a.po + ((size_t)item * kHeads + head) * kDv;
#pragma unroll
  for (int dt = 0; dt < kDvTiles; ++dt) {
    const f4 v = acc[dt] * inv;
    *reinterpret_cast<f4*>(dst + 16 * dt + 4 * g) = v;
  }
  if (g == 0) {
    if (single) a.lse_out[(size_t)b * kHeads + head] = lse;
    else a.plse[(size_t)item * kHeads + head] = lse;
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

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
// 4 * R * D flops for R query rows), so the design is about keeping K / V bytes streaming
// at full rate.  Two variants share the copy machinery below: bf16 (R <= 64 query rows per
// KV head) computes both products on the matrix cores (the kMfma variant, described at the
// kernel); f32 stays on the vector ALUs as follows:
//   * One workgroup of NW <= 8 waves per work item (request, KV head, local token range),
//     two workgroups per CU; wave w owns HPW of the R = q_len * G query rows that share the
//     KV head (q_len query positions per request, see below).
//   * 64-token tiles of K and V rows are copied HBM -> LDS by global_load_lds_dwordx4 (no
//     register staging) with the non-temporal cache policy into a double buffer: tiles 0
//     and 1 are issued up front, then each tile's copies leave right after the barrier that
//     frees its buffer.  The copies are issued from inline assembly and paced by explicit
//     vector-memory counter waits plus a bare s_barrier, so the compiler never drains them
//     before LDS reads.  When the interleave and the block size are multiples of the tile,
//     a tile is one run of consecutive cache rows: a per-wave table (lane k = first row of
//     tile 64 * window + k) locates it with one readlane and the copies are a scalar base
//     plus fixed lane offsets; otherwise each lane walks one token.
//   * K rows sit in 4-row blocks, chunk-major inside a block, the blocks 1088 bytes apart:
//     a lane's row is a base address plus immediate offsets, and the rows that one LDS read
//     serves fall in distinct bank groups.
//   * Scores: lane = token.  The lane pulls its whole K row from LDS into registers; each
//     query head, being wave-uniform, sits in scalar registers (loaded once when a wave owns
//     one head, streamed in 16-dword chunks otherwise) and is the scalar operand of
//     v_fma_f32: no cross-lane reduction.
//   * Online softmax in base 2 (scale * log2 e folded into the scores).  The tile max per
//     head is v_max_f32 with DPP operands (row butterfly, then row broadcasts into the last
//     lane) read into a scalar; running sums stay per lane and are reduced once per item.
//   * P.V: lane = (token group, 16-byte chunk of the V row), the weights going through LDS;
//     the four token groups are summed across rows once per item.
//   * An item that covers a request's whole shard writes (O, lse) directly; otherwise it
//     writes a normalized partial that the split combine merges.
//   * Multi-token decode (q_len > 1: speculative decoding or multi-token prediction, the
//     last q_len cache tokens being the request's own draft tokens): query row i sits at
//     position seq_len - q_len + i and sees the positions up to its own, i.e. a prefix of
//     the shard's local tokens.  Every row of the KV head reads each K / V tile once; a
//     row's causal limit only masks tokens of the last tile or two of a request.
#include "launch.h"

namespace dcp {

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(16))) uint32_t u32x16;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(4))) short s4;

#define DCP_LDS __attribute__((address_space(3)))
#define DCP_CONST __attribute__((address_space(4)))

constexpr int kTile = kGqaTile;      // tokens per tile (= lanes)
constexpr int kRowBytes = kGqaRowBytes;   // D * sizeof(T) for the supported shapes
constexpr int kChunks = kRowBytes / 16;
constexpr int kTileBytes = kTile * kRowBytes;   // 16 KiB of K (and of V) per tile
constexpr int kNBuf = 2;                         // double buffer: one computed, one in flight
constexpr int kSlots = 2 * kTileBytes / 1024;   // 1-KiB copies per tile (K then V)
// K rows sit in 4-row blocks, chunk-major inside a block (16-byte unit 4 * chunk + row),
// with the blocks 1088 bytes apart: row r's chunk c is at a lane base plus the immediate
// 64 c, and the 16 rows read together fall in 16 distinct 16-byte bank groups.
constexpr int kKBlock = 1024 + 64;
constexpr int kKBytes = (kTile / 4) * kKBlock;   // K part of a buffer
constexpr int kBufBytes = kKBytes + kTileBytes;  // K blocks, then the V rows
constexpr float kRescaleSlack = 8.f;             // see the online softmax below

struct GqaKArgs {
  const void* q;
  const char* kp;
  const char* vp;
  const int32_t* bt;
  int hq, hkv, block_size, max_blocks;
  uint32_t num_blocks;
  int rank, cp, interleave;
  float sl2;  // scale * log2(e)
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

__device__ __forceinline__ u32x2 lds_tr16(const char DCP_LDS* p) {
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 DCP_LDS*)p);
  return __builtin_bit_cast(u32x2, v);
}

// V rows of the matrix-core kernel are stored with their 16-byte chunks XOR-swizzled by
// the row: its transposed reads take 8 consecutive rows at one pair of chunks across two
// 16-lane groups, and moving the chunk pair by the row's low three bits puts the 8 rows in 8
// distinct 32-byte slots.  f32 V rows are read row-wise and stored as they are.
template <bool kMfma>
__device__ __forceinline__ int v_swz_t(int r) {
  return kMfma ? (r & 7) << 1 : 0;
}

// Waves and rows per wave for R query rows per KV head: up to 8 waves, rows dealt evenly;
// rows past R (when the waves do not divide R) repeat the last row and are not written.
constexpr int waves_for(int r) { return r >= 8 ? 8 : (r > 4 ? 8 : (r > 2 ? 4 : r)); }
constexpr int rows_per_wave(int r) { return (r + waves_for(r) - 1) / waves_for(r); }

// kMfma: the matrix-core variant, bf16 only: four waves, HPW = 16-row tiles per wave (rows
// past R are padding); a workgroup takes all R <= 48 query rows (three row tiles: 48 rows at
// the G = 16 share's q_len 3 in 98.9 us, against 107.8-116.5 us as two 32-row slices, on
// MI355X; four row tiles spill), or a slice of 32 of them (R > 48: two workgroups per item
// and KV head, the second reading the tiles from L2).  Wave w takes token quarter
// w of every tile for all rows and keeps its own online softmax over those tokens:
//   * S^T (16 tokens x 16 rows) = K (16 x 128) . Q^T on v_mfma_f32_16x16x32_bf16, the K
//     operand (lane = token, 8 dims) read straight from the 4-row K blocks and the query
//     operand resident in registers for the whole item.  Lane (group g, i16) gets row i16,
//     tokens 4 g .. 4 g + 3;
//   * those four weights, packed to bf16, are exactly the P^T operand of
//     v_mfma_f32_16x16x16_bf16 (tokens 4 g .. 4 g + 3 of column i16), so
//     O^T (128 dims x 16 rows) += V^T (128 x 16 tokens) . P^T needs no LDS round trip; the
//     V^T operand (one dim of 4 consecutive tokens) is one ds_read_b64_tr_b16 per 16 dims;
//   * every K and V^T operand read feeds one MFMA per row tile;
//   * a row's maximum over the tile is the max of a lane's four scores combined across the
//     four 16-lane groups (permlane swaps); rows sit in lanes, so the lazy rescale is per
//     lane under a wave-uniform branch;
//   * after the last tile the four token quarters of each row merge through LDS by the LSE
//     identity (weights exp2(m_k - max m), empty quarters weight 0).
// Waves per SIMD the register allocation must allow (HIP's second launch bound): two
// workgroups per CU (their LDS double buffers) give NW / 2 waves per SIMD, at least one;
// the 8-wave f32 variants keep the 4-wave figure (their rows per wave need the registers).
constexpr int min_waves_per_simd(int nw) { return nw >= 4 ? 2 : 1; }

template <bool kBf16, int NW, int HPW>
__global__ __launch_bounds__(64 * NW, min_waves_per_simd(NW)) void gqa_shard_kernel(GqaKArgs a) {
  constexpr bool kMfma = kBf16;   // bf16 runs on the matrix cores, f32 on the vector ALUs
  static_assert(!kMfma || NW == 4, "matrix-core variant: four waves");
  constexpr int kElemBytes = kBf16 ? 2 : 4;
  constexpr int D = kRowBytes / kElemBytes;     // head dim
  constexpr int kDmaPerWave = kSlots / NW;

  // [buffer][K blocks | V rows]
  __shared__ u32x4 kvs[kNBuf * kBufBytes / 16];
  __shared__ uint32_t pbuf[kMfma ? 1 : NW][HPW][kMfma ? 1 : kTile];   // f32 weights
  __shared__ float mls[kMfma ? NW * 16 * HPW * 2 : 1];   // matrix-core variant: (m, l) per row

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  if ((int)blockIdx.x >= a.header[1]) return;
  const int4 it = a.items[blockIdx.x];   // in dispatch order, longest first
  const int b = it.x, j0 = it.y, j1 = it.z;
  const int item = it.w;                 // index of the item's partial
  // matrix-core variant: blockIdx.y = KV head + hkv * (row slice); the slices of one
  // item share its K / V tiles (a later slice's reads mostly hit L2)
  const int kvh = kMfma ? (int)blockIdx.y % a.hkv : (int)blockIdx.y;
  const int rbase = kMfma ? 16 * HPW * ((int)blockIdx.y / a.hkv) : 0;   // slice's first row
  // K / V copies stream with the non-temporal policy, except when two slices read the same
  // tiles: the second then finds them in L2
  const bool nt = !(kMfma && a.q_len * (a.hq / a.hkv) > 16 * HPW);
  const bool single = (a.off[b + 1] - a.off[b]) == 1;
  // The wave's query rows (wave-uniform): row rho = w * HPW + h of the R = q_len * G rows
  // of this KV head is query position qi = rho / G, head kvh * G + rho % G, request row
  // qi * hq + head.  lim[h] = local end of the tokens the row sees in this item.
  const int G = a.hq / a.hkv;
  const int R = a.q_len * G;
  const int RQ = a.q_len * a.hq;               // rows per request
  int rrow[HPW], lim[HPW];
  bool live[HPW];
  int lim_min = j1;
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    int rho = w * HPW + h;
    live[h] = rho < R;
    rho = min(rho, R - 1);
    const int qi = rho / G;
    rrow[h] = qi * a.hq + kvh * G + (rho - qi * G);
    lim[h] = a.q_len == 1 ? j1
                          : min(j1, row_local_end(a.seq_lens, b, a.len_cap, a.q_len, qi,
                                                  a.rank, a.cp, a.interleave));
    lim_min = min(lim_min, lim[h]);
  }
  // the query rows: wave-uniform, read-only -> scalar loads
  const uint32_t DCP_CONST* qbase = reinterpret_cast<const uint32_t DCP_CONST*>(
                                        reinterpret_cast<uintptr_t>(a.q)) +
                                    (size_t)b * RQ * (kRowBytes / 4);
  const uint32_t DCP_CONST* qh = qbase + (size_t)rrow[0] * (kRowBytes / 4);
  const int32_t* btb = a.bt + (size_t)b * a.max_blocks;
  const uint32_t B = (uint32_t)a.block_size;
  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  const bool fast = (a.interleave % kTile) == 0 && (a.block_size % kTile) == 0;
  const char DCP_LDS* kvb = (const char DCP_LDS*)&kvs[0];
  const uint32_t lds_addr = (uint32_t)(uintptr_t)kvb;

  // ---- copy slots of this wave: slot s = w * kDmaPerWave + k, one 1-KiB copy each.
  // s < 16: the K block of rows 4 s .. 4 s + 3, lane l bringing chunk l / 4 of row
  // 4 s + l % 4.  s >= 16: V 16-byte positions q = (s - 16) * 64 + lane, row q / 16, holding
  // chunk (q mod 16) ^ swizzle(row).
  uint32_t slot_src[kDmaPerWave];
  int slot_row[kDmaPerWave];
  uint32_t slot_dst[kDmaPerWave];   // byte offset in the buffer (wave-uniform)
#pragma unroll
  for (int k = 0; k < kDmaPerWave; ++k) {
    const int sl = w * kDmaPerWave + k;
    if (sl < 16) {
      slot_row[k] = 4 * sl + (lane & 3);
      slot_src[k] = (uint32_t)(lane >> 2) * 16;
      slot_dst[k] = (uint32_t)(sl * kKBlock);
    } else {
      const int q = (sl - 16) * 64 + lane;
      const int r = q / kChunks, pc = q % kChunks;
      slot_row[k] = r;
      slot_src[k] = (uint32_t)((pc ^ v_swz_t<kMfma>(r)) * 16);
      slot_dst[k] = (uint32_t)(kKBytes + (sl - 16) * 1024);
    }
    slot_dst[k] = __builtin_amdgcn_readfirstlane(slot_dst[k]);   // M0 operand: keep it scalar
  }

  // ---- tile sources (contiguous tiles): lane k = first cache row of tile 64 * window + k,
  // or ~0 for a bad page; rebuilt once per 64 tiles
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
      else row = ((uint32_t)pg * a.hkv + kvh) * B + (t - lp * B);
    }
    if (__ballot(bad) != 0 && threadIdx.x == 0) atomicOr(&a.header[0], kErrBlockId);
    row_tab = row;
  };
  if (fast) build_table(0);

  // ---- contiguous tiles: where tile ti comes from (rb = byte offset of its first row;
  // rows at or past lim re-read row 0, their tokens being masked), and one of this wave's
  // copies of it
  struct TileSrc {
    size_t rb;
    uint32_t lim;
    uint32_t dst;
  };
  auto locate = [&](int ti, uint64_t& vm) -> TileSrc {
    if ((ti & 63) == 0 && ti > 0) build_table(ti >> 6);
    const int nvalid = min(kTile, j1 - (j0 + ti * kTile));
    const uint32_t row0 = __builtin_amdgcn_readlane(row_tab, ti & 63);
    const bool ok = row0 != ~0u;
    vm = ok ? (nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1)) : 0ull;
    TileSrc ts;
    ts.rb = (size_t)(ok ? row0 : 0u) * kRowBytes;
    ts.lim = ok ? (uint32_t)nvalid : 0u;
    ts.dst = lds_addr + (uint32_t)((ti % kNBuf) * kBufBytes);
    return ts;
  };
  auto copy_slot = [&](const TileSrc& ts, int k) {
    const int sl = w * kDmaPerWave + k;
    const uint32_t voff = (uint32_t)slot_row[k] < ts.lim
                              ? (uint32_t)slot_row[k] * kRowBytes + slot_src[k]
                              : slot_src[k];
    if (nt) copy16_sbase<true>(ts.dst + slot_dst[k], voff, (sl < 16 ? a.kp : a.vp) + ts.rb);
    else copy16_sbase<false>(ts.dst + slot_dst[k], voff, (sl < 16 ? a.kp : a.vp) + ts.rb);
  };
  // ---- all of this wave's HBM -> LDS copies of tile ti; returns the mask of valid tokens
  auto issue_tile = [&](int ti) -> uint64_t {
    const uint32_t dst = lds_addr + (uint32_t)((ti % kNBuf) * kBufBytes);
    if (fast) {
      uint64_t vm;
      const TileSrc ts = locate(ti, vm);
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k) copy_slot(ts, k);
      return vm;
    }
    // general tiles: each lane walks one token; the copies take the row of their token
    const int j = j0 + ti * kTile + lane;
    bool ok = j < j1;
    bool bad = false;
    uint32_t row = 0;
    if (ok) {
      const uint32_t t = dcp_walk_global_pos((uint32_t)j, a.rank, a.cp, a.interleave);
      const uint32_t lp = t / B;
      const int32_t pg = btb[lp];
      if (pg < 0 || (uint32_t)pg >= a.num_blocks) {
        ok = false;
        bad = true;
      } else {
        row = ((uint32_t)pg * a.hkv + kvh) * B + (t - lp * B);
      }
    }
    if (__ballot(bad) != 0 && threadIdx.x == 0) atomicOr(&a.header[0], kErrBlockId);
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
      const int sl = w * kDmaPerWave + k;
      const uint32_t rr = __shfl(row, slot_row[k], 64);
      const char* src = (sl < 16 ? a.kp : a.vp) + (size_t)rr * kRowBytes + slot_src[k];
      if (nt) copy16_vaddr<true>(dst + slot_dst[k], src);
      else copy16_vaddr<false>(dst + slot_dst[k], src);
    }
    return __ballot(ok);
  };

  if constexpr (kMfma) {
    constexpr int RT = HPW;   // 16-row tiles per wave
    const int g = lane >> 4, i16 = lane & 15;
    const int tq = w;         // token quarter of every tile
    // this lane's query row in each row tile (rows past R repeat row R - 1 and are not
    // written) and the local end of the tokens it sees; lim_lo, the smallest such end in
    // the workgroup (position 0), decides when a tile needs masking
    int lim_l[RT];
    bf16x8 qop[RT][4];   // query operand of the 4 k-steps: dims 32 ks + 8 g .. + 7
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int rho = min(rbase + 16 * r + i16, R - 1);
      const int qi = rho / G;
      const int qrow = qi * a.hq + kvh * G + (rho - qi * G);
      lim_l[r] = a.q_len == 1 ? j1
                              : min(j1, row_local_end(a.seq_lens, b, a.len_cap, a.q_len, qi,
                                                      a.rank, a.cp, a.interleave));
      const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                       ((size_t)b * RQ + qrow) * D) + g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qop[r][ks] = __builtin_bit_cast(bf16x8, qp[4 * ks]);
    }
    const int lim_lo = a.q_len == 1 ? j1
                                    : min(j1, row_local_end(a.seq_lens, b, a.len_cap, a.q_len,
                                                            0, a.rank, a.cp, a.interleave));

    float m[RT], negm[RT], ls[RT];
    f4 acc[RT][D / 16];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      m[r] = neg_inf();
      negm[r] = 0.f;
      ls[r] = 0.f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) acc[r][db] = f4{0.f, 0.f, 0.f, 0.f};
    }

    // K operand: tile row 16 tq + i16, chunk 4 ks + g of the 4-row blocks; V^T operand: this
    // lane addresses tile row 16 tq + 4 g + i16 / 4, bytes 8 (i16 mod 4) of the swizzled
    // 32-byte slot of dims 16 db .. 16 db + 15.  Every operand read feeds one MFMA per row
    // tile.
    const int rk = 16 * tq + i16;
    const int koff = (rk >> 2) * kKBlock + (rk & 3) * 16 + 64 * g;
    const int rv = 16 * tq + 4 * g + (i16 >> 2);
    const int voff = kKBytes + rv * kRowBytes + 8 * (i16 & 3);
    const int vsw = rv & 7;

    uint64_t vm0 = issue_tile(0);
    const uint64_t vm_first = ntiles > 1 ? issue_tile(1) : 0ull;
    for (int ti = 0; ti < ntiles; ++ti) {
      // tile ti has landed in every wave's copies; the other buffer is free (see below)
      if (ti == 0 && ntiles > 1) wait_vmcnt<kDmaPerWave>();
      else wait_vmcnt<0>();
      asm volatile("s_barrier" ::: "memory");
      const uint64_t vm1 = ti == 0 ? vm_first : (ti + 1 < ntiles ? issue_tile(ti + 1) : 0ull);
      const char DCP_LDS* tb = kvb + (ti % kNBuf) * kBufBytes;

      // ---- S^T of this wave's 16 tokens x 16 rows, per row tile
      bf16x8 kop[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kop[ks] = *reinterpret_cast<const bf16x8 DCP_LDS*>(tb + koff + 256 * ks);
      f4 sc[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) sc[r] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < RT; ++r)
          sc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks], qop[r][ks], sc[r], 0, 0, 0);

      // ---- online softmax (base 2) per row = per lane column, lazy rescale as in the
      // vector kernel (slack kRescaleSlack), here with a per-lane factor
      const int jt = j0 + ti * kTile;
      const bool partial = vm0 != ~0ull || jt + kTile > lim_lo;   // uniform
      s4 pb[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = sc[r][e] * a.sl2;
        if (partial) {
          asm volatile("");
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tt = 16 * tq + 4 * g + e;
            x[e] = (((vm0 >> tt) & 1) && jt + tt < lim_l[r]) ? x[e] : neg_inf();
          }
        }
        const float tmax = rows_max(max_f(max_f(x[0], x[1]), max_f(x[2], x[3])));
        const bool need = tmax > m[r] + kRescaleSlack;   // m = -inf: any valid token
        if (__builtin_amdgcn_ballot_w64(need) != 0) {      // uniform branch
          const float alpha = need ? __builtin_amdgcn_exp2f(m[r] - tmax) : 1.f;  // -inf -> 0
          m[r] = need ? tmax : m[r];
          negm[r] = need ? -tmax : negm[r];
          ls[r] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 16; ++db) acc[r][db] *= alpha;
        }
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(x[e] + negm[r]);  // masked: 0
        ls[r] += (p[0] + p[1]) + (p[2] + p[3]);
        const f2 p01 = {p[0], p[1]}, p23 = {p[2], p[3]};
        const u32x2 pw = {__builtin_bit_cast(uint32_t, __builtin_convertvector(p01, bf16x2)),
                          __builtin_bit_cast(uint32_t, __builtin_convertvector(p23, bf16x2))};
        pb[r] = __builtin_bit_cast(s4, pw);
      }

      // ---- O^T += V^T P^T, 16 dims per MFMA
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const s4 v = __builtin_bit_cast(s4, lds_tr16(tb + voff + 32 * (db ^ vsw)));
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[r][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pb[r], acc[r][db], 0, 0, 0);
      }
      vm0 = vm1;
    }

    // ---- merge the four token quarters of each row through LDS (the tile buffers are free
    // once every wave has passed the barrier; no copy is in flight).  Scratch rows are
    // (wave, row tile, lane column).
    constexpr int kOStride = D + 4;   // floats per row: rows 16 bytes apart in the banks
    // row tiles merged per pass: all of them where the scratch fits, else one at a time
    constexpr int kPass = NW * 16 * RT * kOStride * 4 <= (int)sizeof(kvs) ? RT : 1;
    constexpr int kRows = 16 * kPass;   // scratch rows per wave and pass
    static_assert(NW * kRows * kOStride * 4 <= (int)sizeof(kvs), "merge scratch");
    float DCP_LDS* osc = (float DCP_LDS*)&kvs[0];
    wait_vmcnt<0>();
    // wave tq finishes dims 32 tq .. 32 tq + 31 of every row
    const int d0 = 32 * tq + 8 * (lane & 3);
#pragma unroll
    for (int r0 = 0; r0 < RT; r0 += kPass) {
      __syncthreads();   // the tile buffers (first pass) or the previous pass's rows are free
#pragma unroll
      for (int rr = 0; rr < kPass; ++rr) {
        const float lt = rows_sum(ls[r0 + rr]);
        const int sr = w * kRows + 16 * rr + i16;
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
          *reinterpret_cast<f4 DCP_LDS*>(osc + sr * kOStride + 16 * db + 4 * g) = acc[r0 + rr][db];
        if (g == 0) {
          mls[sr * 2] = m[r0 + rr];
          mls[sr * 2 + 1] = lt;
        }
      }
      __syncthreads();
#pragma unroll
      for (int rr = 0; rr < kPass; ++rr) {
        const int srow = 16 * rr + (lane >> 2);        // scratch row of this pass
        const int row = 16 * (r0 + rr) + (lane >> 2);  // in the slice; rbase + row in the request
        float mk[4];
        float M = neg_inf();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          mk[k] = mls[(k * kRows + srow) * 2];
          M = max_f(M, mk[k]);
        }
        float L = 0.f;
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float wk = mk[k] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(mk[k] - M);
          L += wk * mls[(k * kRows + srow) * 2 + 1];
          const float DCP_LDS* src = osc + (k * kRows + srow) * kOStride + d0;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const f4 v = *reinterpret_cast<const f4 DCP_LDS*>(src + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[4 * hh + e] += wk * v[e];
          }
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const float lse = L > 0.f ? (M + __log2f(L)) * kLn2 : neg_inf();
        if (rbase + row < R) {
          const int qi_o = (rbase + row) / G;
          const int orow = qi_o * a.hq + kvh * G + (rbase + row - qi_o * G);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] *= inv;
          if (single && a.o_bf16) {
            uint16_t* dstb = static_cast<uint16_t*>(a.o_out) + ((size_t)b * RQ + orow) * D + d0;
            *reinterpret_cast<uint4*>(dstb) =
                make_uint4(f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16),
                           f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16),
                           f32_to_bf16_rne(o[4]) | (f32_to_bf16_rne(o[5]) << 16),
                           f32_to_bf16_rne(o[6]) | (f32_to_bf16_rne(o[7]) << 16));
          } else {
            float* dst = single ? static_cast<float*>(a.o_out) + ((size_t)b * RQ + orow) * D + d0
                                : a.po + ((size_t)item * RQ + orow) * D + d0;
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
          }
          if (tq == 0 && (lane & 3) == 0) {
            if (single) a.lse_out[(size_t)b * RQ + orow] = lse;
            else a.plse[(size_t)item * RQ + orow] = lse;
          }
        }
      }
    }
  } else {
    // running max (log2 units), -m (0 while m is -inf), per-lane share of the running sum,
    // and the lane's NA = 4 dims of each row (16-byte chunk pcl of the V row)
    constexpr int NA = 4;
    float m[HPW], negm[HPW], ls[HPW], acc[HPW][NA];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      m[h] = neg_inf();
      negm[h] = 0.f;
      ls[h] = 0.f;
#pragma unroll
      for (int k = 0; k < NA; ++k) acc[h][k] = 0.f;
    }

    // query of a single head per wave: loaded once into scalar registers
    constexpr bool kQResident = HPW == 1;
    u32x16 qres[kChunks / 4];
    if constexpr (kQResident) {
#pragma unroll
      for (int c = 0; c < kChunks / 4; ++c)
        qres[c] = *reinterpret_cast<const u32x16 DCP_CONST*>(qh + 16 * c);
    }

    // prologue: tiles 0 and 1 in flight (both buffers are free)
    uint64_t vm0 = issue_tile(0);
    const uint64_t vm_first = ntiles > 1 ? issue_tile(1) : 0ull;

    const int pr = lane >> 4, pcl = lane & 15;   // f32 P.V lane: token group, row chunk
    for (int ti = 0; ti < ntiles; ++ti) {
      // this wave's copies of tile ti have landed (loads complete in issue order, so on the
      // first tile only tile 1's copies may still be outstanding); after the barrier every
      // wave's have, and from tile 1 on the buffer of tile ti-1 is free for tile ti+1.  A bare
      // barrier: the fence of __syncthreads would also wait for LDS traffic that needs no
      // ordering here.
      if (ti == 0 && ntiles > 1) wait_vmcnt<kDmaPerWave>();
      else wait_vmcnt<0>();
      asm volatile("s_barrier" ::: "memory");
      const uint64_t vm1 = ti == 0 ? vm_first : (ti + 1 < ntiles ? issue_tile(ti + 1) : 0ull);
      const char DCP_LDS* kb = kvb + (ti % kNBuf) * kBufBytes +
                               (lane >> 2) * kKBlock + (lane & 3) * 16;   // this lane's K row
      const u32x4 DCP_LDS* vt = (const u32x4 DCP_LDS*)(kvb + (ti % kNBuf) * kBufBytes + kKBytes);
      auto kchunk = [&](int c) { return *(const u32x4 DCP_LDS*)(kb + 64 * c); };

      // ---- scores: lane = token
      float s[HPW];
      if constexpr (kQResident) {
        // the whole K row moves to registers at once (64 VGPRs): all 16 reads in flight
        float s2[2] = {0.f, 0.f};
        u32x4 kr[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) kr[c] = kchunk(c);
#pragma unroll
        for (int c = 0; c < kChunks / 4; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t kd = kr[4 * c + e / 4][e % 4];
            const uint32_t qd = qres[c][e];
            s2[e & 1] = fmaf(__uint_as_float(qd), __uint_as_float(kd), s2[e & 1]);
          }
        s[0] = s2[0] + s2[1];
      } else {
        u32x4 krow[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) krow[c] = kchunk(c);
        // 16 query dwords per scalar load, one load ahead of its use; each step is its own
        // scheduling region so that no more than two chunks (32 scalar registers) are live
        constexpr int kQSteps = HPW * (kChunks / 4);
        auto qload = [&](int st) -> u32x16 {
          uint64_t qa = reinterpret_cast<uint64_t>(
              qbase + (size_t)rrow[st / (kChunks / 4)] * (kRowBytes / 4) + 16 * (st % (kChunks / 4)));
          asm volatile("" : "+s"(qa));
          return *reinterpret_cast<const u32x16 DCP_CONST*>(qa);
        };
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
            dst = fmaf(__uint_as_float(qv[st & 1][e]), __uint_as_float(kd), dst);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int h = 0; h < HPW; ++h) s[h] = sacc[h][0] + sacc[h][1];
      }

      // ---- online softmax (base 2); weights to LDS for the P.V lanes.  The running max m
      // only moves when a tile's max exceeds it by more than kRescaleSlack (always on the
      // first tile with a valid token); in between the weights stay below 2^kRescaleSlack and
      // the accumulators are not touched.  The final normalisation by the running sum makes
      // the result exact for any reference m.
      const int jt = j0 + ti * kTile;   // local index of the tile's first token
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        float x = s[h] * a.sl2;
        if (vm0 != ~0ull || jt + kTile > lim_min) {   // partial tile (uniform); the empty asm
          asm volatile("");                            // keeps this a branch
          x = (((vm0 >> lane) & 1) && jt + lane < lim[h]) ? x : neg_inf();
        }
        const float tmax = wave_max_bcast(x);
        if (tmax > m[h] + kRescaleSlack) {   // uniform branch; m = -inf: any valid tile
          const float alpha = __builtin_amdgcn_exp2f(m[h] - tmax);   // m = -inf -> 0
          m[h] = tmax;
          negm[h] = -tmax;
          ls[h] *= alpha;
#pragma unroll
          for (int k = 0; k < NA; ++k) acc[h][k] *= alpha;
        }
        const float p = __builtin_amdgcn_exp2f(x + negm[h]);   // masked: 0
        ls[h] += p;
        pbuf[w][h][lane] = __float_as_uint(p);
      }

      // ---- P.V: lane = (token group pr, 16-byte chunk pcl of the V row)
#pragma unroll
      for (int k = 0; k < kTile / 4; ++k) {
        const u32x4 v = vt[(4 * k + pr) * kChunks + pcl];
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
          const float pp = __uint_as_float(pbuf[w][h][4 * k + pr]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[h][i] = fmaf(pp, __uint_as_float(v[i]), acc[h][i]);
        }
      }
      vm0 = vm1;
    }

    // ---- finalize: O = acc / l, lse = (m + log2 l) ln 2
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const float lt = wave_sum_dpp(ls[h]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? (m[h] + __log2f(lt)) * kLn2 : neg_inf();
      if (!live[h]) continue;   // a repeated row (uniform)
      const int row = rrow[h];
      float* dst = single ? static_cast<float*>(a.o_out) + ((size_t)b * RQ + row) * D
                          : a.po + ((size_t)item * RQ + row) * D;
      uint16_t* dstb = static_cast<uint16_t*>(a.o_out) + ((size_t)b * RQ + row) * D;
      const bool bf16_out = single && a.o_bf16;   // uniform
      // the four token groups of each row chunk are summed across the 16-lane rows
      float o[NA];
#pragma unroll
      for (int k = 0; k < NA; ++k) {
        float v = acc[h][k];
        const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                           false, false);
        v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
        const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                           false, false);
        o[k] = (__uint_as_float(r32[0]) + __uint_as_float(r32[1])) * inv;
      }
      if (pr == 0) {
        if (bf16_out)
          *reinterpret_cast<uint2*>(dstb + 4 * pcl) =
              make_uint2(f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16),
                         f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16));
        else
          *reinterpret_cast<float4*>(dst + 4 * pcl) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (lane == 0) {
        if (single) a.lse_out[(size_t)b * RQ + row] = lse;
        else a.plse[(size_t)item * RQ + row] = lse;
      }
    }
  }
}

// f32: the vector-ALU variant; R = q_len * G query rows per KV head, rows sharing a
// (waves, rows per wave) shape sharing the kernel.
template <int R>
void launch_r(const GqaKArgs& k, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int NW = waves_for(R), HPW = rows_per_wave(R);
  hipExtLaunchKernelGGL((gqa_shard_kernel<false, NW, HPW>), grid, dim3(64 * NW), 0, s, e0, e1,
                        0, k);
}

// Any R <= 64 rows runs on the variant of the next listed size (rows past R repeat the
// last row and are not written).
hipError_t launch_f32(const GqaKArgs& k, int rows, dim3 grid, hipStream_t s, hipEvent_t e0,
                      hipEvent_t e1) {
  if (rows < 1 || rows > 64) return hipErrorInvalidValue;
  if (rows <= 1) launch_r<1>(k, grid, s, e0, e1);
  else if (rows <= 2) launch_r<2>(k, grid, s, e0, e1);
  else if (rows <= 4) launch_r<4>(k, grid, s, e0, e1);
  else if (rows <= 8) launch_r<8>(k, grid, s, e0, e1);
  else if (rows <= 16) launch_r<16>(k, grid, s, e0, e1);
  else if (rows <= 24) launch_r<24>(k, grid, s, e0, e1);
  else if (rows <= 32) launch_r<32>(k, grid, s, e0, e1);
  else if (rows <= 48) launch_r<48>(k, grid, s, e0, e1);
  else launch_r<64>(k, grid, s, e0, e1);
  return hipGetLastError();
}

// bf16: the matrix-core variant, four waves, RT 16-row tiles per wave, one workgroup per
// (item, KV head) or, past 48 rows, per (item, KV head, slice of 32 rows); rows past R pad
// the 16-row tile.  The per-token work,
// 4 R D flops against 4 D bytes of K and V, then stays off the vector ALUs, which did not
// hide entirely under the HBM -> LDS stream at R = 1..8 (measured at the share's shape with
// the vector ALUs doing the bf16 products in v_dot2: 73-76% of HBM peak against 79-82% on
// the matrix cores) and became the bound at R >= 16 (48 / 64 rows: 13% / 10% of HBM peak).
template <int RT>
void launch_m(const GqaKArgs& k, dim3 grid, int slices, hipStream_t s, hipEvent_t e0,
              hipEvent_t e1) {
  const dim3 g(grid.x, grid.y * (unsigned)slices);
  hipExtLaunchKernelGGL((gqa_shard_kernel<true, 4, RT>), g, dim3(256), 0, s, e0, e1, 0,
                        k);
}

hipError_t launch_bf16(const GqaKArgs& k, int rows, dim3 grid, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1) {
  if (rows < 1 || rows > 64) return hipErrorInvalidValue;
  static_assert(kGqaSliceRows <= 48, "at most three 16-row tiles per wave");
  const int slices = gqa_bf16_slices(rows);
  if (slices > 1) launch_m<2>(k, grid, slices, s, e0, e1);
  else if (rows <= 16) launch_m<1>(k, grid, 1, s, e0, e1);
  else if (rows <= 32) launch_m<2>(k, grid, 1, s, e0, e1);
  else launch_m<3>(k, grid, 1, s, e0, e1);
  return hipGetLastError();
}

}  // namespace

// 256-byte rows (bf16 head_dim 128, f32 head_dim 64) and any group of up to 64 query rows
// (q_len * G) per KV head.
hipError_t launch_gqa_shard(const GqaArgs& a, int64_t max_items, const WsPtrs& ws,
                            void* o_out, float* lse_out, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1) {
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
  k.po = static_cast<float*>(ws.po);
  const dim3 grid((unsigned)max_items, (unsigned)a.hkv);
  const int rows = a.rows.q_len * (a.hq / a.hkv);
  return a.dtype == 1 ? launch_bf16(k, rows, grid, stream, ev0, ev1)
                      : launch_f32(k, rows, grid, stream, ev0, ev1);
}

}  // namespace dcp

// gqa_fp8.hip — paged GQA decode attention over one DCP rank's shard, fp8 KV cache (gfx950).
//
// What it computes ("vLLM Decode Context Parallelism for long-context workloads" blog,
// "DCP execution flow", step "Compute", and "GQA backend"): the attention of the gathered
// bf16 queries over the tokens this rank owns, as the bf16 shard kernel does, with the K and
// V pages holding OCP FP8 E4M3 codes and one float32 scale each: a cached value is
// decode(code) * scale.  The pages leave the KV dtype open; this is the lower-byte cache
// variant, half the bytes per token of bf16.
//
// Design (the bf16 kernel's matrix-core variant, re-laid for 128-byte rows):
//   * Four waves per (work item, KV head) for R = q_len * G <= 48 query rows, or per (work
//     item, KV head, slice of 32 rows) for R up to 64, two workgroups per CU; wave w takes
//     token quarter w of every 64-token tile for all rows of the workgroup (one to three
//     16-row tiles, rows past R padding: idle matrix lanes cost nothing in an HBM-bound
//     kernel) and keeps its own online softmax; the quarters merge through LDS by the LSE
//     identity after the last tile, one row tile at a time.
//   * 64-token tiles of K and V rows (8 KiB each) are copied HBM -> LDS by
//     global_load_lds_dwordx4 with the non-temporal policy into a double buffer, paced by
//     each wave's vector-memory counter and a bare s_barrier (a 3-deep ring, two tiles in
//     flight, measured 2% slower).  The 16-byte chunks of a row
//     are XOR-swizzled: K by bits 1-3 of the row, V by bit 2 (see the operand reads).
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16.  The contraction order is free, so k-step
//     ks of lane group g takes dims 32 g + 8 ks .. + 7 for both operands: a lane reads its
//     token's 32 bytes once per tile and converts 8 codes per step to bf16 with
//     v_cvt_scalef32_pk_bf16_fp8 (two codes per instruction, exact).  k_scale folds into
//     the score multiplier.
//   * O^T += V^T . P^T on v_mfma_f32_16x16x16_bf16 with P^T straight from the score
//     registers (lane (g, i16): row i16, tokens 4 g .. 4 g + 3).  The V^T operand (one dim
//     of those four tokens) comes from four 4-byte LDS reads (the four tokens' bytes of dims
//     64 h + 4 i16 .. + 3) and a 4 x 4 byte transpose by v_perm_b32, which yields the
//     operands of four MFMAs at once: MFMA (h, k) has output rows m = dims 64 h + 4 m + k.
//     v_scale multiplies the final output.
#include "launch.h"

namespace dcp {

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(2))) float f2;
typedef __attribute__((ext_vector_type(4))) short s4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
#define DCP_LDS __attribute__((address_space(3)))

constexpr int kTile = kGqaTile;                  // 64 tokens
constexpr int kD = kGqaFp8HeadDim;              // head dim
constexpr int kRow = 128;                        // bytes per cached row (one code per dim)
constexpr int kTileBytes = kTile * kRow;         // 8 KiB of K (and of V) per tile
constexpr int kBufBytes = 2 * kTileBytes;        // K rows, then V rows
constexpr int kNBuf = 2;                         // one computed, one in flight
constexpr int kWaves = 4;
constexpr int kSlots = kBufBytes / 1024;         // 1-KiB copies per tile
constexpr int kDmaPerWave = kSlots / kWaves;     // 4
constexpr float kRescaleSlack = 8.f;

// LDS position of logical 16-byte chunk c of tile row r (an XOR, so also its inverse).
// K: the 16 rows one operand read serves sit at 8 distinct chunk positions, two rows each
// (rows 128 bytes apart), which spreads them over all banks.  V: the four 16-lane groups of
// a read take rows 4 apart; rows of odd r / 4 use the other half of the row.
__device__ __forceinline__ int k_pos(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int v_pos(int r, int c) { return c ^ (((r >> 2) & 1) << 2); }

struct Fp8KArgs {
  const uint16_t* q;   // bf16 [b][q_len * hq][128]
  const char* kp;      // fp8 codes [num_blocks][hkv][B][128]
  const char* vp;
  const int32_t* bt;
  int hq, hkv, block_size, max_blocks;
  uint32_t num_blocks;
  int rank, cp, interleave;
  float sl2;           // scale * k_scale * log2(e)
  float v_scale;
  const int32_t* seq_lens;
  int64_t len_cap;
  int q_len;
  int o_bf16;
  void* o_out;
  float* lse_out;
  int32_t* header;
  const int32_t* off;
  const int4* items;
  float* plse;
  float* po;
};

// Two fp8 codes (bytes 0-1, or 2-3 with kHi) of a dword as a packed bf16 pair.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

template <int RT>
__global__ __launch_bounds__(64 * kWaves, 2) void gqa_fp8_kernel(Fp8KArgs a) {
  constexpr int kOStride = kD + 4;                 // merge scratch: floats per row
  constexpr int kRows = 16;                        // scratch rows per wave (one row tile a pass)
  constexpr int kScratch = kWaves * kRows * kOStride * 4;
  constexpr int kLds = kScratch > kNBuf * kBufBytes ? kScratch : kNBuf * kBufBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kLds];
  __shared__ float mls[kWaves * kRows * 2];        // (m, l) per wave row

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // token quarter
  if ((int)blockIdx.x >= a.header[1]) return;
  const int4 it = a.items[blockIdx.x];   // in dispatch order, longest first
  const int b = it.x, j0 = it.y, j1 = it.z;
  const int item = it.w;
  // blockIdx.y = KV head + hkv * (row slice); the slices of one item share its K / V tiles
  // (a later slice's reads mostly hit L2)
  const int kvh = (int)blockIdx.y % a.hkv;
  const int rbase = 16 * RT * ((int)blockIdx.y / a.hkv);   // first query row of the slice
  // K / V copies stream with the non-temporal policy, except when two slices read the same
  // tiles: the second then finds them in L2
  const bool nt = a.q_len * (a.hq / a.hkv) <= 16 * RT;
  const bool single = (a.off[b + 1] - a.off[b]) == 1;
  const int G = a.hq / a.hkv;
  const int R = a.q_len * G;
  const int RQ = a.q_len * a.hq;
  const int32_t* btb = a.bt + (size_t)b * a.max_blocks;
  const uint32_t B = (uint32_t)a.block_size;
  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  const bool fast = (a.interleave % kTile) == 0 && (a.block_size % kTile) == 0;
  const char DCP_LDS* lds = (const char DCP_LDS*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;

  // ---- copy slots of this wave: slot s = 4 w + k, one 1-KiB copy each: s < 8 brings K rows
  // 8 s .. 8 s + 7, s >= 8 V rows 8 (s - 8) .., lane l the chunk of row 8 s' + l / 8 that
  // belongs at position l mod 8
  uint32_t slot_src[kDmaPerWave];
  int slot_row[kDmaPerWave];
  uint32_t slot_dst[kDmaPerWave];
#pragma unroll
  for (int k = 0; k < kDmaPerWave; ++k) {
    const int s = w * kDmaPerWave + k;
    const bool isk = s < kSlots / 2;
    const int s8 = isk ? s : s - kSlots / 2;
    const int r = 8 * s8 + (lane >> 3), p = lane & 7;
    slot_row[k] = r;
    slot_src[k] = (uint32_t)((isk ? k_pos(r, p) : v_pos(r, p)) * 16);
    slot_dst[k] = __builtin_amdgcn_readfirstlane((uint32_t)((isk ? 0 : kTileBytes) + s8 * 1024));
  }
  auto slot_base = [&](int k) { return (w * kDmaPerWave + k) < kSlots / 2 ? a.kp : a.vp; };

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

  // ---- all of this wave's HBM -> LDS copies of tile ti; returns the mask of valid tokens
  // (rows past the item's end, or of a bad page, re-read a valid row and are masked)
  auto issue_tile = [&](int ti) -> uint64_t {
    const uint32_t dst = lds_addr + (uint32_t)((ti % kNBuf) * kBufBytes);
    if (fast) {
      if ((ti & 63) == 0 && ti > 0) build_table(ti >> 6);
      const int nvalid = min(kTile, j1 - (j0 + ti * kTile));
      const uint32_t row0 = __builtin_amdgcn_readlane(row_tab, ti & 63);
      const bool ok = row0 != ~0u;
      const size_t rb = (size_t)(ok ? row0 : 0u) * kRow;
      const uint32_t lim = ok ? (uint32_t)nvalid : 0u;
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k) {
        const uint32_t voff = (uint32_t)slot_row[k] < lim ? (uint32_t)slot_row[k] * kRow + slot_src[k]
                                                          : slot_src[k];
        if (nt) copy16_sbase<true>(dst + slot_dst[k], voff, slot_base(k) + rb);
        else copy16_sbase<false>(dst + slot_dst[k], voff, slot_base(k) + rb);
      }
      return ok ? (nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1)) : 0ull;
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
      const uint32_t rr = __shfl(row, slot_row[k], 64);
      const char* src = slot_base(k) + (size_t)rr * kRow + slot_src[k];
      if (nt) copy16_vaddr<true>(dst + slot_dst[k], src);
      else copy16_vaddr<false>(dst + slot_dst[k], src);
    }
    return __ballot(ok);
  };

  // ---- this lane's query rows and their visible ends; the query operand of k-step ks is
  // dims 32 g + 8 ks .. + 7 (the K operand's dims of the same step)
  const int g = lane >> 4, i16 = lane & 15;
  const int tq = w;
  int lim_l[RT];
  bf16x8 qop[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int rho = min(rbase + 16 * r + i16, R - 1);
    const int qi = rho / G;
    const int qrow = qi * a.hq + kvh * G + (rho - qi * G);
    lim_l[r] = a.q_len == 1 ? j1
                            : min(j1, row_local_end(a.seq_lens, b, a.len_cap, a.q_len, qi,
                                                    a.rank, a.cp, a.interleave));
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((size_t)b * RQ + qrow) * kD + 32 * g);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qop[r][ks] = __builtin_bit_cast(bf16x8, qp[ks]);
  }
  const int lim_lo = a.q_len == 1 ? j1
                                  : min(j1, row_local_end(a.seq_lens, b, a.len_cap, a.q_len, 0,
                                                          a.rank, a.cp, a.interleave));

  float m[RT], negm[RT], ls[RT];
  f4 acc[RT][kD / 16];   // acc[r][4 h + k][e]: row i16, dim 64 h + 16 g + 4 e + k
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m[r] = neg_inf();
    negm[r] = 0.f;
    ls[r] = 0.f;
#pragma unroll
    for (int d = 0; d < kD / 16; ++d) acc[r][d] = f4{0.f, 0.f, 0.f, 0.f};
  }

  // K operand: row 16 tq + i16, chunks 2 g and 2 g + 1.  V^T operand: rows 16 tq + 4 g + e,
  // the dword of dims 64 h + 4 i16 .. + 3 (chunk 4 h + i16 / 4).
  const int rk = 16 * tq + i16;
  const int koff0 = rk * kRow + 16 * k_pos(rk, 2 * g);
  const int koff1 = rk * kRow + 16 * k_pos(rk, 2 * g + 1);
  int voff[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rv = 16 * tq + 4 * g + e;
      voff[h][e] = kTileBytes + rv * kRow + 16 * v_pos(rv, 4 * h + (i16 >> 2)) + 4 * (i16 & 3);
    }

  uint64_t vm0 = issue_tile(0);
  const uint64_t vm_first = ntiles > 1 ? issue_tile(1) : 0ull;
  for (int ti = 0; ti < ntiles; ++ti) {
    // tile ti has landed in every wave's copies; from tile 1 on the other buffer is free
    if (ti == 0 && ntiles > 1) wait_vmcnt<kDmaPerWave>();
    else wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
    const uint64_t vm1 = ti == 0 ? vm_first : (ti + 1 < ntiles ? issue_tile(ti + 1) : 0ull);
    const char DCP_LDS* tb = lds + (ti % kNBuf) * kBufBytes;

    // ---- S^T of this wave's 16 tokens x 16 rows, per row tile
    const u32x4 kc0 = *reinterpret_cast<const u32x4 DCP_LDS*>(tb + koff0);
    const u32x4 kc1 = *reinterpret_cast<const u32x4 DCP_LDS*>(tb + koff1);
    const uint32_t kw[8] = {kc0.x, kc0.y, kc0.z, kc0.w, kc1.x, kc1.y, kc1.z, kc1.w};
    f4 sc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) sc[r] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 kb = {cvt2<false>(kw[2 * ks]), cvt2<true>(kw[2 * ks]),
                        cvt2<false>(kw[2 * ks + 1]), cvt2<true>(kw[2 * ks + 1])};
      const bf16x8 kop = __builtin_bit_cast(bf16x8, kb);
#pragma unroll
      for (int r = 0; r < RT; ++r)
        sc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[r][ks], sc[r], 0, 0, 0);
    }

    // ---- online softmax (base 2) per row = per lane column; the running max moves only
    // past a slack of kRescaleSlack (per lane, under a wave-uniform branch)
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
        for (int d = 0; d < kD / 16; ++d) acc[r][d] *= alpha;
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

    // ---- O^T += V^T P^T: per half h, the four tokens' dwords of dims 64 h + 4 i16 .. + 3,
    // transposed to one dword per dim (tokens 4 g .. 4 g + 3 in bytes 0..3)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = *reinterpret_cast<const uint32_t DCP_LDS*>(tb + voff[h][e]);
      const uint32_t lo01 = __builtin_amdgcn_perm(t[1], t[0], 0x05010400u);
      const uint32_t hi01 = __builtin_amdgcn_perm(t[1], t[0], 0x07030602u);
      const uint32_t lo23 = __builtin_amdgcn_perm(t[3], t[2], 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(t[3], t[2], 0x07030602u);
      const uint32_t dk[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                              __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                              __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                              __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x2 vb = {cvt2<false>(dk[k]), cvt2<true>(dk[k])};
        const s4 va = __builtin_bit_cast(s4, vb);
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[r][4 * h + k] =
              __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[r], acc[r][4 * h + k], 0, 0, 0);
      }
    }
    vm0 = vm1;
  }

  // ---- merge the four token quarters of each row through LDS, one row tile per pass (the
  // tile buffers are free once every wave has passed the barrier; no copy is in flight).
  // Scratch rows are (wave, lane column), dims in natural order.
  float DCP_LDS* osc = (float DCP_LDS*)smem;
  wait_vmcnt<0>();
  // wave tq finishes dims 32 tq .. 32 tq + 31 of every row
  const int d0 = 32 * tq + 8 * (lane & 3);
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    __syncthreads();   // the tile buffers (first pass) or the previous pass's rows are free
    {
      const float lt = rows_sum(ls[r]);
      const int sr = w * kRows + i16;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f4 v = {acc[r][4 * h][e], acc[r][4 * h + 1][e], acc[r][4 * h + 2][e],
                        acc[r][4 * h + 3][e]};
          *reinterpret_cast<f4 DCP_LDS*>(osc + sr * kOStride + 64 * h + 16 * g + 4 * e) = v;
        }
      if (g == 0) {
        mls[sr * 2] = m[r];
        mls[sr * 2 + 1] = lt;
      }
    }
    __syncthreads();
    const int srow = lane >> 2;                // scratch row of this pass
    const int row = 16 * r + (lane >> 2);      // in the slice; rbase + row in the request
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
    const float inv = L > 0.f ? a.v_scale / L : 0.f;
    const float lse = L > 0.f ? (M + __log2f(L)) * kLn2 : neg_inf();
    if (rbase + row < R) {
      const int qi_o = (rbase + row) / G;
      const int orow = qi_o * a.hq + kvh * G + (rbase + row - qi_o * G);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= inv;
      if (single && a.o_bf16) {
        uint16_t* dstb = static_cast<uint16_t*>(a.o_out) + ((size_t)b * RQ + orow) * kD + d0;
        *reinterpret_cast<uint4*>(dstb) =
            make_uint4(f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16),
                       f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16),
                       f32_to_bf16_rne(o[4]) | (f32_to_bf16_rne(o[5]) << 16),
                       f32_to_bf16_rne(o[6]) | (f32_to_bf16_rne(o[7]) << 16));
      } else {
        float* dst = single ? static_cast<float*>(a.o_out) + ((size_t)b * RQ + orow) * kD + d0
                            : a.po + ((size_t)item * RQ + orow) * kD + d0;
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

}  // namespace

hipError_t launch_gqa_fp8_shard(const GqaArgs& a, float k_scale, float v_scale,
                                int64_t max_items, const WsPtrs& ws, void* o_out,
                                float* lse_out, hipStream_t stream, hipEvent_t ev0,
                                hipEvent_t ev1) {
  Fp8KArgs k;
  k.q = static_cast<const uint16_t*>(a.q);
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
  k.sl2 = a.scale * k_scale * kLog2e;
  k.v_scale = v_scale;
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
  const int rows = a.rows.q_len * (a.hq / a.hkv);
  if (rows < 1 || rows > 64) return hipErrorInvalidValue;
  // rows past one workgroup's share run as 32-row slices (the planner sized the items so)
  const int slices = gqa_bf16_slices(rows);
  const dim3 grid((unsigned)max_items, (unsigned)(a.hkv * slices));
  if (slices == 1 && rows <= 16)
    hipExtLaunchKernelGGL((gqa_fp8_kernel<1>), grid, dim3(64 * kWaves), 0, stream, ev0, ev1, 0, k);
  else if (slices > 1 || rows <= 32)
    hipExtLaunchKernelGGL((gqa_fp8_kernel<2>), grid, dim3(64 * kWaves), 0, stream, ev0, ev1, 0, k);
  else
    hipExtLaunchKernelGGL((gqa_fp8_kernel<3>), grid, dim3(64 * kWaves), 0, stream, ev0, ev1, 0, k);
  return hipGetLastError();
}

}  // namespace dcp

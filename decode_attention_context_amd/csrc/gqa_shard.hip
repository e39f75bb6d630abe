// gqa_shard.hip — paged GQA decode attention over one DCP rank's KV shard (gfx950).
//
// What it computes ("vLLM Decode Context Parallelism for long-context workloads" blog,
// "DCP execution flow", step "Compute", and "GQA backend"): for every request b and query
// head h, the attention of the gathered query q[b][h] over the tokens t < seq_len[b] that
// this rank owns ((t / interleave) mod cp_size == rank), reading KV head h / G, together
// with the natural-log LSE of the scaled scores, so that the partials of all ranks merge
// into exact attention.
//
// Design (HBM-bound: 2 * D * sizeof(T) bytes and 4 * G * D flops per token and KV head):
//   * One wave per work item: a (request, KV head, local token range).  The planner sizes
//     items so that the grid covers every CU several times.
//   * Tiles of 64 local tokens.  The block-table walk gives each lane the cache row of one
//     token; whole rows (256 B) are loaded with coalesced 16-B loads (each load
//     instruction covers 4 complete rows, the row index comes from the owning lane by a
//     lane shuffle) and staged in LDS with an XOR swizzle of the 16-B chunks so that the
//     transposed reads below are bank-conflict free.  The next tile's rows are loaded into
//     registers while the current tile is processed.
//   * Scores: lane = token.  Each lane reads its own K row from LDS chunk by chunk; the G
//     query heads are wave-uniform, so they come from scalar loads and the inner product
//     is one v_dot2_f32_bf16 (bf16) or v_fma_f32 (f32) per element pair with no cross-lane
//     reduction.
//   * Online softmax in base 2 (scale * log2 e folded into the scores): the tile max per
//     head is a wave butterfly; the running sum stays per lane and is reduced once at the
//     end of the item.
//   * P.V: lane = one dword of every V row (2 bf16 dims or 1 f32 dim).  For bf16, token
//     pairs (2k, 2k+1) are packed with v_perm_b32 into (v[2k][d], v[2k+1][d]) and combined
//     with the bf16-rounded weight pairs by v_dot2_f32_bf16 into fp32 accumulators; the
//     weights are broadcast through LDS.
//   * An item that covers a request's whole shard writes (O, lse) directly; otherwise it
//     writes a normalized partial that the split combine merges.
#include "launch.h"

namespace dcp {

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;  // register-friendly 16 B

constexpr int kTile = kGqaTile;  // tokens per tile (= lanes)
constexpr int kRowBytes = 256;   // D * sizeof(T) for the supported shapes
constexpr int kChunks = kRowBytes / 16;
constexpr int kRowsPerLoad = 64 / kChunks;

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

template <bool kBf16, int G>
__global__ __launch_bounds__(64) void gqa_shard_kernel(GqaKArgs a) {
  constexpr int kElemBytes = kBf16 ? 2 : 4;
  constexpr int D = kRowBytes / kElemBytes;     // head dim
  constexpr int E = 16 / kElemBytes;            // elements per 16-B chunk
  constexpr int NA = kBf16 ? 2 : 1;             // accumulators per lane per head

  __shared__ u32x4 tile[kTile * kChunks];       // 16 KiB: K rows, then V rows
  __shared__ uint32_t pbuf[kTile * G];          // softmax weights for P.V

  const int lane = threadIdx.x;
  const int item = blockIdx.x;
  if (item >= a.header[1]) return;
  const int4 it = a.items[item];
  const int b = it.x, j0 = it.y, j1 = it.z;
  const int kvh = blockIdx.y;
  const bool single = (a.off[b + 1] - a.off[b]) == 1;
  // The query heads are wave-uniform and read-only: address them in the constant address
  // space so that they are fetched by scalar loads and used as scalar operands.
  const u32x4 __attribute__((address_space(4)))* qh =
      reinterpret_cast<const u32x4 __attribute__((address_space(4)))*>(
          reinterpret_cast<uintptr_t>(a.q)) +
      ((size_t)b * a.hq + (size_t)kvh * G) * (D * kElemBytes / 16);
  const int32_t* btb = a.bt + (size_t)b * a.max_blocks;
  const uint32_t B = (uint32_t)a.block_size;

  float m[G], ls[G], acc[G][NA];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = neg_inf();
    ls[h] = 0.f;
#pragma unroll
    for (int k = 0; k < NA; ++k) acc[h][k] = 0.f;
  }

  uint32_t row = 0;
  bool valid = false;
  // Cache row (page * Hkv + kvh) * B + slot of local token tj + lane.
  auto rows_for = [&](int tj) {
    const int j = tj + lane;
    valid = j < j1;
    row = 0;
    bool bad = false;
    if (valid) {
      const uint32_t t = dcp_walk_global_pos((uint32_t)j, a.rank, a.cp, a.interleave);
      const uint32_t lp = t / B;
      const int32_t pg = btb[lp];
      if (pg < 0 || (uint32_t)pg >= a.num_blocks) {
        valid = false;
        bad = true;
      } else {
        row = ((uint32_t)pg * a.hkv + kvh) * B + (t - lp * B);
      }
    }
    if (__ballot(bad) != 0 && lane == 0) atomicOr(&a.header[0], kErrBlockId);
  };
  u32x4 kr[kChunks], vr[kChunks];
#define DCP_LOAD_ROWS(base, r)                                                                \
  _Pragma("unroll") for (int i = 0; i < kChunks; ++i) {                                      \
    const uint32_t rr = __shfl(row, kRowsPerLoad * i + lane / kChunks, 64);                  \
    r[i] = *reinterpret_cast<const u32x4*>((base) + (size_t)rr * kRowBytes + (lane % kChunks) * 16); \
  }
#define DCP_STORE_ROWS(r)                                                                     \
  _Pragma("unroll") for (int i = 0; i < kChunks; ++i) {                                      \
    const int rw = kRowsPerLoad * i + lane / kChunks;                                         \
    tile[rw * kChunks + ((lane % kChunks) ^ (rw & 15))] = r[i];                               \
  }

  rows_for(j0);
  DCP_LOAD_ROWS(a.kp, kr);
  DCP_LOAD_ROWS(a.vp, vr);
  for (int tj = j0;; tj += kTile) {
    DCP_STORE_ROWS(kr);
    __syncthreads();
    const bool cur_valid = valid;
    const bool has_next = tj + kTile < j1;
    if (has_next) {
      rows_for(tj + kTile);
      DCP_LOAD_ROWS(a.kp, kr);
    }

    // ---- scores: lane = token
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const u32x4 kc = tile[lane * kChunks + (c ^ (lane & 15))];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const u32x4 qc = qh[(h * D + c * E) * kElemBytes / 16];
        if constexpr (kBf16) {
          s[h] = dot2_bf16(qc.x, kc.x, s[h]);
          s[h] = dot2_bf16(qc.y, kc.y, s[h]);
          s[h] = dot2_bf16(qc.z, kc.z, s[h]);
          s[h] = dot2_bf16(qc.w, kc.w, s[h]);
        } else {
          s[h] = fmaf(__uint_as_float(qc.x), __uint_as_float(kc.x), s[h]);
          s[h] = fmaf(__uint_as_float(qc.y), __uint_as_float(kc.y), s[h]);
          s[h] = fmaf(__uint_as_float(qc.z), __uint_as_float(kc.z), s[h]);
          s[h] = fmaf(__uint_as_float(qc.w), __uint_as_float(kc.w), s[h]);
        }
      }
    }

    // ---- online softmax (base 2)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x = cur_valid ? s[h] * a.sl2 : neg_inf();
      const float mn = fmaxf(m[h], wave_max(x));
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
        reinterpret_cast<uint16_t*>(pbuf)[((lane >> 1) * G + h) * 2 + (lane & 1)] =
            (uint16_t)f32_to_bf16_rne(p);
      } else {
        pbuf[lane * G + h] = __float_as_uint(p);
      }
    }
    __syncthreads();
    DCP_STORE_ROWS(vr);
    __syncthreads();
    if (has_next) {
      DCP_LOAD_ROWS(a.vp, vr);
    }

    // ---- P.V: lane = one dword of every V row
    const uint32_t* tw = reinterpret_cast<const uint32_t*>(tile);
    const int cw = lane >> 2, ww = lane & 3;
    if constexpr (kBf16) {
#pragma unroll 4
      for (int k = 0; k < kTile / 2; ++k) {
        const int r0 = 2 * k, r1 = 2 * k + 1;
        const uint32_t v0 = tw[(r0 * kChunks + (cw ^ (r0 & 15))) * 4 + ww];
        const uint32_t v1 = tw[(r1 * kChunks + (cw ^ (r1 & 15))) * 4 + ww];
        const uint32_t lo = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint32_t pp = pbuf[k * G + h];
          acc[h][0] = dot2_bf16(pp, lo, acc[h][0]);
          acc[h][1] = dot2_bf16(pp, hi, acc[h][1]);
        }
      }
    } else {
#pragma unroll 4
      for (int t = 0; t < kTile; ++t) {
        const float v = __uint_as_float(tw[(t * kChunks + (cw ^ (t & 15))) * 4 + ww]);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][0] = fmaf(__uint_as_float(pbuf[t * G + h]), v, acc[h][0]);
      }
    }
    __syncthreads();
    if (!has_next) break;
  }
#undef DCP_LOAD_ROWS
#undef DCP_STORE_ROWS

  // ---- finalize: O = acc / l, lse = (m + log2 l) ln 2
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lt = wave_sum(ls[h]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (m[h] + __log2f(lt)) * kLn2 : neg_inf();
    const int head = kvh * G + h;
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
    case 1: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 1>), grid, dim3(64), 0, s, k); break;
    case 2: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 2>), grid, dim3(64), 0, s, k); break;
    case 4: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 4>), grid, dim3(64), 0, s, k); break;
    case 8: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 8>), grid, dim3(64), 0, s, k); break;
    case 16: hipLaunchKernelGGL((gqa_shard_kernel<kBf16, 16>), grid, dim3(64), 0, s, k); break;
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

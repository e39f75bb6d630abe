// host_rules.h — the host-side rules of the library, free of any GPU call: argument
// validation of every entry point, the supported-shape predicates, the work-item target of
// a shard call and the workspace layout it sizes.  dcp_api.cpp applies them before any
// launch; being plain C++ (integer arithmetic on the arguments only), they also build with
// a host compiler under address and undefined-behaviour sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "dcp_attn.h"
#include "walker.h"

namespace dcp {

// Tokens per tile of each shard kernel (work items are whole multiples of it).
constexpr int kGqaTile = 64;
constexpr int kMlaTile = 32;
// Most query positions per request (multi-token decode).
constexpr int kMaxQLen = 4;
// Bytes of one GQA K or V row the vector and matrix-core kernels are written for.
constexpr int kGqaRowBytes = 256;
// bf16 GQA: query rows (q_len x group) one workgroup takes per item and KV head (up to three
// 16-row tiles per wave); more rows are cut into slices of 32, one workgroup each
constexpr int kGqaSliceRows = 48;
inline int gqa_bf16_slices(int rows) { return rows > kGqaSliceRows ? (rows + 31) / 32 : 1; }
// Head dim of the fp8-cache GQA kernel.
constexpr int kGqaFp8HeadDim = 128;
// MLA shape ("The memory wall in long-context inference", MLA item): the query heads read
// one 576-wide latent row per token, the first 512 columns of which are the value.  The
// gathered heads of a DCP group: 128 (e.g. 16 per rank under tensor parallelism 8, gathered
// over a DCP group of 8), or 64, 32, 16 for smaller DCP groups.
inline bool mla_heads_supported(int h) { return h == 16 || h == 32 || h == 64 || h == 128; }
constexpr int kMlaDk = 576;
constexpr int kMlaDv = 512;

constexpr int64_t kMaxI32 = 2147483647;

// ---------------------------------------------------------------------------------------
// Workspace layout (every section 256-byte aligned).  Written by the planner, read by the
// shard kernels and the split combine of the same call.
//   header  int32[64]: [0] device error word, [1] number of work items, [2] tokens per item
//   off     int32[batch + 1]: first work item of each request (prefix sum)
//   items   int4[max_items]: (request, local token begin, local token end, partial index),
//           in dispatch order (longest first); a request's partials have consecutive
//           indices off[b] .. off[b+1)
//   plse    float[max_items * rows]:      per-partial log-sum-exp (natural log)
//   po      [max_items * rows * Dv]:      per-partial normalized output, float32 (GQA) or
//                                         bf16 rounded to nearest even (MLA: 128 KiB per
//                                         item and position instead of 256 KiB)
// (rows = query rows per request: q_len * Hq)
// ---------------------------------------------------------------------------------------
struct WsLayout {
  size_t off_off, items_off, plse_off, po_off, total;
  int po_bf16;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline WsLayout ws_layout(int batch, int64_t max_items, int rows, int dv, bool po_bf16) {
  WsLayout w;
  w.po_bf16 = po_bf16 ? 1 : 0;
  w.off_off = 256;
  w.items_off = w.off_off + align256(sizeof(int32_t) * ((size_t)batch + 1));
  w.plse_off = w.items_off + align256(sizeof(int32_t) * 4 * (size_t)max_items);
  w.po_off = w.plse_off + align256(sizeof(float) * (size_t)max_items * rows);
  w.total = w.po_off + align256((po_bf16 ? 2 : 4) * (size_t)max_items * rows * dv);
  return w;
}

// GQA shapes the shard kernels take: 256-byte rows (bf16 D 128 on the matrix cores, f32 D 64
// on the vector ALUs), q_len 1..4 and at most 64 query rows (q_len * group) per KV head.
inline bool gqa_supported(int dtype, int head_dim, int group, int q_len) {
  if (dtype != DCP_F32 && dtype != DCP_BF16) return false;
  const int64_t elem = dtype == DCP_BF16 ? 2 : 4;
  if ((int64_t)head_dim * elem != kGqaRowBytes) return false;
  if (q_len < 1 || q_len > kMaxQLen || group < 1) return false;
  return (int64_t)group * q_len <= 64;
}

// fp8 KV cache (bf16 queries): head dim 128, at most 64 query rows per KV head.
inline bool gqa_fp8_supported(int head_dim, int group, int q_len) {
  if (head_dim != kGqaFp8HeadDim || q_len < 1 || q_len > kMaxQLen || group < 1) return false;
  return (int64_t)group * q_len <= 64;
}

// Shape checks shared by the size query and the shard call.
inline int check_desc(const dcp_attn_desc* d, int q_len, int batch, int64_t max_seq_len, int cp,
                      int il) {
  if (!d || batch < 0 || max_seq_len < 0 || max_seq_len > kMaxI32) return DCP_EINVAL;
  if (q_len < 1) return DCP_EINVAL;
  if (q_len > kMaxQLen) return DCP_EUNSUPPORTED;
  if (cp < 1 || il < 1 || (int64_t)cp * il > kMaxI32) return DCP_EINVAL;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads) return DCP_EINVAL;
  if (d->head_dim_qk < 1 || d->head_dim_v < 1 || d->block_size < 1 || d->max_blocks_per_seq < 1 ||
      d->num_blocks < 1)
    return DCP_EINVAL;
  // cache rows below 2^31 (each factor is at least 1, so dividing keeps the test exact)
  if (d->num_blocks > kMaxI32 / ((int64_t)d->block_size * d->num_kv_heads)) return DCP_EUNSUPPORTED;
  if ((int64_t)d->max_blocks_per_seq * d->block_size > kMaxI32) return DCP_EUNSUPPORTED;
  // query and output elements of one request below 2^31
  if ((int64_t)q_len * d->num_q_heads * std::max(d->head_dim_qk, d->head_dim_v) > kMaxI32)
    return DCP_EUNSUPPORTED;
  if (d->dtype != DCP_F32 && d->dtype != DCP_BF16) return DCP_EINVAL;
  if (d->kind == DCP_GQA) {
    if (d->head_dim_qk != d->head_dim_v) return DCP_EUNSUPPORTED;
    if (!gqa_supported(d->dtype, d->head_dim_qk, d->num_q_heads / d->num_kv_heads, q_len))
      return DCP_EUNSUPPORTED;
  } else if (d->kind == DCP_MLA) {
    if (d->dtype != DCP_BF16 || !mla_heads_supported(d->num_q_heads) || d->num_kv_heads != 1 ||
        d->head_dim_qk != kMlaDk || d->head_dim_v != kMlaDv)
      return DCP_EUNSUPPORTED;
  } else {
    return DCP_EINVAL;
  }
  return DCP_OK;
}

struct Plan {
  int64_t target = 0;
  int tile = kGqaTile;
  int min_chunk = kGqaTile;
  int64_t max_items = 0;
  WsLayout lay{};
};

// Work items of a shard call on a device with `cus` compute units (desc already checked):
// the planner splits the shard's tokens into about `target` items (never more than
// target + batch), about one round of workgroups over the CUs (GQA: one workgroup per
// item and KV head; MLA: one workgroup per item and query position).  Partials are kept
// per query row: q_len * num_q_heads rows per item.
inline bool make_plan(const dcp_attn_desc* d, int q_len, int batch, int cus, Plan* p) {
  if (cus <= 0) return false;
  if (d->kind == DCP_GQA) {
    p->tile = kGqaTile;
    // two resident workgroups (64 KiB double buffer each) per CU and KV head, one round;
    // bf16 queries with more rows per KV head than one workgroup takes run as 32-row slices,
    // one workgroup each per item and KV head, so proportionally fewer items
    const int rows = q_len * (d->num_q_heads / d->num_kv_heads);
    const int slices = d->dtype == DCP_BF16 ? gqa_bf16_slices(rows) : 1;
    p->target = std::max<int64_t>(1, (int64_t)cus * 2 / ((int64_t)d->num_kv_heads * slices));
    p->min_chunk = kGqaTile;
  } else {
    // one workgroup (all heads) per item and query position, one resident workgroup per CU
    // (144 KiB of LDS)
    p->tile = kMlaTile;
    p->target = std::max<int64_t>(1, (int64_t)cus / q_len);
    p->min_chunk = 4 * kMlaTile;
  }
  p->max_items = (int64_t)batch + p->target;
  // MLA split partials in bf16 (the GQA ones are a few KiB per item and stay float32)
  p->lay = ws_layout(batch, p->max_items, q_len * d->num_q_heads, d->head_dim_v,
                     d->kind == DCP_MLA);
  return true;
}

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// fp8 KV cache of a GQA shard call: K / V pages hold fp8 codes, values code * scale.
struct KvFp8 {
  float k_scale, v_scale;
};

// Every check of a shard call before its launches, in order; on DCP_OK with batch > 0,
// *plan holds the work plan and the workspace is large enough for it.  `cus()` returns the
// device's compute-unit count (0 if it could not be read: DCP_ELAUNCH); it is called only
// once every argument has passed.
template <class CusFn>
inline int check_shard_args(const dcp_attn_desc* d, int q_len, int o_dtype, const void* q,
                            const void* kv, const void* v, const int32_t* bt,
                            const int32_t* lens, int batch, int64_t max_seq_len, int rank,
                            int cp, int il, float scale, const void* o, const float* lse,
                            const void* ws, size_t ws_bytes, const KvFp8* fp8, CusFn&& cus,
                            Plan* plan) {
  const int st = check_desc(d, q_len, batch, max_seq_len, cp, il);
  if (st != DCP_OK) return st;
  if (fp8) {
    if (d->kind != DCP_GQA || d->dtype != DCP_BF16) return DCP_EUNSUPPORTED;
    if (!gqa_fp8_supported(d->head_dim_qk, d->num_q_heads / d->num_kv_heads, q_len))
      return DCP_EUNSUPPORTED;
    if (!std::isfinite(fp8->k_scale) || !std::isfinite(fp8->v_scale)) return DCP_EINVAL;
  }
  if (o_dtype != DCP_F32 && o_dtype != DCP_BF16) return DCP_EINVAL;
  if (rank < 0 || rank >= cp || !std::isfinite(scale)) return DCP_EINVAL;
  if (batch == 0) return DCP_OK;
  if (!q || !kv || !bt || !lens || !o || !lse) return DCP_EINVAL;
  if (d->kind == DCP_GQA ? v == nullptr : v != nullptr) return DCP_EINVAL;
  if (!aligned(q, 16) || !aligned(kv, 16) || (v && !aligned(v, 16)) || !aligned(o, 16))
    return DCP_EINVAL;
  if (!make_plan(d, q_len, batch, cus(), plan)) return DCP_ELAUNCH;
  if (!ws || !aligned(ws, 256) || ws_bytes < plan->lay.total) return DCP_EWORKSPACE;
  return DCP_OK;
}

// Checks of a merge call before its launch (DCP_OK with batch == 0: nothing to do).
inline int check_merge_args(const void* o_partials, int in_dtype, const float* lse_partials,
                            int cp_size, int batch, int num_heads, int head_dim_v,
                            const void* o_out, int out_dtype) {
  if (cp_size < 1 || batch < 0 || num_heads < 1 || head_dim_v < 1) return DCP_EINVAL;
  if (out_dtype != DCP_F32 && out_dtype != DCP_BF16) return DCP_EINVAL;
  if (in_dtype != DCP_F32 && in_dtype != DCP_BF16) return DCP_EINVAL;
  // each factor is at least 1: the product stays below 2^40 exactly when this holds
  if ((int64_t)batch * num_heads > ((int64_t)1 << 40) / ((int64_t)head_dim_v * cp_size))
    return DCP_EUNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!o_partials || !lse_partials || !o_out) return DCP_EINVAL;
  if (!aligned(o_partials, 16) || !aligned(o_out, 16)) return DCP_EINVAL;
  return DCP_OK;
}

// Checks of a shard-slots call before its launch.
inline int check_slots_args(const int32_t* block_table, const int32_t* seq_lens, int batch,
                            int max_blocks_per_seq, int block_size, int64_t num_blocks,
                            int rank, int cp_size, int interleave, const int64_t* out_offsets,
                            const int64_t* slots_out, const void* workspace) {
  if (batch < 0 || max_blocks_per_seq < 1 || block_size < 1 || num_blocks < 1) return DCP_EINVAL;
  if (cp_size < 1 || interleave < 1 || rank < 0 || rank >= cp_size) return DCP_EINVAL;
  if ((int64_t)cp_size * interleave > kMaxI32 ||
      (int64_t)max_blocks_per_seq * block_size > kMaxI32)
    return DCP_EUNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!block_table || !seq_lens || !out_offsets || !slots_out) return DCP_EINVAL;
  if (!workspace || !aligned(workspace, 256)) return DCP_EWORKSPACE;
  return DCP_OK;
}

}  // namespace dcp

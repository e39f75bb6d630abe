// dcp_api.cpp — the C ABI of include/dcp_attn.h: argument validation, workspace sizing
// and the launch sequence of a shard call (plan -> shard kernel -> split combine).
#include <algorithm>
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "api_internal.h"
#include "dcp_attn.h"
#include "launch.h"

namespace {

using dcp::WsLayout;

constexpr int64_t kMaxI32 = 2147483647;

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks shared by the size query and the shard call.
int check_desc(const dcp_attn_desc* d, int q_len, int batch, int64_t max_seq_len, int cp,
               int il) {
  if (!d || batch < 0 || max_seq_len < 0 || max_seq_len > kMaxI32) return DCP_EINVAL;
  if (q_len < 1) return DCP_EINVAL;
  if (q_len > dcp::kMaxQLen) return DCP_EUNSUPPORTED;
  if (cp < 1 || il < 1 || (int64_t)cp * il > kMaxI32) return DCP_EINVAL;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads) return DCP_EINVAL;
  if (d->head_dim_qk < 1 || d->head_dim_v < 1 || d->block_size < 1 || d->max_blocks_per_seq < 1 ||
      d->num_blocks < 1)
    return DCP_EINVAL;
  if (d->num_blocks * (int64_t)d->block_size * d->num_kv_heads > kMaxI32) return DCP_EUNSUPPORTED;
  if ((int64_t)d->max_blocks_per_seq * d->block_size > kMaxI32) return DCP_EUNSUPPORTED;
  if (d->dtype != DCP_F32 && d->dtype != DCP_BF16) return DCP_EINVAL;
  if (d->kind == DCP_GQA) {
    if (d->head_dim_qk != d->head_dim_v) return DCP_EUNSUPPORTED;
    if (!dcp::gqa_supported(d->dtype, d->head_dim_qk, d->num_q_heads / d->num_kv_heads, q_len))
      return DCP_EUNSUPPORTED;
  } else if (d->kind == DCP_MLA) {
    if (d->dtype != DCP_BF16 || d->num_q_heads != 128 || d->num_kv_heads != 1 ||
        d->head_dim_qk != 576 || d->head_dim_v != 512)
      return DCP_EUNSUPPORTED;
  } else {
    return DCP_EINVAL;
  }
  return DCP_OK;
}

struct Plan {
  int64_t target = 0;
  int tile = 64;
  int min_chunk = 64;
  int64_t max_items = 0;
  WsLayout lay{};
};

// Work items: the planner splits the shard's tokens into about `target` items (never more
// than target + batch), about one round of workgroups over the CUs (GQA: one workgroup per
// item and KV head; MLA: one workgroup per item and query position).  Partials are kept per query row: q_len * num_q_heads rows per item.
bool make_plan(const dcp_attn_desc* d, int q_len, int batch, Plan* p) {
  const int cus = device_cus();
  if (cus <= 0) return false;
  if (d->kind == DCP_GQA) {
    p->tile = dcp::kGqaTile;
    // two resident workgroups (64 KiB double buffer each) per CU and KV head, one round;
    // bf16 queries with more than 32 rows per KV head take two workgroups (32-row slices)
    // per item and KV head, so half the items
    const int rows = q_len * (d->num_q_heads / d->num_kv_heads);
    const int slices = (d->dtype == DCP_BF16 && rows > 32) ? 2 : 1;
    p->target = std::max<int64_t>(1, (int64_t)cus * 2 / (d->num_kv_heads * slices));
    p->min_chunk = dcp::kGqaTile;
  } else {
    // one workgroup (all heads) per item and query position, one resident workgroup per CU
    // (144 KiB of LDS)
    p->tile = dcp::kMlaTile;
    p->target = std::max<int64_t>(1, (int64_t)cus / q_len);
    p->min_chunk = 4 * dcp::kMlaTile;
  }
  p->max_items = (int64_t)batch + p->target;
  // MLA split partials in bf16 (the GQA ones are a few KiB per item and stay float32)
  p->lay = dcp::ws_layout(batch, p->max_items, q_len * d->num_q_heads, d->head_dim_v,
                          d->kind == DCP_MLA);
  return true;
}

// fp8 KV cache of a GQA shard call: K / V pages hold fp8 codes, values code * scale.
struct KvFp8 {
  float k_scale, v_scale;
};

int shard_impl(const dcp_attn_desc* d, int q_len, int o_dtype, const void* q, const void* kv,
               const void* v, const int32_t* bt, const int32_t* lens, int batch,
               int64_t max_seq_len, int rank, int cp, int il, float scale, void* o, float* lse,
               void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
               const KvFp8* fp8 = nullptr) {
  int st = check_desc(d, q_len, batch, max_seq_len, cp, il);
  if (st != DCP_OK) return st;
  if (fp8) {
    if (d->kind != DCP_GQA || d->dtype != DCP_BF16) return DCP_EUNSUPPORTED;
    if (!dcp::gqa_fp8_supported(d->head_dim_qk, d->num_q_heads / d->num_kv_heads, q_len))
      return DCP_EUNSUPPORTED;
    if (!std::isfinite(fp8->k_scale) || !std::isfinite(fp8->v_scale)) return DCP_EINVAL;
  }
  if (o_dtype != DCP_F32 && o_dtype != DCP_BF16) return DCP_EINVAL;
  const int o_bf16 = o_dtype == DCP_BF16;
  if (rank < 0 || rank >= cp || !std::isfinite(scale)) return DCP_EINVAL;
  if (batch == 0) return DCP_OK;
  if (!q || !kv || !bt || !lens || !o || !lse) return DCP_EINVAL;
  if (d->kind == DCP_GQA ? v == nullptr : v != nullptr) return DCP_EINVAL;
  if (!aligned(q, 16) || !aligned(kv, 16) || (v && !aligned(v, 16)) || !aligned(o, 16))
    return DCP_EINVAL;
  Plan p;
  if (!make_plan(d, q_len, batch, &p)) return DCP_ELAUNCH;
  if (!ws || !aligned(ws, 256) || ws_bytes < p.lay.total) return DCP_EWORKSPACE;
  const dcp::WsPtrs w = dcp::ws_ptrs(ws, p.lay);
  const int64_t len_cap = (int64_t)d->max_blocks_per_seq * d->block_size;
  const dcp::RowArgs rows{lens, len_cap, q_len};

  hipError_t e = dcp::launch_plan(lens, batch, rank, cp, il, len_cap, p.target, p.tile,
                                  p.min_chunk, w, stream);
  if (e != hipSuccess) return DCP_ELAUNCH;
  if (d->kind == DCP_GQA) {
    dcp::GqaArgs a{q, kv, v, bt, d->num_q_heads, d->num_kv_heads, d->head_dim_qk, d->block_size,
                   d->max_blocks_per_seq, d->num_blocks, rank, cp, il, scale, d->dtype, rows,
                   o_bf16};
    e = fp8 ? dcp::launch_gqa_fp8_shard(a, fp8->k_scale, fp8->v_scale, p.max_items, w, o, lse,
                                        stream, ev0, ev1)
            : dcp::launch_gqa_shard(a, p.max_items, w, o, lse, stream, ev0, ev1);
  } else {
    dcp::MlaArgs a{q, kv, bt, d->block_size, d->max_blocks_per_seq, d->num_blocks,
                   rank, cp, il, scale, rows, o_bf16};
    e = dcp::launch_mla_shard(a, p.max_items, w, o, lse, stream, ev0, ev1);
  }
  if (e != hipSuccess) return DCP_ELAUNCH;
  e = dcp::launch_split_combine(w, batch, q_len * d->num_q_heads, d->head_dim_v, o, o_bf16, lse,
                                stream);
  return e == hipSuccess ? DCP_OK : DCP_ELAUNCH;
}

}  // namespace

int dcp::shard_call(const dcp_attn_desc* desc, int q_len, int o_dtype, const void* q,
                    const void* kv_pages, const void* v_pages, const int32_t* block_table,
                    const int32_t* seq_lens, int batch, int64_t max_seq_len, int rank,
                    int cp_size, int interleave, float scale, void* o_partial, float* lse,
                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                    hipEvent_t ev_begin, hipEvent_t ev_end) {
  return shard_impl(desc, q_len, o_dtype, q, kv_pages, v_pages, block_table, seq_lens, batch,
                    max_seq_len, rank, cp_size, interleave, scale, o_partial, lse, workspace,
                    workspace_bytes, stream, ev_begin, ev_end);
}

extern "C" {

size_t dcp_workspace_size_mq(const dcp_attn_desc* desc, int q_len, int batch,
                             int64_t max_seq_len, int cp_size, int interleave) {
  if (check_desc(desc, q_len, batch, max_seq_len, cp_size, interleave) != DCP_OK) return 0;
  Plan p;
  if (!make_plan(desc, q_len, batch, &p)) return 0;
  return p.lay.total;
}

size_t dcp_workspace_size(const dcp_attn_desc* desc, int batch, int64_t max_seq_len,
                          int cp_size, int interleave) {
  return dcp_workspace_size_mq(desc, 1, batch, max_seq_len, cp_size, interleave);
}

int dcp_attn_shard(const dcp_attn_desc* desc, const void* q, const void* kv_pages,
                   const void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                   int batch, int64_t max_seq_len, int rank, int cp_size, int interleave,
                   float scale, float* o_partial, float* lse, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return shard_impl(desc, 1, DCP_F32, q, kv_pages, v_pages, block_table, seq_lens, batch,
                    max_seq_len, rank, cp_size, interleave, scale, o_partial, lse, workspace,
                    workspace_bytes, stream, nullptr, nullptr);
}

int dcp_attn_shard_ex(const dcp_attn_desc* desc, int q_len, int o_dtype, const void* q,
                      const void* kv_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* seq_lens, int batch, int64_t max_seq_len, int rank,
                      int cp_size, int interleave, float scale, void* o_partial, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t ev_begin, hipEvent_t ev_end) {
  return shard_impl(desc, q_len, o_dtype, q, kv_pages, v_pages, block_table, seq_lens, batch,
                    max_seq_len, rank, cp_size, interleave, scale, o_partial, lse, workspace,
                    workspace_bytes, stream, ev_begin, ev_end);
}

int dcp_attn_shard_fp8kv(const dcp_attn_desc* desc, int q_len, int o_dtype, const void* q,
                         const void* k_pages, const void* v_pages, float k_scale,
                         float v_scale, const int32_t* block_table, const int32_t* seq_lens,
                         int batch, int64_t max_seq_len, int rank, int cp_size, int interleave,
                         float scale, void* o_partial, float* lse, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, hipEvent_t ev_begin,
                         hipEvent_t ev_end) {
  const KvFp8 f{k_scale, v_scale};
  return shard_impl(desc, q_len, o_dtype, q, k_pages, v_pages, block_table, seq_lens, batch,
                    max_seq_len, rank, cp_size, interleave, scale, o_partial, lse, workspace,
                    workspace_bytes, stream, ev_begin, ev_end, &f);
}

int dcp_attn_shard_mq(const dcp_attn_desc* desc, int q_len, const void* q, const void* kv_pages,
                      const void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                      int batch, int64_t max_seq_len, int rank, int cp_size, int interleave,
                      float scale, float* o_partial, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return shard_impl(desc, q_len, DCP_F32, q, kv_pages, v_pages, block_table, seq_lens, batch,
                    max_seq_len, rank, cp_size, interleave, scale, o_partial, lse, workspace,
                    workspace_bytes, stream, nullptr, nullptr);
}

int dcp_attn_shard_mq_timed(const dcp_attn_desc* desc, int q_len, const void* q,
                            const void* kv_pages, const void* v_pages,
                            const int32_t* block_table, const int32_t* seq_lens, int batch,
                            int64_t max_seq_len, int rank, int cp_size, int interleave,
                            float scale, float* o_partial, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream, hipEvent_t ev_begin,
                            hipEvent_t ev_end) {
  return shard_impl(desc, q_len, DCP_F32, q, kv_pages, v_pages, block_table, seq_lens, batch,
                    max_seq_len, rank, cp_size, interleave, scale, o_partial, lse, workspace,
                    workspace_bytes, stream, ev_begin, ev_end);
}

int dcp_attn_shard_timed(const dcp_attn_desc* desc, const void* q, const void* kv_pages,
                         const void* v_pages, const int32_t* block_table,
                         const int32_t* seq_lens, int batch, int64_t max_seq_len, int rank,
                         int cp_size, int interleave, float scale, float* o_partial,
                         float* lse, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  return shard_impl(desc, 1, DCP_F32, q, kv_pages, v_pages, block_table, seq_lens, batch,
                    max_seq_len, rank, cp_size, interleave, scale, o_partial, lse, workspace,
                    workspace_bytes, stream, ev_begin, ev_end);
}

int dcp_merge_ex(const void* o_partials, int in_dtype, const float* lse_partials, int cp_size,
                 int batch, int num_heads, int head_dim_v, void* o_out, int out_dtype,
                 float* lse_out, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (cp_size < 1 || batch < 0 || num_heads < 1 || head_dim_v < 1) return DCP_EINVAL;
  if (out_dtype != DCP_F32 && out_dtype != DCP_BF16) return DCP_EINVAL;
  if (in_dtype != DCP_F32 && in_dtype != DCP_BF16) return DCP_EINVAL;
  if ((int64_t)batch * num_heads * head_dim_v * cp_size > ((int64_t)1 << 40)) return DCP_EUNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!o_partials || !lse_partials || !o_out) return DCP_EINVAL;
  if (!aligned(o_partials, 16) || !aligned(o_out, 16)) return DCP_EINVAL;
  const hipError_t e = dcp::launch_merge(o_partials, in_dtype == DCP_BF16, lse_partials, cp_size,
                                         batch, num_heads, head_dim_v, o_out,
                                         out_dtype == DCP_BF16, lse_out, stream, ev_begin, ev_end);
  return e == hipSuccess ? DCP_OK : DCP_ELAUNCH;
}

int dcp_merge_timed(const float* o_partials, const float* lse_partials, int cp_size, int batch,
                    int num_heads, int head_dim_v, void* o_out, int out_dtype, float* lse_out,
                    hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  return dcp_merge_ex(o_partials, DCP_F32, lse_partials, cp_size, batch, num_heads, head_dim_v,
                      o_out, out_dtype, lse_out, stream, ev_begin, ev_end);
}

int dcp_merge(const float* o_partials, const float* lse_partials, int cp_size, int batch,
              int num_heads, int head_dim_v, void* o_out, int out_dtype, float* lse_out,
              hipStream_t stream) {
  return dcp_merge_timed(o_partials, lse_partials, cp_size, batch, num_heads, head_dim_v, o_out,
                         out_dtype, lse_out, stream, nullptr, nullptr);
}

int dcp_shard_slots(const int32_t* block_table, const int32_t* seq_lens, int batch,
                    int max_blocks_per_seq, int block_size, int64_t num_blocks, int rank,
                    int cp_size, int interleave, const int64_t* out_offsets,
                    int64_t* slots_out, void* workspace, hipStream_t stream) {
  if (batch < 0 || max_blocks_per_seq < 1 || block_size < 1 || num_blocks < 1) return DCP_EINVAL;
  if (cp_size < 1 || interleave < 1 || rank < 0 || rank >= cp_size) return DCP_EINVAL;
  if ((int64_t)cp_size * interleave > kMaxI32 ||
      (int64_t)max_blocks_per_seq * block_size > kMaxI32)
    return DCP_EUNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!block_table || !seq_lens || !out_offsets || !slots_out) return DCP_EINVAL;
  if (!workspace || !aligned(workspace, 256)) return DCP_EWORKSPACE;
  const hipError_t e = dcp::launch_shard_slots(
      block_table, seq_lens, batch, max_blocks_per_seq, block_size, num_blocks, rank, cp_size,
      interleave, out_offsets, slots_out, static_cast<int32_t*>(workspace), stream);
  return e == hipSuccess ? DCP_OK : DCP_ELAUNCH;
}

int64_t dcp_local_len(int64_t seq_len, int rank, int cp_size, int interleave) {
  if (seq_len < 0 || cp_size < 1 || interleave < 1 || rank < 0 || rank >= cp_size) return -1;
  return dcp_walk_local_count(seq_len, rank, cp_size, interleave);
}

int dcp_check_parallel(int tp, int dcp, int num_kv_heads, int is_mla) {
  if (tp < 1 || dcp < 1) return 0;
  int copies;
  if (is_mla) {
    copies = tp;
  } else {
    if (num_kv_heads < 1) return 0;
    copies = tp / num_kv_heads;
  }
  return (copies >= dcp && copies % dcp == 0) ? 1 : 0;
}

const char* dcp_status_string(int status) {
  switch (status) {
    case DCP_OK: return "DCP_OK";
    case DCP_EINVAL: return "DCP_EINVAL: invalid argument";
    case DCP_EUNSUPPORTED: return "DCP_EUNSUPPORTED: shape or dtype not implemented";
    case DCP_ELAUNCH: return "DCP_ELAUNCH: HIP runtime error";
    case DCP_EWORKSPACE: return "DCP_EWORKSPACE: workspace null, misaligned or too small";
    case DCP_ESCRATCH:
      return "DCP_ESCRATCH: the call needs more scratch than the library's static array holds";
    default: return "unknown dcp_status";
  }
}

int dcp_read_device_errors(const void* workspace, hipStream_t stream, int32_t* errors_out) {
  if (!workspace || !errors_out) return DCP_EINVAL;
  if (hipMemcpyAsync(errors_out, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, stream) !=
      hipSuccess)
    return DCP_ELAUNCH;
  return hipStreamSynchronize(stream) == hipSuccess ? DCP_OK : DCP_ELAUNCH;
}

}  // extern "C"

// dcp_api.cpp — the C ABI of include/dcp_attn.h: the launch sequence of a shard call
// (plan -> shard kernel -> split combine) after the checks and the workspace sizing of
// host_rules.h.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "api_internal.h"
#include "dcp_attn.h"
#include "launch.h"

namespace {

using dcp::KvFp8;
using dcp::Plan;

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

int shard_impl(const dcp_attn_desc* d, int q_len, int o_dtype, const void* q, const void* kv,
               const void* v, const int32_t* bt, const int32_t* lens, int batch,
               int64_t max_seq_len, int rank, int cp, int il, float scale, void* o, float* lse,
               void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
               const KvFp8* fp8 = nullptr) {
  Plan p;
  const int st = dcp::check_shard_args(d, q_len, o_dtype, q, kv, v, bt, lens, batch, max_seq_len,
                                       rank, cp, il, scale, o, lse, ws, ws_bytes, fp8,
                                       device_cus, &p);
  if (st != DCP_OK || batch == 0) return st;
  const int o_bf16 = o_dtype == DCP_BF16;
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
    dcp::MlaArgs a{q, kv, bt, d->num_q_heads, d->block_size, d->max_blocks_per_seq, d->num_blocks,
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
  if (dcp::check_desc(desc, q_len, batch, max_seq_len, cp_size, interleave) != DCP_OK) return 0;
  Plan p;
  if (!dcp::make_plan(desc, q_len, batch, device_cus(), &p)) return 0;
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
  const int st = dcp::check_merge_args(o_partials, in_dtype, lse_partials, cp_size, batch,
                                       num_heads, head_dim_v, o_out, out_dtype);
  if (st != DCP_OK || batch == 0) return st;
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
  const int st = dcp::check_slots_args(block_table, seq_lens, batch, max_blocks_per_seq,
                                       block_size, num_blocks, rank, cp_size, interleave,
                                       out_offsets, slots_out, workspace);
  if (st != DCP_OK || batch == 0) return st;
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

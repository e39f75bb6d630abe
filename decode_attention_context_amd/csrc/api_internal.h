// api_internal.h — the shard call behind the dcp_attn_shard* entry points (internal).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "dcp_attn.h"

namespace dcp {

// Argument checks, work plan, attention kernel and split combine of one shard call, with
// the workspace given by the caller; the arguments and results are those of
// dcp_attn_shard_ex.
int shard_call(const dcp_attn_desc* desc, int q_len, int o_dtype, const void* q,
               const void* kv_pages, const void* v_pages, const int32_t* block_table,
               const int32_t* seq_lens, int batch, int64_t max_seq_len, int rank, int cp_size,
               int interleave, float scale, void* o_partial, float* lse, void* workspace,
               size_t workspace_bytes, hipStream_t stream, hipEvent_t ev_begin,
               hipEvent_t ev_end);

}  // namespace dcp

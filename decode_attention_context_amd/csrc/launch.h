// launch.h — host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dcp {

// Work planning of one shard call: per-request owned-token counts, the tokens-per-item
// split size and the flat list of (request, local token range) items.
hipError_t launch_plan(const int32_t* seq_lens, int batch, int rank, int cp, int interleave,
                       int64_t len_cap, int64_t target_items, int tile, int min_chunk,
                       const WsPtrs& ws, hipStream_t stream);

// LSE merge of `n` partials per row (rows = batch * heads); ev0 / ev1 (nullable) take the
// merge kernel's own start and end time stamps.
// Partials are float32, or bf16 when in_bf16.
hipError_t launch_merge(const void* o_partials, int in_bf16, const float* lse_partials, int n,
                        int batch, int heads, int dv, void* o_out, int out_bf16, float* lse_out,
                        hipStream_t stream, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// Combine of the split partials of each request into the shard output (float32, or bf16
// rounded to nearest even when out_bf16).
hipError_t launch_split_combine(const WsPtrs& ws, int batch, int hq, int dv, void* o_out,
                                int out_bf16, float* lse_out, hipStream_t stream);

// Query rows of a request: q_len positions x the query heads.  Row i of a multi-token
// request sits at position seq_len - q_len + i and sees the positions up to its own, so it
// reads the shard's local tokens j < (tokens of a (seq_len - q_len + 1 + i)-token sequence
// the rank stores).  With q_len = 1 every row sees all of the shard's tokens.
struct RowArgs {
  const int32_t* seq_lens;
  int64_t len_cap;   // block-table capacity in tokens (seq_len is clamped to it)
  int q_len;
};

struct GqaArgs {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  int hq, hkv, head_dim, block_size, max_blocks;
  int64_t num_blocks;
  int rank, cp, interleave;
  float scale;
  int dtype;  // 0 f32, 1 bf16
  RowArgs rows;
  int o_bf16;  // partial output O in bf16 (round to nearest even) instead of float32
};
// ev0 / ev1 (nullable): events stamped with the attention kernel's own start and end.
hipError_t launch_gqa_shard(const GqaArgs& a, int64_t max_items, const WsPtrs& ws,
                            void* o_out, float* lse_out, hipStream_t stream,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// fp8 KV cache (OCP FP8 E4M3 codes, one float32 scale per tensor; bf16 queries): the same
// shard with K / V values decode(code) * scale.  Supported for head_dim 128 and up to 64
// query rows (q_len * group) per KV head.
hipError_t launch_gqa_fp8_shard(const GqaArgs& a, float k_scale, float v_scale,
                                int64_t max_items, const WsPtrs& ws, void* o_out,
                                float* lse_out, hipStream_t stream, hipEvent_t ev0 = nullptr,
                                hipEvent_t ev1 = nullptr);

struct MlaArgs {
  const void* q;
  const void* latent;
  const int32_t* block_table;
  int heads;   // query heads: 16, 32, 64 or 128
  int block_size, max_blocks;
  int64_t num_blocks;
  int rank, cp, interleave;
  float scale;
  RowArgs rows;
  int o_bf16;  // partial output O in bf16 (round to nearest even) instead of float32
};
hipError_t launch_mla_shard(const MlaArgs& a, int64_t max_items, const WsPtrs& ws,
                            void* o_out, float* lse_out, hipStream_t stream,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

hipError_t launch_shard_slots(const int32_t* block_table, const int32_t* seq_lens, int batch,
                              int max_blocks, int block_size, int64_t num_blocks, int rank,
                              int cp, int interleave, const int64_t* out_offsets,
                              int64_t* slots_out, int32_t* err_word, hipStream_t stream);

}  // namespace dcp

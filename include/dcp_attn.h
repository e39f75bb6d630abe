/*
 * dcp_attn.h — C ABI of the MI355X (gfx950) decode-context-parallel attention library.
 *
 * Decode context parallelism (DCP) shards a sequence's KV cache along the sequence
 * dimension: every DCP rank stores a subset of the token positions of every request, the
 * gathered query attends to each rank's local slice, and the per-rank partial outputs are
 * combined with their log-sum-exp values by the online-softmax merge.
 *   Sources: "vLLM Decode Context Parallelism for long-context workloads" (agentlenshq.com
 *   blog), sections "How DCP works" and "DCP execution flow"; "Context Parallel Guide"
 *   (vLLM Ascend docs), sections "Usage -> Decode Context Parallel" and
 *   "Decode Context Parallel -> Constraints".
 *
 * Ownership rule (the --cp-kv-cache-interleave-size flag of the guide): token t of a
 * sequence lives on rank (t / interleave) mod cp_size.  The blog's contiguous split of a
 * 200K-token request over four GPUs is the case interleave = seq_len / cp_size.
 *
 * On one GPU the other ranks' shards are virtual: `rank`, `cp_size` and `interleave`
 * select which token positions of one paged cache a call reads.  On a real DCP group a
 * rank calls dcp_attn_shard with rank = 0, cp_size = 1 on its own local cache.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers unless marked host; all tensors are dense
 *     and row-major in the layouts documented below.  The caller owns every buffer; the
 *     library allocates nothing and keeps no state between calls, except for the static
 *     scratch array of dcp_attn_shard_noalloc (described there).
 *   - Work is enqueued on `stream` and never synchronizes with the host, except in
 *     dcp_read_device_errors, which says so.  The calls can be recorded in a HIP graph.
 *   - Argument errors are detected on the host before anything is launched and returned
 *     as a negative dcp_status.  No C++ exception crosses this interface.
 *   - Contract violations that only the device can see (a seq_len larger than the block
 *     table covers, a block id outside [0, num_blocks)) never fault: the offending tokens
 *     are skipped and a bit is set in the workspace's error word.
 */
#ifndef DCP_ATTN_H
#define DCP_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point that returns int. */
typedef enum {
  DCP_OK = 0,
  DCP_EINVAL = -1,        /* a bad argument (null pointer, size out of range, rank >= cp_size, ...) */
  DCP_EUNSUPPORTED = -2,  /* a valid but unimplemented shape or dtype */
  DCP_ELAUNCH = -3,       /* the HIP runtime rejected a launch or a query */
  DCP_EWORKSPACE = -4,    /* the workspace is null, too small or misaligned */
  DCP_ESCRATCH = -5       /* dcp_attn_shard_noalloc: the call needs more than the library's
                             static scratch (DCP_NOALLOC_SCRATCH_BYTES) */
} dcp_status;

/* Element types. */
typedef enum { DCP_F32 = 0, DCP_BF16 = 1 } dcp_dtype;

/* Attention variants.  GQA: Hq query heads share Hkv KV heads in contiguous groups of
 * G = Hq / Hkv (query head h reads KV head h / G), separate K and V caches.
 * MLA: one latent row per token is shared by all query heads (blog, "The memory wall in
 * long-context inference", MLA item): the key is the whole row and the value is its first
 * head_dim_v columns. */
typedef enum { DCP_GQA = 0, DCP_MLA = 1 } dcp_kind;

/* Bits of the device error word (see dcp_read_device_errors). */
#define DCP_DEVERR_SEQ_LEN 1   /* seq_len < 0 or > max_blocks_per_seq * block_size; clamped */
#define DCP_DEVERR_BLOCK_ID 2  /* a block id outside [0, num_blocks); its tokens are skipped */

/* Shape of the paged cache and the heads.
 *   GQA: k_pages, v_pages  [num_blocks][num_kv_heads][block_size][head_dim]  (dtype),
 *        q [batch][num_q_heads][head_dim] (dtype); head_dim_qk == head_dim_v.
 *        Supported: BF16 with head_dim 128, or F32 with head_dim 64 (256-byte rows), and
 *        any group G = num_q_heads / num_kv_heads with q_len * G <= 64 query rows per KV
 *        head (q_len = 1 except in dcp_attn_shard_mq / _ex / _fp8kv / _noalloc).  Every
 *        other GQA shape returns DCP_EUNSUPPORTED without launching.
 *   MLA: latent_pages [num_blocks][block_size][head_dim_qk] (BF16),
 *        q [batch][num_q_heads][head_dim_qk] (BF16).
 *        Supported: num_q_heads 16, 32, 64 or 128 (the heads gathered over a DCP group:
 *        e.g. 16 per rank under tensor parallelism 8, times the DCP size), head_dim_qk 576,
 *        head_dim_v 512, num_kv_heads 1.  Every other MLA shape returns DCP_EUNSUPPORTED.
 *   Every kind: num_blocks * block_size * num_kv_heads < 2^31. */
typedef struct {
  int32_t kind;               /* dcp_kind */
  int32_t dtype;              /* dcp_dtype of q and the cache */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t block_size;         /* tokens per cache page (the guide's --block-size) */
  int32_t max_blocks_per_seq; /* columns of block_table */
  int64_t num_blocks;         /* pages in the cache */
} dcp_attn_desc;

/* Bytes of workspace dcp_attn_shard needs for this shape on the current device.
 * Host-only and pure apart from reading the device's compute-unit count.  Returns 0 when
 * the arguments are invalid.  The workspace must be 256-byte aligned. */
size_t dcp_workspace_size(const dcp_attn_desc* desc, int batch, int64_t max_seq_len,
                          int cp_size, int interleave);

/* Partial decode attention of the gathered queries against one rank's shard.
 * (blog, "DCP execution flow", step "Compute": each GPU attends the gathered query against
 * its local KV slice; step 3 needs the partial output together with its LSE.)
 *
 *   q            gathered queries (layouts above).
 *   kv_pages     GQA: K pages; MLA: latent pages.
 *   v_pages      GQA: V pages; MLA: must be NULL.
 *   block_table  int32 [batch][max_blocks_per_seq]: physical page of each logical page of
 *                the GLOBAL sequence (token t is in page block_table[b][t / block_size],
 *                slot t % block_size).  Entries past a sequence's last page are not read.
 *   seq_lens     int32 [batch]: global context length of each request.
 *   max_seq_len  host: an upper bound of seq_lens (used only to validate and size work).
 *   rank, cp_size, interleave   host: the shard, 0 <= rank < cp_size, interleave >= 1.
 *   scale        host: scores are scale * q.k.
 *   o_partial    out float32 [batch][num_q_heads][head_dim_v]: softmax-weighted values
 *                over the shard's tokens.
 *   lse          out float32 [batch][num_q_heads]: natural-log log-sum-exp of the shard's
 *                scaled scores.  A request whose shard is empty gets lse = -inf, O = 0.
 *   workspace    device scratch of at least dcp_workspace_size() bytes.  Its first
 *                int32 is the device error word (DCP_DEVERR_*) of the latest call.  It
 *                holds the call's plan and split partials until the call's kernels end:
 *                calls in flight at the same time need workspaces of their own (calls in
 *                order on one stream may share one).  A request's shard may be cut into
 *                several work items whose partials are combined by their LSE; the GQA
 *                kernels keep those split partials in float32, the MLA kernel in bf16
 *                (round to nearest even; their LSE stays float32), which halves the bytes
 *                of the 512-wide latent rows.
 * Returns DCP_OK or a negative dcp_status (nothing launched). */
int dcp_attn_shard(const dcp_attn_desc* desc, const void* q, const void* kv_pages,
                   const void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                   int batch, int64_t max_seq_len, int rank, int cp_size, int interleave,
                   float scale, float* o_partial, float* lse, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* dcp_attn_shard with instrumentation: when non-null, `ev_begin` and `ev_end` (created by
 * the caller with timing enabled) take the start and end time stamps of the shard's
 * attention kernel itself (launched through hipExtLaunchKernel; the planning and
 * split-combine launches fall outside them), so hipEventElapsedTime gives that kernel's
 * duration alone.  Same arguments, results and errors as dcp_attn_shard. */
int dcp_attn_shard_timed(const dcp_attn_desc* desc, const void* q, const void* kv_pages,
                         const void* v_pages, const int32_t* block_table,
                         const int32_t* seq_lens, int batch, int64_t max_seq_len, int rank,
                         int cp_size, int interleave, float scale, float* o_partial,
                         float* lse, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end);

/* Multi-token decode: dcp_attn_shard for q_len query positions per request (speculative
 * decoding or multi-token prediction verifying draft tokens under DCP; the "Context Parallel
 * Guide" lists speculative decoding among the features that work with DCP, and the blog's
 * "Roadmap" section names it).  The request's last q_len cache tokens are its draft tokens:
 * query position i (0 <= i < q_len) sits at global position seq_len - q_len + i and attends
 * every position up to and including its own, a causal mask aligned to the end of the
 * sequence.  On a shard that is the rank's tokens among the first seq_len - q_len + 1 + i
 * positions; a position with none of them (or a negative position, seq_len < q_len) gets
 * lse = -inf and O = 0.  Each K / V (latent) row is read from HBM once for all positions.
 *   q          [batch][q_len][num_q_heads][head_dim_qk] (dtype)
 *   o_partial  out float32 [batch][q_len][num_q_heads][head_dim_v]
 *   lse        out float32 [batch][q_len][num_q_heads]
 *   q_len      host: 1 .. 4; 1 is exactly dcp_attn_shard.  More returns DCP_EUNSUPPORTED.
 *   workspace  at least dcp_workspace_size_mq() bytes.
 * Every other argument, the merge of the partials (dcp_merge with num_heads =
 * q_len * num_q_heads), the errors and the ownership are as for dcp_attn_shard. */
size_t dcp_workspace_size_mq(const dcp_attn_desc* desc, int q_len, int batch,
                             int64_t max_seq_len, int cp_size, int interleave);
int dcp_attn_shard_mq(const dcp_attn_desc* desc, int q_len, const void* q, const void* kv_pages,
                      const void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                      int batch, int64_t max_seq_len, int rank, int cp_size, int interleave,
                      float scale, float* o_partial, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);
/* dcp_attn_shard_mq with the attention kernel's own start / end stamped into the caller's
 * events, as dcp_attn_shard_timed. */
int dcp_attn_shard_mq_timed(const dcp_attn_desc* desc, int q_len, const void* q,
                            const void* kv_pages, const void* v_pages,
                            const int32_t* block_table, const int32_t* seq_lens, int batch,
                            int64_t max_seq_len, int rank, int cp_size, int interleave,
                            float scale, float* o_partial, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream, hipEvent_t ev_begin,
                            hipEvent_t ev_end);

/* The general shard call: q_len query positions per request as in dcp_attn_shard_mq, the
 * partial output O in o_dtype, and optional timing events as in dcp_attn_shard_timed.
 *   o_dtype    DCP_F32: o_partial is float32 (as in dcp_attn_shard);
 *              DCP_BF16: o_partial is bf16 [batch][q_len][num_q_heads][head_dim_v], each
 *              value the float32 result rounded to nearest even.  The partials every rank
 *              exchanges and the merge reads then take half the bytes (the blog's "DCP
 *              execution flow" exchanges partial outputs with their LSE; the LSE stays
 *              float32).  Split partials inside the workspace are as in dcp_attn_shard.
 *   ev_begin, ev_end   nullable; as in dcp_attn_shard_timed.
 * Every other argument, the workspace (dcp_workspace_size_mq) and the errors are as for
 * dcp_attn_shard_mq; dcp_attn_shard, _timed, _mq and _mq_timed are this call with
 * o_dtype = DCP_F32. */
int dcp_attn_shard_ex(const dcp_attn_desc* desc, int q_len, int o_dtype, const void* q,
                      const void* kv_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* seq_lens, int batch, int64_t max_seq_len, int rank,
                      int cp_size, int interleave, float scale, void* o_partial, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t ev_begin, hipEvent_t ev_end);

/* The shard call of a GQA cache stored in fp8 (the lower-byte KV variant: the pages leave
 * the KV dtype open).  k_pages / v_pages hold OCP FP8 E4M3 codes (uint8; sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent 0 subnormal; S.1111.111 NaN, no infinities),
 * [num_blocks][num_kv_heads][block_size][head_dim], 16-byte aligned; the cached key / value
 * is decode(code) * k_scale / v_scale (finite floats).  desc->kind = DCP_GQA and
 * desc->dtype = DCP_BF16 describe the bf16 queries; head_dim 128 and up to 64 query rows
 * (q_len * num_q_heads / num_kv_heads) per KV head are supported, other shapes return
 * DCP_EUNSUPPORTED without launching.  Scores are scale * q . k; everything else (q_len,
 * o_dtype, outputs, workspace from dcp_workspace_size_mq with the same desc, events,
 * errors) is as in dcp_attn_shard_ex.  A code of NaN in a page the call reads gives NaN
 * outputs for the rows that see it. */
int dcp_attn_shard_fp8kv(const dcp_attn_desc* desc, int q_len, int o_dtype, const void* q,
                         const void* k_pages, const void* v_pages, float k_scale,
                         float v_scale, const int32_t* block_table, const int32_t* seq_lens,
                         int batch, int64_t max_seq_len, int rank, int cp_size, int interleave,
                         float scale, void* o_partial, float* lse, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, hipEvent_t ev_begin,
                         hipEvent_t ev_end);

/* The shard call for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): dcp_attn_shard_ex without
 * a workspace argument and without timing events.  The plan and the split partials live in
 * a static device array of DCP_NOALLOC_SCRATCH_BYTES bytes that the library holds on every
 * device it runs on until the process ends; the call itself allocates nothing.
 *   Runs on the current HIP device; `stream` must belong to it.
 *   A call that needs more than DCP_NOALLOC_SCRATCH_BYTES of workspace
 *   (dcp_workspace_size_mq with the same arguments) returns DCP_ESCRATCH without launching.
 *   Every call on one device shares that device's array: calls whose kernels overlap on one
 *   device (on different streams, or from several host threads without ordering) race and
 *   give wrong results.  Calls in order on one stream are safe; each call's planner
 *   rewrites the plan and the error word before its kernels read them.
 *   The device error word (DCP_DEVERR_*) is kept in the array and is not readable by the
 *   caller; device-side contract violations are handled as in dcp_attn_shard (tokens
 *   skipped, no fault).
 * Every other argument, the results and the errors are as in dcp_attn_shard_ex. */
#define DCP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dcp_attn_shard_noalloc(const dcp_attn_desc* desc, int q_len, int o_dtype, const void* q,
                           const void* kv_pages, const void* v_pages,
                           const int32_t* block_table, const int32_t* seq_lens, int batch,
                           int64_t max_seq_len, int rank, int cp_size, int interleave,
                           float scale, void* o_partial, float* lse, hipStream_t stream);

/* LSE-weighted merge of cp_size partials into attention over the union of their tokens
 * (blog, "DCP execution flow", step 3: the LSE values reweight the partial results with
 * the online-softmax trick).  With m = max of the finite lse_r:
 *   w_r = exp(lse_r - m), or exactly 0 when lse_r is not finite (O_r is then not read);
 *   lse = m + ln(sum_r w_r);  O = sum_r w_r O_r / sum_r w_r.
 * A row whose partials are all empty gets O = 0 and lse = -inf.
 *   o_partials    float32 [cp_size][batch][num_heads][head_dim_v]
 *   lse_partials  float32 [cp_size][batch][num_heads]
 *   o_out         [batch][num_heads][head_dim_v] of out_dtype (F32, or BF16 rounded to
 *                 nearest even); may not alias the inputs.
 *   lse_out       float32 [batch][num_heads], or NULL.
 * Returns DCP_OK or a negative dcp_status (nothing launched). */
int dcp_merge(const float* o_partials, const float* lse_partials, int cp_size, int batch,
              int num_heads, int head_dim_v, void* o_out, int out_dtype, float* lse_out,
              hipStream_t stream);

/* dcp_merge with instrumentation: when non-null, `ev_begin` and `ev_end` (created by the
 * caller with timing enabled) take the start and end time stamps of the merge kernel itself
 * (launched through hipExtLaunchKernel), so hipEventElapsedTime gives its duration alone.
 * Same arguments, results and errors as dcp_merge. */
int dcp_merge_timed(const float* o_partials, const float* lse_partials, int cp_size, int batch,
                    int num_heads, int head_dim_v, void* o_out, int out_dtype, float* lse_out,
                    hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end);

/* The general merge: dcp_merge with the partials o_partials in in_dtype (DCP_F32: float32;
 * DCP_BF16: bf16, e.g. as written by dcp_attn_shard_ex, widened exactly to float32 before
 * the float32 arithmetic) and optional timing events as in dcp_merge_timed (nullable).
 * dcp_merge and dcp_merge_timed are this call with in_dtype = DCP_F32. */
int dcp_merge_ex(const void* o_partials, int in_dtype, const float* lse_partials, int cp_size,
                 int batch, int num_heads, int head_dim_v, void* o_out, int out_dtype,
                 float* lse_out, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end);

/* Physical slots (page * block_size + t % block_size, int64) of the tokens a rank stores,
 * in ascending global position t: the library's block-table walk made visible.
 * out_offsets  int64 [batch]: where request b's slots start in slots_out; request b
 *              writes dcp_local_len(seq_lens[b], ...) entries.  A token whose block id is
 *              outside [0, num_blocks) gets slot -1.
 * num_blocks   host: pages in the cache (to validate block ids).
 * workspace    device, >= 256 bytes, 256-aligned: its first int32 receives the error word
 *              as in dcp_attn_shard.
 * Returns DCP_OK or a negative dcp_status. */
int dcp_shard_slots(const int32_t* block_table, const int32_t* seq_lens, int batch,
                    int max_blocks_per_seq, int block_size, int64_t num_blocks, int rank,
                    int cp_size, int interleave, const int64_t* out_offsets,
                    int64_t* slots_out, void* workspace, hipStream_t stream);

/* Host, pure: number of tokens of a seq_len-token sequence that `rank` stores.
 * Returns -1 for invalid arguments. */
int64_t dcp_local_len(int64_t seq_len, int rank, int cp_size, int interleave);

/* Host, pure: 1 when a DCP size is allowed by the guide's constraints, else 0.
 * MLA (is_mla != 0): tp >= dcp and tp % dcp == 0.  GQA: with copies = tp / num_kv_heads
 * (integer division), copies >= dcp and copies % dcp == 0.
 * ("Context Parallel Guide", "Decode Context Parallel -> Constraints"; blog, sections
 * "MLA backend" and "GQA backend".) */
int dcp_check_parallel(int tp, int dcp, int num_kv_heads, int is_mla);

/* Host: a static string naming a dcp_status. */
const char* dcp_status_string(int status);

/* Reads the device error word of the latest shard or slots call that used `workspace`
 * into *errors_out (DCP_DEVERR_* bits; 0 = clean).  Synchronizes `stream`. */
int dcp_read_device_errors(const void* workspace, hipStream_t stream, int32_t* errors_out);

#ifdef __cplusplus
}
#endif

#endif /* DCP_ATTN_H */

// noalloc.hip — dcp_attn_shard_noalloc: the shard call with its workspace in a static
// device array, for callers that cannot allocate device memory.
//
// `scratch` below is a device variable of fixed size.  In host code its name only stands in
// for it (passing it to a kernel would hand the kernel a host address), so its device
// address is looked up once per device with hipGetSymbolAddress, on the first call made
// with that device current, and only that address is ever used.  The array then holds each
// call's plan, error word and split partials exactly as a caller's workspace would.
#include <mutex>

#include <hip/hip_runtime.h>

#include "api_internal.h"
#include "dcp_attn.h"

namespace {

constexpr size_t kScratchBytes = DCP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device (null: not looked up)

// The device address of this device's `scratch` (looked up on first use), or null.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int dcp_attn_shard_noalloc(const dcp_attn_desc* desc, int q_len, int o_dtype,
                                      const void* q, const void* kv_pages, const void* v_pages,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int batch, int64_t max_seq_len, int rank, int cp_size,
                                      int interleave, float scale, void* o_partial, float* lse,
                                      hipStream_t stream) {
  const size_t need = dcp_workspace_size_mq(desc, q_len, batch, max_seq_len, cp_size, interleave);
  if (need > kScratchBytes) return DCP_ESCRATCH;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return DCP_ELAUNCH;
  // need == 0 (invalid arguments): the call below returns the matching status
  return dcp::shard_call(desc, q_len, o_dtype, q, kv_pages, v_pages, block_table, seq_lens,
                         batch, max_seq_len, rank, cp_size, interleave, scale, o_partial, lse,
                         ws, kScratchBytes, stream, nullptr, nullptr);
}

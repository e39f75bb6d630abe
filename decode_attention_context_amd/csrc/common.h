// common.h — device helpers and the workspace layout shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "walker.h"

namespace dcp {

// ---------------------------------------------------------------------------------------
// Workspace layout (every section 256-byte aligned).  Written by the planner, read by the
// shard kernels and the split combine of the same call.
//   header  int32[64]: [0] device error word, [1] number of work items, [2] tokens per item
//   off     int32[batch + 1]: first work item of each request (prefix sum)
//   items   int4[max_items]: (request, local token begin, local token end, 0)
//   plse    float[max_items * Hq]:      per-item log-sum-exp (natural log)
//   po      float[max_items * Hq * Dv]: per-item normalized partial output
// ---------------------------------------------------------------------------------------
struct WsLayout {
  size_t off_off, items_off, plse_off, po_off, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline WsLayout ws_layout(int batch, int64_t max_items, int hq, int dv) {
  WsLayout w;
  w.off_off = 256;
  w.items_off = w.off_off + align256(sizeof(int32_t) * (size_t)(batch + 1));
  w.plse_off = w.items_off + align256(sizeof(int32_t) * 4 * (size_t)max_items);
  w.po_off = w.plse_off + align256(sizeof(float) * (size_t)max_items * hq);
  w.total = w.po_off + align256(sizeof(float) * (size_t)max_items * hq * dv);
  return w;
}

struct WsPtrs {
  int32_t* header;
  int32_t* off;
  int4* items;
  float* plse;
  float* po;
};

inline WsPtrs ws_ptrs(void* base, const WsLayout& w) {
  char* p = static_cast<char*>(base);
  return WsPtrs{reinterpret_cast<int32_t*>(p), reinterpret_cast<int32_t*>(p + w.off_off),
                reinterpret_cast<int4*>(p + w.items_off), reinterpret_cast<float*>(p + w.plse_off),
                reinterpret_cast<float*>(p + w.po_off)};
}

constexpr int kErrSeqLen = 1;
constexpr int kErrBlockId = 2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Butterfly reductions across the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// DPP lane permutations inside each 16-lane row (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7 - i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15 - i within each 16 lanes

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), kCtrl,
                                                    0xF, 0xF, false));
}

// Max / sum over all 64 lanes without LDS: a DPP butterfly inside each 16-lane row, then
// the four row results are read into scalars.  The result is wave-uniform.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  const int vi = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(vi, 0)),
                     __int_as_float(__builtin_amdgcn_readlane(vi, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(vi, 32)),
                     __int_as_float(__builtin_amdgcn_readlane(vi, 48))));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  const int vi = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(vi, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(vi, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(vi, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(vi, 48)));
}

// float -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace dcp

// common.h — device helpers and the workspace layout shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_rules.h"
#include "walker.h"

namespace dcp {

struct WsPtrs {
  int32_t* header;
  int32_t* off;
  int4* items;
  float* plse;
  void* po;
  int po_bf16;   // po holds bf16 values (else float32)
};

inline WsPtrs ws_ptrs(void* base, const WsLayout& w) {
  char* p = static_cast<char*>(base);
  return WsPtrs{reinterpret_cast<int32_t*>(p), reinterpret_cast<int32_t*>(p + w.off_off),
                reinterpret_cast<int4*>(p + w.items_off), reinterpret_cast<float*>(p + w.plse_off),
                p + w.po_off, w.po_bf16};
}

constexpr int kErrSeqLen = 1;
constexpr int kErrBlockId = 2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Local end of the shard's tokens that query row `qi` of a q_len-row request sees: the
// rank's tokens of the first seq_len - q_len + 1 + qi positions (seq_len clamped to the
// block table as the planner clamps it).
__device__ __forceinline__ int row_local_end(const int32_t* seq_lens, int b, int64_t len_cap,
                                             int q_len, int qi, int rank, int cp, int il) {
  int64_t L = seq_lens[b];
  L = L < 0 ? 0 : (L > len_cap ? len_cap : L);
  const int64_t Lq = L - q_len + 1 + qi;   // below 2^31 (len_cap is)
  return Lq <= 0 ? 0
                 : (int)dcp_walk_local_count32((uint32_t)Lq, (uint32_t)rank, (uint32_t)cp,
                                               (uint32_t)il);
}

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

// Max of two floats as v_maximum3_f32 computes it: no quieting of the operands first (which
// fmaxf implies and costs an instruction per operand that the compiler cannot prove
// canonical).  It differs from fmaxf only for NaN operands; the kernels compare finite
// values and -inf.
__device__ __forceinline__ float max_f(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Row-local lane permutation (every lane reads a lane of its own 16-lane row, so the
// bound control never applies); an undefined old value lets the compiler fuse the move
// into the consuming VALU op (v_max_f32_dpp, v_add_f32_dpp).
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}

// The same value combined across the four 16-lane rows: lanes i, i+16, i+32, i+48 swap
// through v_permlane16_swap / v_permlane32_swap (no LDS, no scalar round trip).
__device__ __forceinline__ float rows_max(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Max / sum over all 64 lanes without LDS: a DPP butterfly inside each 16-lane row, then
// the row results are combined by lane swaps.  The result is the same in every lane.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  return rows_max(v);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return rows_sum(v);
}

// Max over all 64 lanes, returned wave-uniform.  v_max_f32 takes its first operand through
// DPP: a butterfly inside each 16-lane row, then row_bcast:15 (rows 1 and 3 take the last
// lane of the row below) and row_bcast:31 (rows 2 and 3 take lane 31), which leaves the
// maximum of the whole wave in lane 63.  Every DPP step reads the register that the VALU op
// before it wrote, so two wait states precede it.
__device__ __forceinline__ float wave_max_bcast(float v) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf"
      : "+v"(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Max / sum over lanes 0..7 (DPP steps inside each 8-lane group), returned wave-uniform
// from lane 0.  Each DPP step reads the register the VALU op before it wrote, so two wait
// states precede it.
__device__ __forceinline__ float lanes8_max(float v) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf"
      : "+v"(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
}
__device__ __forceinline__ float lanes8_sum(float v) {
  asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf"
      : "+v"(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int kVm>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((kVm & 0xF) | ((kVm >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 16-byte-per-lane HBM -> LDS copy: LDS bytes [lds + 16 lane, + 16) <- global
// sbase + voff (scalar base, 32-bit lane offset).  M0 carries the LDS address: it is an
// input operand of the statement, so the compiler writes it (and knows it is read); one
// wait state separates that write from the copy that reads it.  kNt selects the
// non-temporal cache policy (nt): a plain stream of HBM -> LDS copies runs at about
// 7.1 TB/s with it against 5.9 TB/s without on MI355X.  The copy is invisible to the
// compiler's wait-count tracking, so it never drains it before LDS reads: the kernels
// pace the copies with explicit vector-memory counter waits.
template <bool kNt>
__device__ __forceinline__ void copy16_sbase(uint32_t lds, uint32_t voff, const char* sbase) {
  if constexpr (kNt)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds)
                 : "memory");
}
// The same from a per-lane 64-bit address.
template <bool kNt>
__device__ __forceinline__ void copy16_vaddr(uint32_t lds, const char* src) {
  if constexpr (kNt)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "{m0}"(lds)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "{m0}"(lds)
                 : "memory");
}

// float -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace dcp

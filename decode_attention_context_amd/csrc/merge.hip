// merge.hip — LSE-weighted merge of partial attention outputs.
//
// The merge of the DCP execution flow ("vLLM Decode Context Parallelism for long-context
// workloads" blog, section "DCP execution flow", step 3): partials (O_r, lse_r) computed
// over disjoint token sets combine, with m = max of the finite lse_r and
// w_r = exp(lse_r - m) (exactly 0 for a non-finite lse_r, whose O_r is never read), into
//     lse = m + ln sum w_r,     O = sum w_r O_r / sum w_r,
// which is the attention over the union of the token sets.  The same row merge combines
// the split-K partials of one shard call, whose items cover disjoint local token ranges.
//
// One wave merges one (request, head) row: the n lse values are loaded one per lane and
// reduced with DPP (no serial chain of loads).  With at most 8 partials (every cp_size in
// practice) each lane issues the loads of all its partial-row chunks together with the lse
// load, so a row costs one memory round trip; weights of empty partials are exactly 0 and
// their rows (which may hold garbage) are excluded by a select, never multiplied.  More
// partials are streamed eight at a time, empty ones not read.  A split combine over few
// rows gives each 64 * VEC columns of a row a wave of its own instead.  The kernel is
// HBM-bound.
#include <type_traits>

#include "launch.h"

namespace dcp {

namespace {

template <int VEC>
struct VecT;
template <>
struct VecT<1> { using T = float; };
template <>
struct VecT<2> { using T = __attribute__((ext_vector_type(2))) float; };
template <>
struct VecT<4> { using T = __attribute__((ext_vector_type(4))) float; };

// Partial loads with the non-temporal cache policy (nt) or plain (the launcher picks by
// size), plain stores.  Measured on MI355X with eight partials of 128 heads x 512 dims,
// caches flushed: at 512 requests (1.21 GB moved) 203 us with nt loads against 226 us with
// plain loads and 213 us with nt loads and stores.
template <typename T, bool kNt = true>
__device__ __forceinline__ T ld(const float* p) {
  if constexpr (kNt) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else return *reinterpret_cast<const T*>(p);
}
// the partials' LSE values: plain loads (a few bytes per row; measured slightly faster)
__device__ __forceinline__ float ld_lse(const float* p) { return *p; }
template <typename T>
__device__ __forceinline__ void st(float* p, T v) {
  *reinterpret_cast<T*>(p) = v;
}

template <bool kNt, typename T>
__device__ __forceinline__ T nt_or_plain(const T* p) {
  if constexpr (kNt) return __builtin_nontemporal_load(p);
  else return *p;
}

// VEC consecutive elements of a partial row as floats: float32 partials are loaded as they
// are, bf16 partials (2 bytes per element) are loaded at half the width and widened exactly.
template <int VEC, bool kBf16In, bool kNt>
__device__ __forceinline__ typename VecT<VEC>::T ldp(const void* base, int64_t elem) {
  using V = typename VecT<VEC>::T;
  if constexpr (!kBf16In) {
    return ld<V, kNt>(static_cast<const float*>(base) + elem);
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + elem;
    V v;
    float* pv = reinterpret_cast<float*>(&v);
    if constexpr (VEC == 4) {
      typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
      const u32x2 u = nt_or_plain<kNt>(reinterpret_cast<const u32x2*>(p));
      pv[0] = __uint_as_float(u.x << 16);
      pv[1] = __uint_as_float(u.x & 0xffff0000u);
      pv[2] = __uint_as_float(u.y << 16);
      pv[3] = __uint_as_float(u.y & 0xffff0000u);
    } else if constexpr (VEC == 2) {
      const uint32_t u = nt_or_plain<kNt>(reinterpret_cast<const uint32_t*>(p));
      pv[0] = __uint_as_float(u << 16);
      pv[1] = __uint_as_float(u & 0xffff0000u);
    } else {
      pv[0] = __uint_as_float((uint32_t)nt_or_plain<kNt>(p) << 16);
    }
    return v;
  }
}

// bf16 partials kept as loaded (VEC / 2 32-bit words, or one 16-bit value) until their use,
// so that the loads in flight take half the registers of the widened values
template <int VEC>
struct RawBf16;
template <>
struct RawBf16<4> { using T = __attribute__((ext_vector_type(2))) uint32_t; };
template <>
struct RawBf16<2> { using T = uint32_t; };
template <>
struct RawBf16<1> { using T = uint16_t; };

template <int VEC, bool kNt>
__device__ __forceinline__ typename RawBf16<VEC>::T ld_raw_bf16(const void* base, int64_t elem) {
  using T = typename RawBf16<VEC>::T;
  return nt_or_plain<kNt>(reinterpret_cast<const T*>(static_cast<const uint16_t*>(base) + elem));
}

template <int VEC>
__device__ __forceinline__ void widen_bf16(const typename RawBf16<VEC>::T& u, float (&f)[VEC]) {
  if constexpr (VEC == 1) {
    f[0] = __uint_as_float((uint32_t)u << 16);
  } else if constexpr (VEC == 2) {
    f[0] = __uint_as_float(u << 16);
    f[1] = __uint_as_float(u & 0xffff0000u);
  } else {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
}

template <int VEC>
__device__ __forceinline__ void vfma(float (&acc)[VEC], float w, const typename VecT<VEC>::T& v) {
  const float* p = reinterpret_cast<const float*>(&v);
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = fmaf(w, p[i], acc[i]);
}

// Merge `n` partial rows o_base[r * o_stride + c] with lse l_base[r * l_stride] over the
// columns c in [c0, c1) (a multiple of 64 * VEC wide, or the whole row); lse_out, when given,
// receives the merged lse.  The lse values are spread over the lanes (64 per pass) and
// reduced with DPP, so the row costs one round trip for them; the partial rows are then
// streamed in batches of kB whose loads all leave before the first is used (bf16 partials
// held raw until use), a batch's tail predicated rather than loaded one partial at a time.
template <int VEC, bool kBf16In, bool kNt, int kB = 8>
__device__ __forceinline__ void merge_row(const void* __restrict__ o_base, int64_t o_stride,
                                          const float* __restrict__ l_base, int64_t l_stride,
                                          int n, int c0, int c1, float* __restrict__ out_f32,
                                          uint16_t* __restrict__ out_bf16,
                                          float* __restrict__ lse_out, int lane) {
  using V = typename VecT<VEC>::T;
  auto lse_at = [&](int r) -> float {
    if (r >= n) return neg_inf();
    const float x = ld_lse(l_base + r * l_stride);
    return __builtin_isfinite(x) ? x : neg_inf();
  };
  float m = neg_inf();
  for (int r0 = 0; r0 < n; r0 += 64) m = fmaxf(m, lse_at(r0 + lane));
  m = wave_max_dpp(m);
  if (m == neg_inf()) {
    // every partial is empty
    for (int d = c0 + lane * VEC; d < c1; d += 64 * VEC) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        if (out_f32) out_f32[d + i] = 0.f;
        else out_bf16[d + i] = 0;
      }
    }
    if (lse_out && lane == 0) *lse_out = neg_inf();
    return;
  }
  const float m2 = m * kLog2e;
  float wpart = 0.f;
  for (int r0 = 0; r0 < n; r0 += 64) {
    const float x = lse_at(r0 + lane);
    wpart += x == neg_inf() ? 0.f : exp2f(fmaf(x, kLog2e, -m2));
  }
  const float inv = 1.f / wave_sum_dpp(wpart);
  // The column loop is wave-uniform: every lane computes its weight wl in every pass, since
  // the weights are read across lanes (readlane); lanes past the row's end (dv not a
  // multiple of 64 VEC) load and store nothing.
  for (int d0 = c0; d0 < c1; d0 += 64 * VEC) {
    const int d = d0 + lane * VEC;
    const bool act = d < c1;
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    for (int r0 = 0; r0 < n; r0 += 64) {
      const float x = lse_at(r0 + lane);
      const float wl = x == neg_inf() ? 0.f : exp2f(fmaf(x, kLog2e, -m2));
      const int nr = n - r0 < 64 ? n - r0 : 64;
      for (int r = 0; r < nr; r += kB) {
        float wv[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u)   // 0 past the row's partials (readlane of lanes >= nr)
          wv[u] = r + u < nr ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), r + u))
                             : 0.f;
        if constexpr (kBf16In) {
          typename RawBf16<VEC>::T v[kB];
#pragma unroll
          for (int u = 0; u < kB; ++u)
            if (wv[u] != 0.f && act)
              v[u] = ld_raw_bf16<VEC, kNt>(o_base, (int64_t)(r0 + r + u) * o_stride + d);
#pragma unroll
          for (int u = 0; u < kB; ++u) {
            if (wv[u] != 0.f && act) {
              float f[VEC];
              widen_bf16<VEC>(v[u], f);
#pragma unroll
              for (int i = 0; i < VEC; ++i) acc[i] = fmaf(wv[u], f[i], acc[i]);
            }
          }
        } else {
          V v[kB];
#pragma unroll
          for (int u = 0; u < kB; ++u)
            if (wv[u] != 0.f && act)
              v[u] = ldp<VEC, false, kNt>(o_base, (int64_t)(r0 + r + u) * o_stride + d);
#pragma unroll
          for (int u = 0; u < kB; ++u)
            if (wv[u] != 0.f && act) vfma<VEC>(acc, wv[u], v[u]);
        }
      }
    }
    if (!act) continue;
    if (out_f32) {
      V o;
      float* po = reinterpret_cast<float*>(&o);
#pragma unroll
      for (int i = 0; i < VEC; ++i) po[i] = acc[i] * inv;
      st<V>(out_f32 + d, o);
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) out_bf16[d + i] = (uint16_t)f32_to_bf16_rne(acc[i] * inv);
    }
  }
  if (lse_out && lane == 0) *lse_out = (m2 - __log2f(inv)) * kLn2;
}

// One wave merges the columns [c0, c0 + 64 * VEC) of a row (a split combine with few rows).
// The first kB partials' loads leave together with the lse loads, before their weights are
// known, so a row of at most kB partials costs one round trip; later partials follow in
// batches of kB.  Every item of a request has a partial row in the workspace, so the early
// loads stay in bounds; an empty partial's row (any bits) is never used.
template <int VEC, bool kBf16In, int kB>
__device__ __forceinline__ void merge_cols(const void* __restrict__ o_base, int64_t o_stride,
                                           const float* __restrict__ l_base, int64_t l_stride,
                                           int n, int c0, float* __restrict__ out_f32,
                                           uint16_t* __restrict__ out_bf16,
                                           float* __restrict__ lse_out, int lane) {
  using V = typename VecT<VEC>::T;
  using R = typename std::conditional<kBf16In, typename RawBf16<VEC>::T, V>::type;
  const int d = c0 + lane * VEC;
  auto load = [&](int r) -> R {
    const int64_t e = (int64_t)r * o_stride + d;
    if constexpr (kBf16In) return ld_raw_bf16<VEC, false>(o_base, e);
    else return ld<V, false>(static_cast<const float*>(o_base) + e);
  };
  R first[kB];
#pragma unroll
  for (int u = 0; u < kB; ++u)
    if (u < n) first[u] = load(u);
  auto lse_at = [&](int r) -> float {
    if (r >= n) return neg_inf();
    const float x = ld_lse(l_base + r * l_stride);
    return __builtin_isfinite(x) ? x : neg_inf();
  };
  float m = neg_inf();
  for (int r0 = 0; r0 < n; r0 += 64) m = fmaxf(m, lse_at(r0 + lane));
  m = wave_max_dpp(m);
  if (m == neg_inf()) {
    // every partial is empty
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      if (out_f32) out_f32[d + i] = 0.f;
      else out_bf16[d + i] = 0;
    }
    if (lse_out && lane == 0) *lse_out = neg_inf();
    return;
  }
  const float m2 = m * kLog2e;
  float wpart = 0.f;
  for (int r0 = 0; r0 < n; r0 += 64) {
    const float x = lse_at(r0 + lane);
    wpart += x == neg_inf() ? 0.f : exp2f(fmaf(x, kLog2e, -m2));
  }
  const float inv = 1.f / wave_sum_dpp(wpart);
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  auto add = [&](float w, const R& v) {
    float f[VEC];
    if constexpr (kBf16In) {
      widen_bf16<VEC>(v, f);
    } else {
#pragma unroll
      for (int i = 0; i < VEC; ++i) f[i] = reinterpret_cast<const float*>(&v)[i];
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = fmaf(w, f[i], acc[i]);
  };
  for (int r0 = 0; r0 < n; r0 += 64) {
    const float x = lse_at(r0 + lane);
    const float wl = x == neg_inf() ? 0.f : exp2f(fmaf(x, kLog2e, -m2));
    const int nr = n - r0 < 64 ? n - r0 : 64;
    // the weight of partial r0 + r + u (0 past the row's partials: lanes >= nr)
    auto wt = [&](int r, int u) -> float {
      return r + u < nr ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), r + u))
                        : 0.f;
    };
    if (r0 == 0) {
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const float w = wt(0, u);
        if (w != 0.f) add(w, first[u]);
      }
    }
    for (int r = r0 == 0 ? kB : 0; r < nr; r += kB) {
      float wv[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) wv[u] = wt(r, u);
      R v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (wv[u] != 0.f) v[u] = load(r0 + r + u);
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (wv[u] != 0.f) add(wv[u], v[u]);
    }
  }
  if (out_f32) {
    V o;
    float* po = reinterpret_cast<float*>(&o);
#pragma unroll
    for (int i = 0; i < VEC; ++i) po[i] = acc[i] * inv;
    st<V>(out_f32 + d, o);
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) out_bf16[d + i] = (uint16_t)f32_to_bf16_rne(acc[i] * inv);
  }
  if (lse_out && lane == 0) *lse_out = (m2 - __log2f(inv)) * kLn2;
}

// At most 8 partials and 2 chunks of 64 * VEC floats per lane: all loads up front.  The n
// lse values sit in lanes 0..7 and are reduced inside that 8-lane group; the weighted sum
// accumulates in place in the registers of the first partial, so that the loads in flight
// (up to 64 registers) leave room for the most waves per SIMD.  When every partial is empty
// all weights are 0 and the row comes out as O = 0, lse = -inf.
// merge_row_small for bf16 partials: the same steps, with the loads held raw (RawBf16) and
// a separate float accumulator per chunk.
template <int VEC, bool kBf16Out, bool kNt>
__device__ __forceinline__ void merge_row_small_bf16in(const void* __restrict__ o_base,
                                                       int64_t o_stride,
                                                       const float* __restrict__ l_base,
                                                       int64_t l_stride, int n, int dv,
                                                       void* __restrict__ out,
                                                       float* __restrict__ lse_out, int lane) {
  using V = typename VecT<VEC>::T;
  using R = typename RawBf16<VEC>::T;
  constexpr int kMaxN = 8, kMaxC = 2;
  const int nc = dv / (64 * VEC);
  float x = lane < n ? ld_lse(l_base + lane * l_stride) : neg_inf();
  R v[kMaxN][kMaxC];
#pragma unroll
  for (int r = 0; r < kMaxN; ++r)
#pragma unroll
    for (int c = 0; c < kMaxC; ++c)
      if (r < n && c < nc)
        v[r][c] = ld_raw_bf16<VEC, kNt>(o_base, (int64_t)r * o_stride + (c * 64 + lane) * VEC);
  x = __builtin_isfinite(x) ? x : neg_inf();
  const float m2 = lanes8_max(x) * kLog2e;   // -inf when every partial is empty
  const float wl = x == neg_inf() ? 0.f : exp2f(fmaf(x, kLog2e, -m2));
  const float sum = lanes8_sum(wl);
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  float acc[kMaxC][VEC];
#pragma unroll
  for (int c = 0; c < kMaxC; ++c)
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[c][i] = 0.f;
  // partials with weight 0 are never multiplied (their rows may hold anything)
#pragma unroll
  for (int r = 0; r < kMaxN; ++r) {
    if (r < n) {
      const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), r));
      if (wr != 0.f) {
#pragma unroll
        for (int c = 0; c < kMaxC; ++c) {
          if (c < nc) {
            float f[VEC];
            widen_bf16<VEC>(v[r][c], f);
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[c][i] = fmaf(wr, f[i], acc[c][i]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < kMaxC; ++c) {
    if (c < nc) {
      const int d = (c * 64 + lane) * VEC;
      if constexpr (!kBf16Out) {
        V o;
        float* po = reinterpret_cast<float*>(&o);
#pragma unroll
        for (int i = 0; i < VEC; ++i) po[i] = acc[c][i] * inv;
        st<V>(static_cast<float*>(out) + d, o);
      } else {
        uint16_t* ob = static_cast<uint16_t*>(out);
#pragma unroll
        for (int i = 0; i < VEC; ++i) ob[d + i] = (uint16_t)f32_to_bf16_rne(acc[c][i] * inv);
      }
    }
  }
  if (lse_out && lane == 0) *lse_out = sum > 0.f ? (m2 + __log2f(sum)) * kLn2 : neg_inf();
}

template <int VEC, bool kBf16Out, bool kBf16In, bool kNt>
__device__ __forceinline__ void merge_row_small(const void* __restrict__ o_base,
                                                int64_t o_stride,
                                                const float* __restrict__ l_base,
                                                int64_t l_stride, int n, int dv,
                                                void* __restrict__ out,
                                                float* __restrict__ lse_out, int lane) {
  if constexpr (kBf16In) {
    merge_row_small_bf16in<VEC, kBf16Out, kNt>(o_base, o_stride, l_base, l_stride, n, dv, out,
                                          lse_out, lane);
    return;
  }
  using V = typename VecT<VEC>::T;
  constexpr int kMaxN = 8, kMaxC = 2;
  const int nc = dv / (64 * VEC);
  float x = lane < n ? ld_lse(l_base + lane * l_stride) : neg_inf();
  V v[kMaxN][kMaxC];
#pragma unroll
  for (int r = 0; r < kMaxN; ++r)
#pragma unroll
    for (int c = 0; c < kMaxC; ++c)
      if (r < n && c < nc)
        v[r][c] = ldp<VEC, kBf16In, kNt>(o_base, (int64_t)r * o_stride + (c * 64 + lane) * VEC);
  x = __builtin_isfinite(x) ? x : neg_inf();
  const float m2 = lanes8_max(x) * kLog2e;   // -inf when every partial is empty
  const float wl = x == neg_inf() ? 0.f : exp2f(fmaf(x, kLog2e, -m2));
  const float sum = lanes8_sum(wl);
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  // partials with weight 0 are never multiplied (their rows may hold anything)
#pragma unroll
  for (int r = 0; r < kMaxN; ++r) {
    if (r < n) {
      const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), r));
#pragma unroll
      for (int c = 0; c < kMaxC; ++c) {
        if (c < nc) {
          float* a = reinterpret_cast<float*>(&v[0][c]);
          const float* pv = reinterpret_cast<const float*>(&v[r][c]);
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            if (r == 0) a[i] = wr != 0.f ? wr * a[i] : 0.f;
            else a[i] = wr != 0.f ? fmaf(wr, pv[i], a[i]) : a[i];
          }
        }
      }
    }
  }
  if (n == 0) {
#pragma unroll
    for (int c = 0; c < kMaxC; ++c) v[0][c] = V{};
  }
#pragma unroll
  for (int c = 0; c < kMaxC; ++c) {
    if (c < nc) {
      const int d = (c * 64 + lane) * VEC;
      const float* a = reinterpret_cast<const float*>(&v[0][c]);
      if constexpr (!kBf16Out) {
        V o;
        float* po = reinterpret_cast<float*>(&o);
#pragma unroll
        for (int i = 0; i < VEC; ++i) po[i] = a[i] * inv;
        st<V>(static_cast<float*>(out) + d, o);
      } else {
        uint16_t* ob = static_cast<uint16_t*>(out);
#pragma unroll
        for (int i = 0; i < VEC; ++i) ob[d + i] = (uint16_t)f32_to_bf16_rne(a[i] * inv);
      }
    }
  }
  if (lse_out && lane == 0) *lse_out = sum > 0.f ? (m2 + __log2f(sum)) * kLn2 : neg_inf();
}

// whether a row qualifies for merge_row_small
__host__ __device__ __forceinline__ bool merge_small_ok(int n, int dv, int vec) {
  return n <= 8 && dv % (64 * vec) == 0 && dv <= 2 * 64 * vec;
}

// split combine: waves (rows, or column chunks of rows) per workgroup
constexpr int kRowsPerBlock = 4;
// Split combines whose rows come to at most this many column chunks give each chunk a wave
// of its own: two waves per SIMD on 256 CUs, which is also what that kernel's registers
// allow (it holds up to 32 partial chunks per lane).
constexpr int64_t kWideCombineWaves = 2048;
// dcp_merge rows (waves) per workgroup.  Measured on MI355X, eight float32 partials of
// 64 x 128 rows x 512 dims from HBM: 28.4 us at 16 rows against 29.0 us at 8, 29.4 us at 4
// and 31.4 us at 1 (fewer, larger workgroups reach the stream's full rate sooner), 512 x 128
// rows equal; bf16 partials of 512 x 128 rows (held raw until use): 114.5 us at 4 rows,
// 113.0-115.0 at 8 and 115.7-116.7 at 16.
template <bool kBf16In>
constexpr int merge_rows_per_block() { return kBf16In ? 4 : 16; }

// dcp_merge with at most 8 partials: one row per wave, all loads up front
template <int VEC, bool kBf16Out, bool kBf16In, bool kNt>
__global__ __launch_bounds__(64 * merge_rows_per_block<kBf16In>()) void merge_small_kernel(
    const void* __restrict__ o_partials, const float* __restrict__ lse_partials, int n,
    int batch, int heads, int dv, void* __restrict__ out, float* __restrict__ lse_out) {
  const int64_t row = (int64_t)blockIdx.x * merge_rows_per_block<kBf16In>() +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rows = (int64_t)batch * heads;
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  void* o = kBf16Out ? (void*)(static_cast<uint16_t*>(out) + row * dv)
                     : (void*)(static_cast<float*>(out) + row * dv);
  const void* ob = kBf16In ? (const void*)(static_cast<const uint16_t*>(o_partials) + row * dv)
                           : (const void*)(static_cast<const float*>(o_partials) + row * dv);
  merge_row_small<VEC, kBf16Out, kBf16In, kNt>(ob, rows * dv, lse_partials + row, rows, n, dv,
                                               o, lse_out ? lse_out + row : nullptr, lane);
}

template <int VEC, bool kBf16In, bool kNt>
__global__ __launch_bounds__(64 * merge_rows_per_block<kBf16In>()) void merge_kernel(
    const void* __restrict__ o_partials, const float* __restrict__ lse_partials, int n,
    int batch, int heads, int dv, float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16,
    float* __restrict__ lse_out) {
  const int64_t row = (int64_t)blockIdx.x * merge_rows_per_block<kBf16In>() +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rows = (int64_t)batch * heads;
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const void* ob = kBf16In ? (const void*)(static_cast<const uint16_t*>(o_partials) + row * dv)
                           : (const void*)(static_cast<const float*>(o_partials) + row * dv);
  merge_row<VEC, kBf16In, kNt>(ob, rows * dv, lse_partials + row, rows, n, 0, dv,
                               out_f32 ? out_f32 + row * dv : nullptr,
                               out_bf16 ? out_bf16 + row * dv : nullptr,
                               lse_out ? lse_out + row : nullptr, lane);
}

// Split combine: request b's items [off[b], off[b+1]) hold partials of every head.  A
// request with a single item was written directly by the shard kernel; a request with no
// item (empty shard) gets O = 0, lse = -inf.
// Split partials are float32, or bf16 when kBf16In (widened exactly).
// One wave per row, or with kWide (few rows: long sequences split over many items) one wave
// per 64 * VEC columns of a row, whose first 32 bf16 (16 float32) partial loads leave with
// the lse loads: a row of up to 32 items costs one round trip instead of one per 8 partials.
// Measured on MI355X, MLA over 8 requests x 50000 local tokens (1024 rows of 512 columns,
// 32 bf16 partials each): 11.0 us against 24.8 us one wave per row; 64 requests (8192 rows,
// 4 partials) 9.7 us one wave per row against 24 us column-split.  The wave of the first
// columns writes lse.
template <int VEC, bool kBf16Out, bool kBf16In, bool kWide>
__global__ __launch_bounds__(64 * kRowsPerBlock) void split_combine_kernel(
    const int32_t* __restrict__ off, const float* __restrict__ plse, const void* __restrict__ po,
    int batch, int hq, int dv, void* __restrict__ o_out, float* __restrict__ lse_out) {
  const int64_t wave = (int64_t)blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int kCols = 64 * VEC;
  const int chunks = kWide ? dv / kCols : 1;   // the launcher picks kWide only if dv % kCols == 0
  const int64_t row = kWide ? wave / chunks : wave;
  const int c0 = kWide ? (int)(wave - row * chunks) * kCols : 0;
  if (row >= (int64_t)batch * hq) return;
  const int b = (int)(row / hq), h = (int)(row - (int64_t)b * hq);
  const int i0 = off[b], n = off[b + 1] - i0;
  if (n == 1) return;
  const int lane = threadIdx.x & 63;
  float* of = kBf16Out ? nullptr : static_cast<float*>(o_out) + row * dv;
  uint16_t* obf = kBf16Out ? static_cast<uint16_t*>(o_out) + row * dv : nullptr;
  const int64_t e0 = ((int64_t)i0 * hq + h) * dv;   // first element of the request's partials
  const void* pb = kBf16In ? (const void*)(static_cast<const uint16_t*>(po) + e0)
                           : (const void*)(static_cast<const float*>(po) + e0);
  // the split partials were just written by the shard kernel: plain loads (cache hits)
  if constexpr (kWide)
    merge_cols<VEC, kBf16In, kBf16In ? 32 : 16>(pb, (int64_t)hq * dv, plse + (int64_t)i0 * hq + h,
                                                hq, n, c0, of, obf,
                                                c0 == 0 ? lse_out + row : nullptr, lane);
  else if (merge_small_ok(n, dv, VEC))
    merge_row_small<VEC, kBf16Out, kBf16In, false>(pb, (int64_t)hq * dv,
                                                   plse + (int64_t)i0 * hq + h, hq, n, dv,
                                                   kBf16Out ? (void*)obf : (void*)of,
                                                   lse_out + row, lane);
  else
    merge_row<VEC, kBf16In, false>(pb, (int64_t)hq * dv, plse + (int64_t)i0 * hq + h, hq, n,
                                   0, dv, of, obf, lse_out + row, lane);
}

int pick_vec(int dv) {
  if (dv % 256 == 0) return 4;
  if (dv % 128 == 0) return 2;
  return 1;
}

}  // namespace

hipError_t launch_merge(const void* o_partials, int in_bf16, const float* lse_partials, int n,
                        int batch, int heads, int dv, void* o_out, int out_bf16, float* lse_out,
                        hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t rows = (int64_t)batch * heads;
  // rows per workgroup of the kernel launched below (its template argument I = in_bf16)
  const int rpb = in_bf16 ? merge_rows_per_block<true>() : merge_rows_per_block<false>();
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  const dim3 block(64 * rpb);
  float* of = out_bf16 ? nullptr : static_cast<float*>(o_out);
  uint16_t* ob = out_bf16 ? static_cast<uint16_t*>(o_out) : nullptr;
  const int vec = pick_vec(dv);
  // Partials that fit well inside the 256 MB last-level cache (MALL) are usually still there
  // when the merge follows the shard calls: plain loads hit it (measured at the MLA decode
  // shape, 134 MB of float32 partials: 23.1 us in cache against 26.0 us with nt loads, and
  // 28.6 against 28.0 us from HBM).  Larger ones stream with the nt policy (1.21 GB: 203
  // against 226 us).
  const double part_bytes = (double)n * rows * dv * (in_bf16 ? 2 : 4);
  const bool nt = part_bytes > 192.0 * 1024 * 1024;
  if (merge_small_ok(n, dv, vec)) {
#define DCP_MERGE_SMALL(V, B, I)                                                               \
  do {                                                                                         \
    if (nt)                                                                                    \
      hipExtLaunchKernelGGL((merge_small_kernel<V, B, I, true>), grid, block, 0, stream, ev0,  \
                            ev1, 0, o_partials, lse_partials, n, batch, heads, dv, o_out,      \
                            lse_out);                                                          \
    else                                                                                       \
      hipExtLaunchKernelGGL((merge_small_kernel<V, B, I, false>), grid, block, 0, stream, ev0, \
                            ev1, 0, o_partials, lse_partials, n, batch, heads, dv, o_out,      \
                            lse_out);                                                          \
  } while (0)
#define DCP_MERGE_SMALL_V(B, I)            \
  if (vec == 4) DCP_MERGE_SMALL(4, B, I);  \
  else if (vec == 2) DCP_MERGE_SMALL(2, B, I); \
  else DCP_MERGE_SMALL(1, B, I)
    if (out_bf16) {
      if (in_bf16) { DCP_MERGE_SMALL_V(true, true); } else { DCP_MERGE_SMALL_V(true, false); }
    } else {
      if (in_bf16) { DCP_MERGE_SMALL_V(false, true); } else { DCP_MERGE_SMALL_V(false, false); }
    }
#undef DCP_MERGE_SMALL_V
#undef DCP_MERGE_SMALL
    return hipGetLastError();
  }
#define DCP_MERGE(V, I)                                                                        \
  do {                                                                                         \
    if (nt)                                                                                    \
      hipExtLaunchKernelGGL((merge_kernel<V, I, true>), grid, block, 0, stream, ev0, ev1, 0,   \
                            o_partials, lse_partials, n, batch, heads, dv, of, ob, lse_out);   \
    else                                                                                       \
      hipExtLaunchKernelGGL((merge_kernel<V, I, false>), grid, block, 0, stream, ev0, ev1, 0,  \
                            o_partials, lse_partials, n, batch, heads, dv, of, ob, lse_out);   \
  } while (0)
  if (in_bf16) {
    if (vec == 4) DCP_MERGE(4, true);
    else if (vec == 2) DCP_MERGE(2, true);
    else DCP_MERGE(1, true);
  } else {
    if (vec == 4) DCP_MERGE(4, false);
    else if (vec == 2) DCP_MERGE(2, false);
    else DCP_MERGE(1, false);
  }
#undef DCP_MERGE
  return hipGetLastError();
}

hipError_t launch_split_combine(const WsPtrs& ws, int batch, int hq, int dv, void* o_out,
                                int out_bf16, float* lse_out, hipStream_t stream) {
  const int64_t rows = (int64_t)batch * hq;
  const int vec = pick_vec(dv);
  const int64_t chunks = dv % (64 * vec) == 0 ? dv / (64 * vec) : 1;
  const bool wide = chunks > 1 && rows * chunks <= kWideCombineWaves;
  const int64_t waves = wide ? rows * chunks : rows;
  const dim3 grid((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
  const dim3 block(64 * kRowsPerBlock);
#define DCP_COMBINE(V, B, I)                                                                   \
  do {                                                                                         \
    if (wide)                                                                                  \
      hipLaunchKernelGGL((split_combine_kernel<V, B, I, true>), grid, block, 0, stream, ws.off, \
                         ws.plse, ws.po, batch, hq, dv, o_out, lse_out);                       \
    else                                                                                       \
      hipLaunchKernelGGL((split_combine_kernel<V, B, I, false>), grid, block, 0, stream,       \
                         ws.off, ws.plse, ws.po, batch, hq, dv, o_out, lse_out);               \
  } while (0)
#define DCP_COMBINE_I(V, B)                \
  if (ws.po_bf16) DCP_COMBINE(V, B, true); \
  else DCP_COMBINE(V, B, false)
  switch (vec * 2 + (out_bf16 ? 1 : 0)) {
    case 8: DCP_COMBINE_I(4, false); break;
    case 9: DCP_COMBINE_I(4, true); break;
    case 4: DCP_COMBINE_I(2, false); break;
    case 5: DCP_COMBINE_I(2, true); break;
    case 2: DCP_COMBINE_I(1, false); break;
    default: DCP_COMBINE_I(1, true);
  }
#undef DCP_COMBINE_I
#undef DCP_COMBINE
  return hipGetLastError();
}

}  // namespace dcp

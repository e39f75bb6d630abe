// Host-rule checks built by tests/test_host_sanitized.py with address and undefined-
// behaviour sanitizers (any finding aborts the run).  Covers the walker (ownership and the
// local-to-global map of "How DCP works": token t on rank (t / I) mod C) and the argument
// checks, work-item targets and workspace layout of the shard, merge and slots calls.
//
//   host_rules_check self                 every check below; prints "ok" at the end
//   host_rules_check count L rank C I     local token count (64-bit and 32-bit forms)
//   host_rules_check positions L rank C I the count, then every owned global position
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <limits>
#include <vector>

#include "host_rules.h"

namespace {

int g_fail = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
      if (++g_fail > 20) exit(1);                          \
    }                                                      \
  } while (0)

typedef __int128 i128;

constexpr int64_t kLmax = 2147483647;   // sequence lengths stay below 2^31

uint64_t g_rng = 0x9e3779b97f4a7c15ull;
uint64_t next_u64() {   // splitmix64
  uint64_t z = (g_rng += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
template <class T, size_t N>
T pick(const T (&pool)[N]) { return pool[next_u64() % N]; }

// ---- walker: brute force on small sequences ------------------------------------------
void walker_small() {
  for (int C = 1; C <= 9; ++C)
    for (int I = 1; I <= 70; I += (I < 10 ? 1 : 7))
      for (int L = 0; L <= 3 * C * I + 5; ++L)
        for (int r = 0; r < C; ++r) {
          std::vector<uint32_t> owned;
          for (int t = 0; t < L; ++t)
            if ((t / I) % C == r) owned.push_back((uint32_t)t);
          const int64_t n64 = dcp_walk_local_count(L, r, C, I);
          const uint32_t n32 = dcp_walk_local_count32((uint32_t)L, (uint32_t)r, (uint32_t)C,
                                                      (uint32_t)I);
          CHECK(n64 == (int64_t)owned.size(), "L %d r %d C %d I %d: %lld vs %zu", L, r, C, I,
                (long long)n64, owned.size());
          CHECK(n32 == owned.size(), "L %d r %d C %d I %d (32-bit)", L, r, C, I);
          for (size_t j = 0; j < owned.size(); ++j)
            CHECK(dcp_walk_global_pos((uint32_t)j, r, C, I) == owned[j], "pos j %zu", j);
        }
}

// ---- walker: every position below 2^31 - 1 for a few (C, I) ---------------------------
// Visits t = 0, 1, ..., 2^31 - 2 in order; the j-th token met on rank r must be the walker's
// global position of local index j, and at checkpoints the closed-form counts of the prefix
// must equal the running counts.
void walker_exhaustive(uint32_t C, uint32_t I) {
  const uint64_t Lmax = (uint64_t)kLmax;
  std::vector<uint32_t> cnt(C, 0);
  uint64_t t = 0;
  uint64_t next_check = 1;
  for (uint64_t c = 0; t < Lmax; ++c) {
    const uint32_t r = (uint32_t)(c % C);
    for (uint32_t i = 0; i < I && t < Lmax; ++i, ++t) {
      const uint32_t j = cnt[r]++;
      if (dcp_walk_global_pos(j, r, C, I) != (uint32_t)t) {
        CHECK(false, "C %u I %u: local %u of rank %u maps to %u, expected %llu", C, I, j, r,
              dcp_walk_global_pos(j, r, C, I), (unsigned long long)t);
        return;
      }
    }
    if (t >= next_check || t >= Lmax) {
      for (uint32_t q = 0; q < C; ++q) {
        CHECK(dcp_walk_local_count((int64_t)t, q, C, I) == cnt[q], "count64 L %llu",
              (unsigned long long)t);
        CHECK(dcp_walk_local_count32((uint32_t)t, q, C, I) == cnt[q], "count32 L %llu",
              (unsigned long long)t);
      }
      next_check = t + 1 + (next_u64() % (1u << 22));
    }
  }
  uint64_t total = 0;
  for (uint32_t q = 0; q < C; ++q) total += cnt[q];
  CHECK(total == Lmax, "total %llu", (unsigned long long)total);
}

// ---- walker: invariants at the 2^31 bounds (random and extreme parameters) ------------
void walker_bounds() {
  const uint32_t Is[] = {1, 2, 3, 16, 64, 127, 128, 4096, 65536, 1u << 20, 1000003u,
                         (1u << 30) - 1};
  const uint32_t Cs[] = {1, 2, 3, 4, 7, 8, 16, 64, 1024};
  for (int it = 0; it < 200000; ++it) {
    const uint32_t I = pick(Is), C = pick(Cs);
    if ((uint64_t)I * C > (uint64_t)kLmax) continue;
    uint32_t L;
    switch (it % 4) {
      case 0: L = (uint32_t)kLmax; break;
      case 1: L = (uint32_t)(next_u64() % ((uint64_t)kLmax + 1)); break;
      case 2: L = (uint32_t)((uint64_t)I * C * (next_u64() % 4096)) ; break;
      default: L = (uint32_t)(next_u64() % (4ull * I * C + 3)); break;
    }
    if (L > (uint32_t)kLmax) L = (uint32_t)kLmax;
    uint64_t total = 0;
    for (uint32_t r = 0; r < C && r < 64; ++r) {
      const int64_t n = dcp_walk_local_count(L, r, C, I);
      CHECK(n >= 0 && (uint64_t)n == dcp_walk_local_count32(L, r, C, I), "L %u r %u C %u I %u",
            L, r, C, I);
      // closed form against a count of whole chunks: chunk k (tokens kI .. kI + I - 1) sits
      // on rank k mod C; ranks below r get one more chunk than r in a partial round
      const uint64_t chunks = L / I, rest = L % I;
      const uint64_t mine = chunks / C + (r < chunks % C ? 1 : 0);
      const uint64_t expect = mine * I + (chunks % C == r ? rest : 0);
      CHECK((uint64_t)n == expect, "L %u r %u C %u I %u: %lld vs %llu", L, r, C, I,
            (long long)n, (unsigned long long)expect);
      total += (uint64_t)n;
      if (n > 0) {
        const uint32_t last = dcp_walk_global_pos((uint32_t)n - 1, r, C, I);
        CHECK(last < L && (last / I) % C == r, "last L %u r %u C %u I %u", L, r, C, I);
        const uint64_t after = (uint64_t)(n / I) * I * C + (uint64_t)r * I + n % I;
        CHECK(after >= L, "the walk does not end at L: L %u r %u", L, r);
      }
    }
    if (C <= 64) CHECK(total == L, "sum over ranks L %u C %u I %u", L, C, I);
  }
}

// ---- argument checks against the contract written independently in 128-bit ----------
int expect_desc(const dcp_attn_desc* d, int q_len, int batch, int64_t msl, int cp, int il) {
  if (!d || batch < 0 || msl < 0 || msl > 2147483647) return DCP_EINVAL;
  if (q_len < 1) return DCP_EINVAL;
  if (q_len > 4) return DCP_EUNSUPPORTED;
  if (cp < 1 || il < 1 || (i128)cp * il > 2147483647) return DCP_EINVAL;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0)
    return DCP_EINVAL;
  if (d->head_dim_qk < 1 || d->head_dim_v < 1 || d->block_size < 1 ||
      d->max_blocks_per_seq < 1 || d->num_blocks < 1)
    return DCP_EINVAL;
  if ((i128)d->num_blocks * d->block_size * d->num_kv_heads > 2147483647) return DCP_EUNSUPPORTED;
  if ((i128)d->max_blocks_per_seq * d->block_size > 2147483647) return DCP_EUNSUPPORTED;
  const int dmax = d->head_dim_qk > d->head_dim_v ? d->head_dim_qk : d->head_dim_v;
  if ((i128)q_len * d->num_q_heads * dmax > 2147483647) return DCP_EUNSUPPORTED;
  if (d->dtype != DCP_F32 && d->dtype != DCP_BF16) return DCP_EINVAL;
  const i128 group = d->num_q_heads / d->num_kv_heads;
  if (d->kind == DCP_GQA) {
    const i128 row_bytes = (i128)d->head_dim_qk * (d->dtype == DCP_BF16 ? 2 : 4);
    if (d->head_dim_qk != d->head_dim_v || row_bytes != 256 || group * q_len > 64)
      return DCP_EUNSUPPORTED;
    return DCP_OK;
  }
  if (d->kind == DCP_MLA) {
    const bool heads_ok = d->num_q_heads == 16 || d->num_q_heads == 32 ||
                          d->num_q_heads == 64 || d->num_q_heads == 128;
    if (d->dtype != DCP_BF16 || !heads_ok || d->num_kv_heads != 1 ||
        d->head_dim_qk != 576 || d->head_dim_v != 512)
      return DCP_EUNSUPPORTED;
    return DCP_OK;
  }
  return DCP_EINVAL;
}

const int32_t kInts[] = {std::numeric_limits<int32_t>::min(), -7, -1, 0, 1, 2, 3, 4, 5, 7, 8,
                         16, 32, 63, 64, 65, 100, 127, 128, 129, 256, 512, 576, 1000, 4096,
                         65536, 1 << 20, 1 << 24, (1 << 30) - 1, 1 << 30,
                         std::numeric_limits<int32_t>::max()};
const int64_t kI64s[] = {std::numeric_limits<int64_t>::min(), -1, 0, 1, 2, 1000, 1 << 20,
                         2147483647LL, 2147483648LL, 1LL << 40, 1LL << 62,
                         std::numeric_limits<int64_t>::max()};

dcp_attn_desc random_desc(bool plausible) {
  dcp_attn_desc d;
  if (plausible) {
    // mostly valid shapes with one field (sometimes) pushed to an extreme
    const bool mla = next_u64() & 1;
    const int32_t groups[] = {1, 2, 3, 5, 7, 8, 12, 16, 21, 32, 64, 65};
    const int32_t hkvs[] = {1, 2, 4, 8, 16, 64};
    d.kind = mla ? DCP_MLA : DCP_GQA;
    d.dtype = (mla || (next_u64() & 1)) ? DCP_BF16 : DCP_F32;
    d.num_kv_heads = mla ? 1 : pick(hkvs);
    const int32_t mla_heads[] = {16, 32, 64, 128, 48, 256};
    d.num_q_heads = mla ? pick(mla_heads) : d.num_kv_heads * pick(groups);
    d.head_dim_qk = mla ? 576 : (d.dtype == DCP_BF16 ? 128 : 64);
    d.head_dim_v = mla ? 512 : d.head_dim_qk;
    const int32_t bss[] = {1, 16, 64, 128, 1024};
    d.block_size = pick(bss);
    d.max_blocks_per_seq = 1 + (int32_t)(next_u64() % 4096);
    d.num_blocks = 1 + (int64_t)(next_u64() % 100000);
    switch (next_u64() % 12) {
      case 0: d.num_q_heads = pick(kInts); break;
      case 1: d.num_kv_heads = pick(kInts); break;
      case 2: d.head_dim_qk = pick(kInts); break;
      case 3: d.head_dim_v = pick(kInts); break;
      case 4: d.block_size = pick(kInts); break;
      case 5: d.max_blocks_per_seq = pick(kInts); break;
      case 6: d.num_blocks = pick(kI64s); break;
      case 7: d.dtype = pick(kInts); break;
      case 8: d.kind = pick(kInts); break;
      default: break;
    }
  } else {
    d.kind = pick(kInts);
    d.dtype = pick(kInts);
    d.num_q_heads = pick(kInts);
    d.num_kv_heads = pick(kInts);
    d.head_dim_qk = pick(kInts);
    d.head_dim_v = pick(kInts);
    d.block_size = pick(kInts);
    d.max_blocks_per_seq = pick(kInts);
    d.num_blocks = pick(kI64s);
  }
  return d;
}

void layout_invariants(const dcp_attn_desc& d, int q_len, int batch, int cus,
                       const dcp::Plan& p) {
  const dcp::WsLayout& w = p.lay;
  CHECK(p.target >= 1 && p.max_items == (int64_t)batch + p.target, "target %lld",
        (long long)p.target);
  if (d.kind == DCP_GQA) {
    const int64_t rows = (int64_t)q_len * (d.num_q_heads / d.num_kv_heads);
    // bf16 queries: up to 48 rows per workgroup, more as two 32-row slices
    const int64_t slices = (d.dtype == DCP_BF16 && rows > 48) ? 2 : 1;
    CHECK(p.target == std::max<int64_t>(1, 2LL * cus / (d.num_kv_heads * slices)), "gqa target");
    CHECK(p.tile == 64 && p.min_chunk == 64 && w.po_bf16 == 0, "gqa plan");
  } else {
    CHECK(p.target == std::max<int64_t>(1, cus / q_len), "mla target");
    CHECK(p.tile == 32 && p.min_chunk == 128 && w.po_bf16 == 1, "mla plan");
  }
  const i128 rows = (i128)q_len * d.num_q_heads;
  const i128 need_off = 4 * ((i128)batch + 1), need_items = 16 * (i128)p.max_items;
  const i128 need_plse = 4 * (i128)p.max_items * rows;
  const i128 need_po = (w.po_bf16 ? 2 : 4) * (i128)p.max_items * rows * d.head_dim_v;
  CHECK(w.off_off == 256, "header");
  CHECK(w.off_off % 256 == 0 && w.items_off % 256 == 0 && w.plse_off % 256 == 0 &&
            w.po_off % 256 == 0 && w.total % 256 == 0, "alignment");
  CHECK((i128)w.items_off - w.off_off >= need_off, "off section");
  CHECK((i128)w.plse_off - w.items_off >= need_items, "items section");
  CHECK((i128)w.po_off - w.plse_off >= need_plse, "plse section");
  CHECK((i128)w.total - w.po_off >= need_po, "po section");
  CHECK((i128)w.total - w.po_off < need_po + 256, "po section not padded beyond alignment");
}

void desc_fuzz() {
  const int qls[] = {-1, 0, 1, 2, 3, 4, 5, 1 << 30};
  const int batches[] = {-1, 0, 1, 3, 64, 512, 1 << 20, std::numeric_limits<int>::max()};
  const int64_t msls[] = {-1, 0, 1, 67584, 200000, 2147483647LL, 2147483648LL,
                          std::numeric_limits<int64_t>::max()};
  const int cps[] = {-1, 0, 1, 2, 3, 4, 8, 16, 1 << 16, std::numeric_limits<int>::max()};
  const int ils[] = {-1, 0, 1, 3, 16, 64, 128, 1 << 16, std::numeric_limits<int>::max()};
  const int cuss[] = {1, 80, 104, 256, 304};
  int ok = 0;
  for (int it = 0; it < 400000; ++it) {
    const dcp_attn_desc d = random_desc(it % 3 != 0);
    const int q_len = (it % 5 == 0) ? pick(qls) : 1 + (int)(next_u64() % 4);
    const int batch = pick(batches);
    const int64_t msl = pick(msls);
    const int cp = pick(cps), il = pick(ils);
    const int got = dcp::check_desc(&d, q_len, batch, msl, cp, il);
    const int want = expect_desc(&d, q_len, batch, msl, cp, il);
    CHECK(got == want, "check_desc %d vs %d (kind %d dtype %d hq %d hkv %d dk %d dv %d B %d "
          "mb %d nb %lld ql %d batch %d cp %d il %d)", got, want, d.kind, d.dtype,
          d.num_q_heads, d.num_kv_heads, d.head_dim_qk, d.head_dim_v, d.block_size,
          d.max_blocks_per_seq, (long long)d.num_blocks, q_len, batch, cp, il);
    if (got == DCP_OK) {
      ++ok;
      const int cus = pick(cuss);
      dcp::Plan p;
      CHECK(dcp::make_plan(&d, q_len, batch, cus, &p), "make_plan");
      layout_invariants(d, q_len, batch, cus, p);
    }
  }
  CHECK(dcp::check_desc(nullptr, 1, 1, 1, 1, 1) == DCP_EINVAL, "null desc");
  CHECK(ok > 10000, "too few valid descriptors drawn: %d", ok);
}

// workspace bytes of a (valid) shard shape on a device with `cus` compute units
size_t ws_need(const dcp_attn_desc* d, int q_len, int batch, int cus, dcp::Plan* p) {
  CHECK(dcp::check_desc(d, q_len, batch, 32768, 8, 128) == DCP_OK, "shape");
  CHECK(dcp::make_plan(d, q_len, batch, cus, p), "plan");
  return p->lay.total;
}

// ---- the shard call's remaining checks, in order -------------------------------------
void shard_args() {
  alignas(256) static char buf[4096];
  dcp_attn_desc d{DCP_GQA, DCP_BF16, 8, 1, 128, 128, 128, 256, 4096};
  const void* q = buf;
  const void* kv = buf + 256;
  const void* v = buf + 512;
  const int32_t* bt = reinterpret_cast<const int32_t*>(buf + 768);
  const int32_t* lens = reinterpret_cast<const int32_t*>(buf + 1024);
  const void* o = buf + 1280;
  const float* lse = reinterpret_cast<const float*>(buf + 1536);
  int cus_calls = 0;
  auto cus = [&]() { ++cus_calls; return 256; };
  dcp::Plan p;
  const size_t need = ws_need(&d, 1, 64, 256, &p);
  auto call = [&](const dcp_attn_desc* dd, int ql, int odt, const void* qq, const void* kk,
                  const void* vv, const int32_t* b, const int32_t* l, int batch, int rank,
                  int cp, float scale, const void* oo, const float* ls, const void* ws,
                  size_t wsb, const dcp::KvFp8* f8) {
    dcp::Plan pp;
    return dcp::check_shard_args(dd, ql, odt, qq, kk, vv, b, l, batch, 32768, rank, cp, 128,
                                 scale, oo, ls, ws, wsb, f8, cus, &pp);
  };
  const void* ws = buf;   // never dereferenced: only its address is checked
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need, nullptr) ==
            DCP_OK, "valid call");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need - 1,
             nullptr) == DCP_EWORKSPACE, "workspace one byte short");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, buf + 16, need,
             nullptr) == DCP_EWORKSPACE, "workspace misaligned");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, nullptr, need,
             nullptr) == DCP_EWORKSPACE, "workspace null");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 2, 2, 0.1f, o, lse, ws, need, nullptr) ==
            DCP_EINVAL, "rank == cp");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, -1, 2, 0.1f, o, lse, ws, need, nullptr) ==
            DCP_EINVAL, "rank < 0");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, NAN, o, lse, ws, need, nullptr) ==
            DCP_EINVAL, "NaN scale");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, INFINITY, o, lse, ws, need,
             nullptr) == DCP_EINVAL, "inf scale");
  CHECK(call(&d, 1, 7, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need, nullptr) ==
            DCP_EINVAL, "bad o_dtype");
  CHECK(call(&d, 1, DCP_F32, q, kv, nullptr, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need,
             nullptr) == DCP_EINVAL, "GQA without V");
  CHECK(call(&d, 1, DCP_F32, buf + 8, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need,
             nullptr) == DCP_EINVAL, "q misaligned");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, buf + 4, lse, ws, need,
             nullptr) == DCP_EINVAL, "o misaligned");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, nullptr, lens, 64, 0, 2, 0.1f, o, lse, ws, need,
             nullptr) == DCP_EINVAL, "null block table");
  const int before = cus_calls;
  CHECK(call(&d, 1, DCP_F32, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 2, 0.1f,
             nullptr, nullptr, nullptr, 0, nullptr) == DCP_OK, "batch 0 needs no buffers");
  CHECK(cus_calls == before, "the device is not queried for a call with nothing to do");
  auto no_cus = []() { return 0; };
  dcp::Plan pp;
  CHECK(dcp::check_shard_args(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 32768, 0, 2, 128, 0.1f,
                              o, lse, ws, need, nullptr, no_cus, &pp) == DCP_ELAUNCH,
        "no device");
  const dcp::KvFp8 good{0.5f, 2.0f}, bad{INFINITY, 1.0f};
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need, &good) ==
            DCP_OK, "fp8 cache");
  CHECK(call(&d, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need, &bad) ==
            DCP_EINVAL, "fp8 scale inf");
  dcp_attn_desc f32 = d;
  f32.dtype = DCP_F32;
  f32.head_dim_qk = f32.head_dim_v = 64;
  CHECK(call(&f32, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need, &good) ==
            DCP_EUNSUPPORTED, "fp8 cache with f32 queries");
  dcp_attn_desc g80 = d;
  g80.num_q_heads = 80;
  CHECK(call(&g80, 1, DCP_F32, q, kv, v, bt, lens, 64, 0, 2, 0.1f, o, lse, ws, need, &good) ==
            DCP_EUNSUPPORTED, "fp8 cache with 80 rows per KV head");
  dcp_attn_desc mla{DCP_MLA, DCP_BF16, 128, 1, 576, 512, 64, 1056, 100000};
  dcp::Plan pm;
  const size_t need_mla = ws_need(&mla, 2, 64, 256, &pm);
  CHECK(call(&mla, 2, DCP_BF16, q, kv, nullptr, bt, lens, 64, 7, 8, 0.07f, o, lse, ws,
             need_mla, nullptr) == DCP_OK, "MLA q_len 2");
  CHECK(call(&mla, 2, DCP_BF16, q, kv, v, bt, lens, 64, 7, 8, 0.07f, o, lse, ws, need_mla,
             nullptr) == DCP_EINVAL, "MLA with a V pointer");
  CHECK(call(&mla, 2, DCP_BF16, q, kv, nullptr, bt, lens, 64, 7, 8, 0.07f, o, lse, ws,
             need_mla, &good) == DCP_EUNSUPPORTED, "MLA with an fp8 cache");
}

int expect_merge(int in_dt, int cp, int batch, int heads, int dv, int out_dt, bool ptrs,
                 bool aligned16) {
  if (cp < 1 || batch < 0 || heads < 1 || dv < 1) return DCP_EINVAL;
  if (out_dt != DCP_F32 && out_dt != DCP_BF16) return DCP_EINVAL;
  if (in_dt != DCP_F32 && in_dt != DCP_BF16) return DCP_EINVAL;
  if ((i128)batch * heads * dv * cp > ((i128)1 << 40)) return DCP_EUNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!ptrs) return DCP_EINVAL;
  if (!aligned16) return DCP_EINVAL;
  return DCP_OK;
}

void merge_fuzz() {
  alignas(16) static char buf[64];
  for (int it = 0; it < 200000; ++it) {
    const int cp = pick(kInts), batch = pick(kInts), heads = pick(kInts), dv = pick(kInts);
    const int in_dt = (it % 7 == 0) ? pick(kInts) : (int)(next_u64() % 2);
    const int out_dt = (it % 11 == 0) ? pick(kInts) : (int)(next_u64() % 2);
    const bool ptrs = (it % 13) != 0, al = (it % 17) != 0;
    const void* po = ptrs ? (al ? buf : buf + 4) : nullptr;
    const int got = dcp::check_merge_args(po, in_dt, ptrs ? reinterpret_cast<float*>(buf) : nullptr,
                                          cp, batch, heads, dv, ptrs ? buf : nullptr, out_dt);
    const int want = expect_merge(in_dt, cp, batch, heads, dv, out_dt, ptrs, al);
    CHECK(got == want, "merge %d vs %d (cp %d b %d h %d dv %d)", got, want, cp, batch, heads, dv);
  }
}

int expect_slots(int batch, int mb, int bs, int64_t nb, int rank, int cp, int il, bool ptrs,
                 bool ws_ok) {
  if (batch < 0 || mb < 1 || bs < 1 || nb < 1) return DCP_EINVAL;
  if (cp < 1 || il < 1 || rank < 0 || rank >= cp) return DCP_EINVAL;
  if ((i128)cp * il > 2147483647 || (i128)mb * bs > 2147483647) return DCP_EUNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!ptrs) return DCP_EINVAL;
  if (!ws_ok) return DCP_EWORKSPACE;
  return DCP_OK;
}

void slots_fuzz() {
  alignas(256) static char buf[512];
  for (int it = 0; it < 200000; ++it) {
    const int batch = pick(kInts), mb = pick(kInts), bs = pick(kInts), rank = pick(kInts);
    const int cp = pick(kInts), il = pick(kInts);
    const int64_t nb = pick(kI64s);
    const bool ptrs = (it % 13) != 0, ws_ok = (it % 7) != 0;
    const int32_t* p32 = ptrs ? reinterpret_cast<const int32_t*>(buf) : nullptr;
    const int64_t* p64 = ptrs ? reinterpret_cast<const int64_t*>(buf) : nullptr;
    const void* ws = ws_ok ? buf : ((it % 2) ? nullptr : buf + 8);
    const int got = dcp::check_slots_args(p32, p32, batch, mb, bs, nb, rank, cp, il, p64, p64, ws);
    const int want = expect_slots(batch, mb, bs, nb, rank, cp, il, ptrs, ws_ok);
    CHECK(got == want, "slots %d vs %d", got, want);
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc == 6 && (!strcmp(argv[1], "count") || !strcmp(argv[1], "positions"))) {
    const int64_t L = atoll(argv[2]);
    const int r = atoi(argv[3]), C = atoi(argv[4]), I = atoi(argv[5]);
    const int64_t n = dcp_walk_local_count(L, r, C, I);
    const uint32_t n32 = dcp_walk_local_count32((uint32_t)L, r, C, I);
    printf("%lld %u\n", (long long)n, n32);
    if (!strcmp(argv[1], "positions"))
      for (int64_t j = 0; j < n; ++j) printf("%u\n", dcp_walk_global_pos((uint32_t)j, r, C, I));
    return 0;
  }
  if (argc != 2 || strcmp(argv[1], "self")) {
    fprintf(stderr, "usage: %s self | count L rank C I | positions L rank C I\n", argv[0]);
    return 2;
  }
  walker_small();
  walker_bounds();
  const uint32_t ex[][2] = {{8, 64}, {3, 1}, {5, 1000003}};
  for (const auto& ci : ex) walker_exhaustive(ci[0], ci[1]);
  desc_fuzz();
  shard_args();
  merge_fuzz();
  slots_fuzz();
  if (g_fail) {
    fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  printf("ok\n");
  return 0;
}

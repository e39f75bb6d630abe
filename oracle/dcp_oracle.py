"""Plain fp64 CPU oracle for decode context parallelism (DCP) shard attention and LSE merge.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this module. The HIP library never calls it, and this module
imports nothing from the HIP side: it takes numpy arrays and returns numpy arrays.

Sources (cited by page title and section):
  [Blog]  "vLLM Decode Context Parallelism for long-context workloads" (agentlenshq.com,
          zh-TW).  Sections used: "How DCP works" (sequence-dimension sharding with the
          200K-token / 4-GPU example), "DCP execution flow" (gathered Q, local attention
          against the local KV slice, partial outputs plus LSE merged with the
          online-softmax trick), "MLA backend", "GQA backend" (the size constraints).
  [Guide] "Context Parallel Guide" (vLLM Ascend docs).  Sections used: "Usage ->
          Decode Context Parallel" (--block-size and --cp-kv-cache-interleave-size),
          "Decode Context Parallel -> Constraints" (MLA and GQA size rules, and setting
          the interleave size to the KV block size).

Everything is computed in float64 from the exact input values (bf16 inputs are upcast
exactly by the caller).  Every function here is the plain definition of what it computes;
there is no tiling, fusion or reordering.

Readings taken where the pages are silent (also listed in the design notes):
  R1  token t of a sequence lives on DCP rank floor(t / interleave) mod cp_size.  The
      blog's contiguous 200K/4-GPU split is the special case interleave = L / cp_size.
  R2  owned tokens are listed in ascending global position.
  R3  lse is the natural-log log-sum-exp of the scaled scores scale * q.k.
  R4  an empty shard yields O = 0 and lse = -inf; the merge gives such a partial weight 0
      whatever its O holds.
  R5  the decode query attends to every token t < seq_len with no mask.
  R6  GQA query head h reads KV head h // (Hq / Hkv).
  R7  MLA: one latent row per token serves as the key (all 576 columns) and its first 512
      columns serve as the value.
  R8  multi-token decode (speculative decoding / multi-token prediction combined with DCP,
      a pairing the guide lists as supported and the blog's roadmap names): a request
      carries q_len query rows whose keys and values are already the last q_len tokens of
      its cache; row i sits at position seq_len - q_len + i and attends every position up
      to and including its own (a causal mask among the draft tokens, aligned to the end
      of the sequence).  A row whose position is negative attends nothing.
  R9  fp8 KV cache (the lower-byte KV variant; the pages leave the KV dtype open): K and V
      pages hold OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa bits;
      exponent 0 is subnormal; S.1111.111 is NaN; no infinities), each tensor with one
      float32 scale: the cached value is decode(code) * scale.  Attention is then the plain
      definition over those values; queries keep their own dtype.
"""

import math

import numpy as np

NEG_INF = float("-inf")


# ----------------------------------------------------------------------------------------
# Ownership and the block-table walk  ([Blog] "How DCP works"; [Guide] "Usage -> Decode
# Context Parallel", the --cp-kv-cache-interleave-size and --block-size flags)
# ----------------------------------------------------------------------------------------

def owner_of(t, cp_size, interleave):
    """DCP rank that stores global token position t (reading R1)."""
    return (np.asarray(t) // interleave) % cp_size


def owned_tokens(seq_len, rank, cp_size, interleave):
    """Global positions t < seq_len stored on `rank`, ascending (reading R2).

    A plain filter over every position: deliberately not a closed form."""
    t = np.arange(int(seq_len), dtype=np.int64)
    return t[owner_of(t, cp_size, interleave) == rank]


def owned_count(seq_len, rank, cp_size, interleave):
    """Number of tokens a rank stores for a sequence of length seq_len."""
    return int(owned_tokens(seq_len, rank, cp_size, interleave).size)


def owned_slots(block_table_row, seq_len, block_size, rank, cp_size, interleave):
    """Physical cache slot of every owned token: page = block_table_row[t // B], slot
    index page * B + t % B, in ascending t.  int64."""
    t = owned_tokens(seq_len, rank, cp_size, interleave)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // block_size]
    return pages * block_size + t % block_size


# ----------------------------------------------------------------------------------------
# Attention over an explicit token set  ([Blog] "DCP execution flow", step "Compute")
# ----------------------------------------------------------------------------------------

def attend(q, k, v, scale):
    """Softmax attention of one decode query over T tokens, with its log-sum-exp.

    q: [Hq, Dk]; k: [T, Hkv, Dk]; v: [T, Hkv, Dv]; query head h uses KV head
    h // (Hq // Hkv) (reading R6).  Returns (O [Hq, Dv], lse [Hq]) in float64, where
    lse_h = ln sum_t exp(s_ht), s_ht = scale * q_h . k_t (reading R3) and
    O_h = sum_t exp(s_ht - lse_h) v_t.  T = 0 gives O = 0, lse = -inf (reading R4)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq = q.shape[0]
    t_count, hkv = k.shape[0], k.shape[1]
    group = hq // hkv
    out = np.zeros((hq, v.shape[2]), dtype=np.float64)
    lse = np.full(hq, NEG_INF, dtype=np.float64)
    if t_count == 0:
        return out, lse
    for h in range(hq):
        g = h // group
        s = scale * (k[:, g, :] @ q[h])          # [T]
        mx = s.max()
        e = np.exp(s - mx)
        lse[h] = mx + math.log(e.sum())
        w = np.exp(s - lse[h])                    # softmax weights
        out[h] = w @ v[:, g, :]
    return out, lse


def attend_bruteforce(q, k, v, scale, dv=None):
    """The same definition as `attend` in scalar pure-Python loops (tiny inputs only).
    `dv` is needed only when there are no tokens to read the value width from."""
    hq, dk = len(q), len(q[0])
    t_count = len(k)
    hkv = len(k[0]) if t_count else 1
    dv = len(v[0][0]) if t_count else dv
    group = hq // hkv
    out, lse = [], []
    for h in range(hq):
        g = h // group
        scores = []
        for t in range(t_count):
            acc = 0.0
            for d in range(dk):
                acc += float(q[h][d]) * float(k[t][g][d])
            scores.append(scale * acc)
        if not scores:
            out.append([0.0] * dv)
            lse.append(NEG_INF)
            continue
        total = sum(math.exp(s) for s in scores)
        lse.append(math.log(total))
        row = []
        for d in range(dv):
            row.append(sum(math.exp(s) / total * float(v[t][g][d]) for t, s in enumerate(scores)))
        out.append(row)
    return out, lse


# ----------------------------------------------------------------------------------------
# Paged cache gathers (the data layouts the library uses)
#   GQA: k_pages, v_pages [num_blocks][Hkv][B][D]
#   MLA: latent_pages     [num_blocks][B][576]  (key = whole row, value = row[:512])
# ----------------------------------------------------------------------------------------

def _gqa_rows(pages, block_table_row, tokens, block_size):
    pg = np.asarray(block_table_row, dtype=np.int64)[tokens // block_size]
    sl = tokens % block_size
    # [T, Hkv, D]
    return np.asarray(pages)[pg, :, sl, :]


def _mla_rows(latent_pages, block_table_row, tokens, block_size):
    pg = np.asarray(block_table_row, dtype=np.int64)[tokens // block_size]
    sl = tokens % block_size
    return np.asarray(latent_pages)[pg, sl, :]   # [T, Dk]


def gqa_shard(q_b, k_pages, v_pages, block_table_row, seq_len, rank, cp_size, interleave,
              scale, block_size):
    """Partial (O_r, lse_r) of one request for DCP rank `rank`: attention of the gathered
    query over the tokens that rank stores ([Blog] "DCP execution flow", "Compute")."""
    t = owned_tokens(seq_len, rank, cp_size, interleave)
    k = _gqa_rows(k_pages, block_table_row, t, block_size)
    v = _gqa_rows(v_pages, block_table_row, t, block_size)
    return attend(q_b, k, v, scale)


def gqa_full(q_b, k_pages, v_pages, block_table_row, seq_len, scale, block_size):
    """Unsharded attention of one request over all tokens t < seq_len (reading R5)."""
    t = np.arange(int(seq_len), dtype=np.int64)
    k = _gqa_rows(k_pages, block_table_row, t, block_size)
    v = _gqa_rows(v_pages, block_table_row, t, block_size)
    return attend(q_b, k, v, scale)


MLA_DV = 512


def mla_shard(q_b, latent_pages, block_table_row, seq_len, rank, cp_size, interleave,
              scale, block_size, dv=MLA_DV):
    """MLA partial for one request: every query head reads the single shared latent row
    ([Blog] "The memory wall", MLA item; reading R7)."""
    t = owned_tokens(seq_len, rank, cp_size, interleave)
    rows = _mla_rows(latent_pages, block_table_row, t, block_size)
    return attend(q_b, rows[:, None, :], rows[:, None, :dv], scale)


def mla_full(q_b, latent_pages, block_table_row, seq_len, scale, block_size, dv=MLA_DV):
    t = np.arange(int(seq_len), dtype=np.int64)
    rows = _mla_rows(latent_pages, block_table_row, t, block_size)
    return attend(q_b, rows[:, None, :], rows[:, None, :dv], scale)


# ----------------------------------------------------------------------------------------
# Multi-token decode (reading R8; [Guide] "Overview", the speculative-decoding + DCP entry of
# the feature table; [Blog] "Roadmap")
# ----------------------------------------------------------------------------------------

def query_positions(seq_len, q_len):
    """Global position of each of the q_len query rows: seq_len - q_len + i."""
    return int(seq_len) - int(q_len) + np.arange(int(q_len), dtype=np.int64)


def _attend_rows(q_rows, tokens, keys, values, seq_len, scale):
    """Row i attends the listed tokens at positions <= its own (R8)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    pos = query_positions(seq_len, q_rows.shape[0])
    outs, lses = [], []
    for i in range(q_rows.shape[0]):
        sel = tokens <= pos[i]
        o, l = attend(q_rows[i], keys[sel], values[sel], scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def gqa_shard_mq(q_rows, k_pages, v_pages, block_table_row, seq_len, rank, cp_size,
                 interleave, scale, block_size):
    """Partial (O_r [q_len, Hq, Dv], lse_r [q_len, Hq]) of one request's q_len query rows
    ([q_len, Hq, D]) over the tokens `rank` stores, each row causally masked (R8)."""
    t = owned_tokens(seq_len, rank, cp_size, interleave)
    k = _gqa_rows(k_pages, block_table_row, t, block_size)
    v = _gqa_rows(v_pages, block_table_row, t, block_size)
    return _attend_rows(q_rows, t, k, v, seq_len, scale)


def gqa_full_mq(q_rows, k_pages, v_pages, block_table_row, seq_len, scale, block_size):
    """Unsharded multi-token attention: every row over all positions up to its own."""
    t = np.arange(int(seq_len), dtype=np.int64)
    k = _gqa_rows(k_pages, block_table_row, t, block_size)
    v = _gqa_rows(v_pages, block_table_row, t, block_size)
    return _attend_rows(q_rows, t, k, v, seq_len, scale)


def mla_shard_mq(q_rows, latent_pages, block_table_row, seq_len, rank, cp_size, interleave,
                 scale, block_size, dv=MLA_DV):
    """MLA partial of q_len query rows ([q_len, 128, 576]) over a rank's tokens (R7, R8)."""
    t = owned_tokens(seq_len, rank, cp_size, interleave)
    rows = _mla_rows(latent_pages, block_table_row, t, block_size)
    return _attend_rows(q_rows, t, rows[:, None, :], rows[:, None, :dv], seq_len, scale)


def mla_full_mq(q_rows, latent_pages, block_table_row, seq_len, scale, block_size, dv=MLA_DV):
    t = np.arange(int(seq_len), dtype=np.int64)
    rows = _mla_rows(latent_pages, block_table_row, t, block_size)
    return _attend_rows(q_rows, t, rows[:, None, :], rows[:, None, :dv], seq_len, scale)


# ----------------------------------------------------------------------------------------
# LSE merge  ([Blog] "DCP execution flow", step 3: partial outputs and LSE values are
# combined with the online-softmax trick)
# ----------------------------------------------------------------------------------------

# ----------------------------------------------------------------------------------------
# fp8 KV cache (reading R9): the values an fp8 cache represents, then the plain definitions
# ----------------------------------------------------------------------------------------

def fp8_e4m3_decode(codes):
    """Exact float64 values of OCP FP8 E4M3 codes (uint8): (-1)^s * (1 + m/8) * 2^(e-7) for
    exponent e in 1..15, (-1)^s * (m/8) * 2^-6 for e = 0, NaN for the code S.1111.111."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp8_kv_values(codes, kv_scale):
    """The cache values an fp8 page array stands for: decode(code) * scale (reading R9)."""
    return fp8_e4m3_decode(codes) * float(kv_scale)


def merge(o_parts, lse_parts):
    """Combine C partials into the attention over the union of their token sets.

    o_parts: [C, ..., Dv]; lse_parts: [C, ...].  With m = max_r lse_r over finite
    entries, w_r = exp(lse_r - m) (exactly 0 where lse_r = -inf, whatever O_r holds):
    lse = m + ln sum_r w_r and O = sum_r w_r O_r / sum_r w_r.  Where every partial is
    empty: O = 0, lse = -inf (reading R4)."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    finite = np.isfinite(lse_parts)
    m = np.where(finite, lse_parts, NEG_INF).max(axis=0)
    any_finite = finite.any(axis=0)
    m_safe = np.where(any_finite, m, 0.0)
    w = np.where(finite, np.exp(np.where(finite, lse_parts, 0.0) - m_safe), 0.0)
    wsum = w.sum(axis=0)
    lse = np.where(any_finite, m_safe + np.log(np.where(any_finite, wsum, 1.0)), NEG_INF)
    o_clean = np.where(finite[..., None], o_parts, 0.0)
    num = (w[..., None] * o_clean).sum(axis=0)
    out = np.where(any_finite[..., None], num / np.where(any_finite, wsum, 1.0)[..., None],
                   0.0)
    return out, lse


# ----------------------------------------------------------------------------------------
# DCP size constraints  ([Guide] "Decode Context Parallel -> Constraints";
# [Blog] "MLA backend", "GQA backend")
# ----------------------------------------------------------------------------------------

def check_parallel(tp, dcp, num_kv_heads, is_mla):
    """True when a DCP size is allowed.  MLA has a single latent KV head, so DCP may split
    the sequence up to the full TP degree: dcp must divide tp.  GQA: TP first splits the
    KV heads; DCP then splits the tp // num_kv_heads redundant copies, so dcp must divide
    that count."""
    if tp < 1 or dcp < 1:
        return False
    copies = tp if is_mla else tp // num_kv_heads
    return copies >= dcp and copies % dcp == 0

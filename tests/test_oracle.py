"""Pins for the CPU oracle, against facts that do not come from the oracle itself.

Each pin is a library routine, a closed form, a page's printed example, brute force on
tiny inputs or an algebraic identity.  The mutation tests at the end plant plausible
mistakes in the oracle (on the CPU) and check that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import dcp_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ ownership / walk pins

def pin_blog_example():
    g = _golden("blog_200k_4gpu_split.json")
    for r, (lo, hi) in enumerate(g["rank_ranges"]):
        t = orc.owned_tokens(g["seq_len"], r, g["cp_size"], g["interleave"])
        assert t.size == hi - lo
        assert t[0] == lo and t[-1] == hi - 1
        assert np.array_equal(t, np.arange(lo, hi))


def pin_partition(seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        L = int(rng.integers(0, 3000))
        C = int(rng.integers(1, 9))
        I = int(rng.choice([1, 2, 3, 7, 16, 64, 128, max(1, L)]))
        seen = np.zeros(L, dtype=np.int64)
        for r in range(C):
            t = orc.owned_tokens(L, r, C, I)
            assert np.all(np.diff(t) > 0)
            seen[t] += 1
            # closed form of the count: whole rounds of C chunks plus this rank's share
            # of the last, partial round
            full, rem = divmod(L, I * C)
            assert t.size == full * I + min(max(rem - r * I, 0), I)
            # each owned token's chunk index is congruent to r mod C, and every run of
            # consecutive owned tokens is a whole chunk except possibly the last one
            assert np.all((t // I) % C == r)
        assert np.all(seen == 1)


def pin_slots_hand_example():
    # B = 2, interleave 1, two ranks, logical pages [0, 1] on physical pages [5, 3]:
    # tokens 0..3 sit in slots 10, 11, 6, 7; rank 0 holds tokens 0, 2; rank 1 holds 1, 3.
    bt = np.array([5, 3, -1])
    assert orc.owned_slots(bt, 4, 2, 0, 2, 1).tolist() == [10, 6]
    assert orc.owned_slots(bt, 4, 2, 1, 2, 1).tolist() == [11, 7]
    # interleave 2 on the same table: rank 0 holds tokens 0, 1; rank 1 holds 2, 3.
    assert orc.owned_slots(bt, 4, 2, 0, 2, 2).tolist() == [10, 11]
    assert orc.owned_slots(bt, 3, 2, 1, 2, 2).tolist() == [6]


def test_blog_example():
    pin_blog_example()


def test_partition_and_count_closed_form():
    pin_partition()


def test_slots_hand_example():
    pin_slots_hand_example()


def test_slots_permuted_table():
    rng = np.random.default_rng(3)
    B, L = 16, 1000
    npages = (L + B - 1) // B
    bt = rng.permutation(npages + 5)[:npages]
    for C, I in [(1, 16), (2, 16), (3, 5), (4, 64)]:
        allslots = []
        for r in range(C):
            s = orc.owned_slots(bt, L, B, r, C, I)
            t = orc.owned_tokens(L, r, C, I)
            assert np.array_equal(s // B, bt[t // B])
            assert np.array_equal(s % B, t % B)
            allslots.append(s)
        allslots = np.concatenate(allslots)
        assert np.unique(allslots).size == L


# ------------------------------------------------------------------ attention pins

def _torch_flash_cpu(q, k, v, scale):
    """Library routine: torch's CPU flash attention in float64, which also returns lse.
    q [Hq, D], k [T, Hkv, Dk], v [T, Hkv, Dv]; GQA via repeat_interleave of KV heads."""
    hq, hkv = q.shape[0], k.shape[1]
    rep = hq // hkv
    dk, dv = q.shape[1], v.shape[2]
    # the routine wants one head size: zero columns change neither scores nor outputs
    if dv < dk:
        v = np.concatenate([v, np.zeros(v.shape[:2] + (dk - dv,))], axis=2)
    elif dk < dv:
        q = np.concatenate([q, np.zeros((hq, dv - dk))], axis=1)
        k = np.concatenate([k, np.zeros(k.shape[:2] + (dv - dk,))], axis=2)
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).permute(1, 0, 2)
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).permute(1, 0, 2)
    kt = kt.repeat_interleave(rep, dim=0)[None].contiguous()
    vt = vt.repeat_interleave(rep, dim=0)[None].contiguous()
    o, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        qt, kt, vt, 0.0, False, scale=scale)
    return o[0, :, 0, :dv].numpy(), lse[0, :, 0].numpy()


def pin_attend_library(seed=1):
    rng = np.random.default_rng(seed)
    for hq, hkv, dk, dv, T in [(8, 2, 64, 64, 300), (8, 1, 128, 128, 77), (4, 4, 16, 8, 5),
                               (16, 1, 40, 24, 129)]:
        q = rng.standard_normal((hq, dk))
        k = rng.standard_normal((T, hkv, dk))
        v = rng.standard_normal((T, hkv, dv))
        scale = 1.0 / math.sqrt(dk)
        o, lse = orc.attend(q, k, v, scale)
        o_ref, lse_ref = _torch_flash_cpu(q, k, v, scale)
        np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
        # GQA grouping also against SDPA's own grouped-query path
        if dk == dv:
            sd = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q)[None, :, None, :],
                torch.from_numpy(k).permute(1, 0, 2)[None].contiguous(),
                torch.from_numpy(v).permute(1, 0, 2)[None].contiguous(),
                scale=scale, enable_gqa=True)
            np.testing.assert_allclose(o, sd[0, :, 0, :].numpy(), rtol=1e-10, atol=1e-12)


def pin_lse_scipy(seed=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((2, 32))
    k = rng.standard_normal((50, 1, 32))
    v = rng.standard_normal((50, 1, 32))
    _, lse = orc.attend(q, k, v, 0.3)
    for h in range(2):
        scores = 0.3 * np.einsum("td,d->t", k[:, 0, :], q[h])
        assert abs(lse[h] - scipy.special.logsumexp(scores)) < 1e-12


def pin_bruteforce(seed=4):
    rng = np.random.default_rng(seed)
    for hq, hkv, d, T in [(4, 2, 8, 13), (2, 1, 3, 1), (3, 3, 5, 64), (4, 1, 6, 0)]:
        q = rng.standard_normal((hq, d))
        k = rng.standard_normal((T, hkv, d))
        v = rng.standard_normal((T, hkv, d))
        o, lse = orc.attend(q, k, v, 0.7)
        ob, lb = orc.attend_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.7, dv=d)
        np.testing.assert_allclose(o, np.asarray(ob).reshape(o.shape), rtol=1e-12,
                                   atol=1e-13)
        np.testing.assert_allclose(lse, np.asarray(lb, dtype=np.float64), rtol=1e-12)


def pin_closed_forms(seed=5):
    rng = np.random.default_rng(seed)
    T, d = 37, 16
    k = rng.standard_normal((T, 1, d))
    v = rng.standard_normal((T, 1, d))
    # q = 0: every score is 0, so lse = ln T and O is the mean value row
    o, lse = orc.attend(np.zeros((2, d)), k, v, 0.25)
    np.testing.assert_allclose(lse, math.log(T), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0], v[:, 0, :].mean(axis=0), atol=1e-13)
    # one token: the weight is 1, O = v, lse = its score
    q = rng.standard_normal((1, d))
    o, lse = orc.attend(q, k[:1], v[:1], 0.25)
    np.testing.assert_allclose(o[0], v[0, 0], atol=1e-14)
    assert abs(lse[0] - 0.25 * float(q[0] @ k[0, 0])) < 1e-13
    # identical keys: uniform weights
    kk = np.repeat(k[:1], T, axis=0)
    o, lse = orc.attend(q, kk, v, 0.25)
    np.testing.assert_allclose(o[0], v[:, 0, :].mean(axis=0), atol=1e-13)
    np.testing.assert_allclose(lse[0], 0.25 * float(q[0] @ k[0, 0]) + math.log(T), atol=1e-12)
    # shifting every score by c (an extra dimension where q holds c/scale and every key
    # holds 1) shifts lse by c and leaves O unchanged
    c, scale = 3.5, 0.25
    o0, l0 = orc.attend(q, k, v, scale)
    q1 = np.concatenate([q, [[c / scale]]], axis=1)
    k1 = np.concatenate([k, np.ones((T, 1, 1))], axis=2)
    o1, l1 = orc.attend(q1, k1, v, scale)
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    np.testing.assert_allclose(l1, l0 + c, atol=1e-12)


def pin_large_scores(seed=6):
    rng = np.random.default_rng(seed)
    q = 30 * rng.standard_normal((4, 64))
    k = rng.standard_normal((200, 2, 64))
    v = rng.standard_normal((200, 2, 64))
    o, lse = orc.attend(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o_ref, lse_ref = _torch_flash_cpu(q, k, v, 1.0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)


def test_attend_matches_torch_library():
    pin_attend_library()


def test_lse_matches_scipy():
    pin_lse_scipy()


def test_bruteforce_agrees():
    pin_bruteforce()


def test_closed_forms():
    pin_closed_forms()


def test_large_scores():
    pin_large_scores()


# ------------------------------------------------------------------ paged shards + merge

def _paged_gqa(rng, L, B, hkv, d):
    npages = max(1, (L + B - 1) // B)
    nb = npages + 3
    kp = rng.standard_normal((nb, hkv, B, d))
    vp = rng.standard_normal((nb, hkv, B, d))
    bt = rng.permutation(nb)[:npages]
    return kp, vp, bt


def pin_merge_equals_full(seed=7):
    rng = np.random.default_rng(seed)
    for trial in range(24):
        L = int(rng.integers(1, 700))
        B = int(rng.choice([1, 4, 16]))
        C = int(rng.integers(1, 9))
        I = int(rng.choice([1, 3, 16, 64, L]))
        hq, hkv, d = 8, 2, 16
        kp, vp, bt = _paged_gqa(rng, L, B, hkv, d)
        q = rng.standard_normal((hq, d))
        parts = [orc.gqa_shard(q, kp, vp, bt, L, r, C, I, 0.25, B) for r in range(C)]
        o, lse = orc.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        o_f, lse_f = orc.gqa_full(q, kp, vp, bt, L, 0.25, B)
        np.testing.assert_allclose(o, o_f, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, lse_f, rtol=1e-12, atol=1e-12)


def pin_mla_merge_equals_full(seed=8):
    rng = np.random.default_rng(seed)
    B, L, dk, dv = 8, 150, 24, 16
    npages = (L + B - 1) // B
    lat = rng.standard_normal((npages + 2, B, dk))
    bt = rng.permutation(npages + 2)[:npages]
    q = rng.standard_normal((4, dk))
    for C, I in [(1, 8), (3, 8), (4, 5), (8, 1)]:
        parts = [orc.mla_shard(q, lat, bt, L, r, C, I, 0.2, B, dv=dv) for r in range(C)]
        o, lse = orc.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        o_f, lse_f = orc.mla_full(q, lat, bt, L, 0.2, B, dv=dv)
        np.testing.assert_allclose(o, o_f, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, lse_f, rtol=1e-12)
    # value = first dv latent columns: with q = 0 the output is their mean row
    o, _ = orc.mla_full(np.zeros((2, dk)), lat, bt, L, 0.2, B, dv=dv)
    rows = lat[bt[np.arange(L) // B], np.arange(L) % B]
    np.testing.assert_allclose(o[1], rows[:, :dv].mean(axis=0), atol=1e-13)
    # and against the library with key = latent row, value = its prefix
    q = rng.standard_normal((4, dk))
    o, lse = orc.mla_full(q, lat, bt, L, 0.2, B, dv=dv)
    o_ref, lse_ref = _torch_flash_cpu(q, rows[:, None, :], rows[:, None, :dv], 0.2)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)


def pin_merge_properties(seed=9):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((3, 5, 7))
    lse = rng.standard_normal((3, 5)) * 4
    # one partial: the identity, exactly
    o1, l1 = orc.merge(o[:1], lse[:1])
    assert np.array_equal(o1, o[0]) and np.array_equal(l1, lse[0])
    # associativity
    oab, lab = orc.merge(o[:2], lse[:2])
    o3, l3 = orc.merge(np.stack([oab, o[2]]), np.stack([lab, lse[2]]))
    oall, lall = orc.merge(o, lse)
    np.testing.assert_allclose(o3, oall, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l3, lall, rtol=1e-12, atol=1e-14)
    # lse of the merge is the log of the summed exponentials (library routine)
    np.testing.assert_allclose(lall, scipy.special.logsumexp(lse, axis=0), rtol=1e-13)
    # an empty partial (lse = -inf) carrying NaN garbage changes nothing
    o_p = np.concatenate([o, np.full((1, 5, 7), np.nan)])
    l_p = np.concatenate([lse, np.full((1, 5), -np.inf)])
    op, lp = orc.merge(o_p, l_p)
    np.testing.assert_allclose(op, oall, rtol=1e-13)
    np.testing.assert_allclose(lp, lall, rtol=1e-13)
    # every partial empty: O = 0, lse = -inf, no NaN
    oe, le = orc.merge(np.full((2, 5, 7), np.nan), np.full((2, 5), -np.inf))
    assert np.all(oe == 0) and np.all(le == -np.inf)
    # huge lse values do not overflow
    oh, lh = orc.merge(o, lse + 1000.0)
    np.testing.assert_allclose(oh, oall, rtol=1e-12)
    np.testing.assert_allclose(lh, lall + 1000.0, rtol=1e-13)


def pin_empty_shard():
    rng = np.random.default_rng(10)
    kp, vp, bt = _paged_gqa(rng, 5, 4, 1, 8)
    q = rng.standard_normal((2, 8))
    # L = 5, C = 4, I = 2: rank 3 owns chunk 3 = tokens 6, 7, beyond L -> empty
    o, lse = orc.gqa_shard(q, kp, vp, bt, 5, 3, 4, 2, 0.5, 4)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    o, lse = orc.gqa_full(q, kp, vp, bt, 0, 0.5, 4)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def pin_cp1_identity(seed=11):
    rng = np.random.default_rng(seed)
    kp, vp, bt = _paged_gqa(rng, 333, 16, 2, 16)
    q = rng.standard_normal((4, 16))
    o_s, l_s = orc.gqa_shard(q, kp, vp, bt, 333, 0, 1, 16, 0.3, 16)
    o_f, l_f = orc.gqa_full(q, kp, vp, bt, 333, 0.3, 16)
    assert np.array_equal(o_s, o_f) and np.array_equal(l_s, l_f)
    o_m, l_m = orc.merge(o_s[None], l_s[None])
    assert np.array_equal(o_m, o_f) and np.array_equal(l_m, l_f)


def test_merge_equals_full_gqa():
    pin_merge_equals_full()


def test_merge_equals_full_mla():
    pin_mla_merge_equals_full()


def test_merge_properties():
    pin_merge_properties()


def test_empty_shard():
    pin_empty_shard()


def test_cp1_identity():
    pin_cp1_identity()


def test_check_parallel_page_examples():
    for case in _golden("dcp_size_examples.json")["cases"]:
        got = orc.check_parallel(case["tp"], case["dcp"], case["num_kv_heads"], case["is_mla"])
        assert got == case["ok"], case["why"]


# ------------------------------------------------------------------ planted mistakes

ALL_PINS = [pin_blog_example, pin_partition, pin_slots_hand_example, pin_attend_library,
            pin_lse_scipy, pin_bruteforce, pin_closed_forms, pin_large_scores,
            pin_merge_equals_full, pin_mla_merge_equals_full, pin_merge_properties,
            pin_empty_shard, pin_cp1_identity]


def _some_pin_fails():
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            return True
    return False


def _mut_owner_mod_first(t, cp_size, interleave):
    return (np.asarray(t) % cp_size) // max(1, interleave // cp_size)


def _mut_owner_off_by_one(t, cp_size, interleave):
    return ((np.asarray(t) + 1) // interleave) % cp_size


def _mut_attend_no_scale(q, k, v, scale):
    return _orig_attend(q, k, v, 1.0)


def _mut_attend_log2(q, k, v, scale):
    o, lse = _orig_attend(q, k, v, scale)
    return o, lse / math.log(2.0)


def _mut_attend_gqa_modulo(q, k, v, scale):
    hq, hkv = q.shape[0], k.shape[1]
    if hkv == 1 or hq == hkv:
        return _orig_attend(q, k, v, scale)
    perm = [h % hkv for h in range(hq)]
    kk = np.asarray(k)[:, perm, :]
    vv = np.asarray(v)[:, perm, :]
    return _orig_attend(q, kk, vv, scale)


def _mut_attend_no_max(q, k, v, scale):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, hkv = q.shape[0], k.shape[1]
    g = hq // hkv
    out = np.zeros((hq, v.shape[2]))
    lse = np.full(hq, -np.inf)
    if k.shape[0] == 0:
        return out, lse
    for h in range(hq):
        s = scale * (k[:, h // g, :] @ q[h])
        e = np.exp(s)
        lse[h] = math.log(e.sum())
        out[h] = (e / e.sum()) @ v[:, h // g, :]
    return out, lse


def _mut_merge_plain_mean(o_parts, lse_parts):
    o, lse = _orig_merge(o_parts, lse_parts)
    op = np.asarray(o_parts, dtype=np.float64)
    return np.nan_to_num(op).mean(axis=0), lse


def _mut_merge_no_max(o_parts, lse_parts):
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    w = np.exp(lse_parts)
    ws = w.sum(axis=0)
    return (w[..., None] * np.nan_to_num(o_parts)).sum(axis=0) / ws[..., None], np.log(ws)


def _mut_slots_wrong_page(block_table_row, seq_len, block_size, rank, cp_size, interleave):
    t = orc.owned_tokens(seq_len, rank, cp_size, interleave)
    return np.asarray(block_table_row, dtype=np.int64)[t // block_size] + t % block_size


_orig_attend = orc.attend
_orig_merge = orc.merge

MUTANTS = [
    ("owner_of", _mut_owner_mod_first),
    ("owner_of", _mut_owner_off_by_one),
    ("attend", _mut_attend_no_scale),
    ("attend", _mut_attend_log2),
    ("attend", _mut_attend_gqa_modulo),
    ("attend", _mut_attend_no_max),
    ("merge", _mut_merge_plain_mean),
    ("merge", _mut_merge_no_max),
    ("owned_slots", _mut_slots_wrong_page),
]


@pytest.mark.parametrize("attr,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, attr, mutant):
    assert not _some_pin_fails(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(orc, attr, mutant)
    assert _some_pin_fails(), f"no pin caught the planted mistake {mutant.__name__}"

"""Pins for the oracle's multi-token decode (q_len query rows per request, causally masked
among themselves): a library routine with its own lower-right causal mask, closed forms,
brute force, the q_len = 1 reduction to plain decode and merge(shards) = full.  The tests
at the end plant plausible mistakes in the multi-token code (on the CPU) and check that
some pin catches each one.
"""
import math

import numpy as np
import pytest
import torch
from torch.nn.attention.bias import causal_lower_right

from oracle import dcp_oracle as orc


def _paged(rng, L, B, hkv, d):
    npages = max(1, (L + B - 1) // B)
    nb = npages + 2
    kp = rng.standard_normal((nb, hkv, B, d))
    vp = rng.standard_normal((nb, hkv, B, d))
    bt = rng.permutation(nb)[:npages]
    return kp, vp, bt


def _flat(pages, bt, L, B):
    """Rows of positions 0 .. L-1 of a paged GQA cache: [T, Hkv, D]."""
    t = np.arange(L)
    return pages[bt[t // B], :, t % B, :]


def pin_mq_library(seed=41):
    """torch's scaled_dot_product_attention in float64 with the library's own lower-right
    causal bias (query rows aligned to the end of the key sequence)."""
    rng = np.random.default_rng(seed)
    for hq, hkv, d, L, nq, B in [(8, 2, 16, 40, 3, 4), (8, 1, 32, 129, 4, 16),
                                 (4, 4, 8, 5, 2, 2), (16, 1, 8, 4, 4, 1), (2, 1, 8, 9, 1, 4)]:
        kp, vp, bt = _paged(rng, L, B, hkv, d)
        q = rng.standard_normal((nq, hq, d))
        o, lse = orc.gqa_full_mq(q, kp, vp, bt, L, 0.3, B)
        k, v = _flat(kp, bt, L, B), _flat(vp, bt, L, B)
        qt = torch.from_numpy(q).permute(1, 0, 2)[None].contiguous()        # [1, Hq, nq, d]
        kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()        # [1, Hkv, L, d]
        vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
        mask = causal_lower_right(nq, L)._materialize()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=0.3, enable_gqa=True)[0].permute(1, 0, 2)
        np.testing.assert_allclose(o, ref.numpy(), rtol=1e-10, atol=1e-12)
        # lse row by row: scipy-free, log of the summed exponentials of the visible scores
        # as the library's masked softmax denominators see them
        kk = np.repeat(k, hq // hkv, axis=1)                                # [L, Hq, d]
        s = 0.3 * np.einsum("ihd,thd->iht", q, kk)
        s = np.where(mask.numpy()[:, None, :], s, -np.inf)
        ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def pin_mq_mla_library(seed=42):
    rng = np.random.default_rng(seed)
    B, L, dk, dv, nq = 8, 70, 24, 16, 3
    npages = (L + B - 1) // B
    lat = rng.standard_normal((npages + 1, B, dk))
    bt = rng.permutation(npages + 1)[:npages]
    q = rng.standard_normal((nq, 4, dk))
    o, _ = orc.mla_full_mq(q, lat, bt, L, 0.2, B, dv=dv)
    rows = lat[bt[np.arange(L) // B], np.arange(L) % B]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None].contiguous()
    kt = torch.from_numpy(rows)[None, None].expand(1, 4, L, dk).contiguous()
    vt = torch.from_numpy(rows[:, :dv])[None, None].expand(1, 4, L, dv).contiguous()
    mask = causal_lower_right(nq, L)._materialize()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                           scale=0.2)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def pin_mq_closed_forms(seed=43):
    """q = 0: row i of a rank's partial weighs its visible owned tokens uniformly, so
    lse = ln(count) with count from the walker's closed form on the prefix length
    L - q_len + 1 + i, and O is their mean value row; a row with none is empty."""
    rng = np.random.default_rng(seed)
    for L, nq, C, I, B in [(50, 4, 3, 4, 4), (3, 4, 2, 1, 2), (129, 2, 4, 16, 16),
                           (64, 3, 2, 32, 8)]:
        kp, vp, bt = _paged(rng, L, B, 1, 6)
        v = _flat(vp, bt, L, B)[:, 0, :]
        for r in range(C):
            o, lse = orc.gqa_shard_mq(np.zeros((nq, 2, 6)), kp, vp, bt, L, r, C, I, 0.5, B)
            for i in range(nq):
                Li = L - nq + 1 + i
                full, rem = divmod(max(Li, 0), I * C)
                n = full * I + min(max(rem - r * I, 0), I)
                if n == 0:
                    assert np.all(o[i] == 0) and np.all(lse[i] == -np.inf), (L, nq, r, i)
                    continue
                np.testing.assert_allclose(lse[i], math.log(n), atol=1e-13)
                mine = [t for t in range(max(Li, 0)) if (t // I) % C == r]
                np.testing.assert_allclose(o[i, 1], v[mine].mean(axis=0), atol=1e-13)


def pin_mq_bruteforce(seed=44):
    """Row i against brute force over the positions 0 .. L - q_len + i, in scalar loops."""
    rng = np.random.default_rng(seed)
    L, nq, B, hq, hkv, d = 11, 3, 4, 4, 2, 5
    kp, vp, bt = _paged(rng, L, B, hkv, d)
    q = rng.standard_normal((nq, hq, d))
    o, lse = orc.gqa_full_mq(q, kp, vp, bt, L, 0.6, B)
    k, v = _flat(kp, bt, L, B), _flat(vp, bt, L, B)
    for i in range(nq):
        last = L - nq + i
        ob, lb = orc.attend_bruteforce(q[i].tolist(), k[:last + 1].tolist(),
                                       v[:last + 1].tolist(), 0.6)
        np.testing.assert_allclose(o[i], np.asarray(ob), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[i], np.asarray(lb), rtol=1e-12)


def pin_mq_single_row_is_decode(seed=45):
    """q_len = 1 is plain decode: the one row attends every position."""
    rng = np.random.default_rng(seed)
    kp, vp, bt = _paged(rng, 77, 8, 2, 8)
    q = rng.standard_normal((4, 8))
    for r in range(3):
        o1, l1 = orc.gqa_shard_mq(q[None], kp, vp, bt, 77, r, 3, 5, 0.4, 8)
        o0, l0 = orc.gqa_shard(q, kp, vp, bt, 77, r, 3, 5, 0.4, 8)
        assert np.array_equal(o1[0], o0) and np.array_equal(l1[0], l0)


def pin_mq_merge_equals_full(seed=46):
    rng = np.random.default_rng(seed)
    for _ in range(16):
        L = int(rng.integers(1, 300))
        nq = int(rng.integers(1, 5))
        B = int(rng.choice([1, 4, 16]))
        C = int(rng.integers(1, 9))
        I = int(rng.choice([1, 3, 16, 64]))
        kp, vp, bt = _paged(rng, L, B, 2, 8)
        q = rng.standard_normal((nq, 4, 8))
        parts = [orc.gqa_shard_mq(q, kp, vp, bt, L, r, C, I, 0.3, B) for r in range(C)]
        o, lse = orc.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        o_f, l_f = orc.gqa_full_mq(q, kp, vp, bt, L, 0.3, B)
        np.testing.assert_allclose(o, o_f, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, l_f, rtol=1e-12, atol=1e-12)


MQ_PINS = [pin_mq_library, pin_mq_mla_library, pin_mq_closed_forms, pin_mq_bruteforce,
           pin_mq_single_row_is_decode, pin_mq_merge_equals_full]


@pytest.mark.parametrize("pin", MQ_PINS, ids=[p.__name__ for p in MQ_PINS])
def test_mq_pin(pin):
    pin()


def _some_pin_fails():
    for pin in MQ_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            return True
    return False


_orig_rows = orc._attend_rows


def _mut_mask_strict(q_rows, tokens, keys, values, seq_len, scale):
    """Off by one: a row does not see its own position."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    pos = orc.query_positions(seq_len, q_rows.shape[0])
    res = [orc.attend(q_rows[i], keys[tokens < pos[i]], values[tokens < pos[i]], scale)
           for i in range(q_rows.shape[0])]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def _mut_no_mask(q_rows, tokens, keys, values, seq_len, scale):
    """Every row sees every token."""
    return _orig_rows(q_rows, tokens, keys, values, seq_len + len(q_rows), scale)


def _mut_top_left(seq_len, q_len):
    """Causal mask aligned to the start of the sequence (row i sees positions <= i)."""
    return np.arange(int(q_len), dtype=np.int64)


def _mut_reversed(seq_len, q_len):
    """Rows in the opposite order."""
    return (int(seq_len) - 1 - np.arange(int(q_len), dtype=np.int64))


MQ_MUTANTS = [("_attend_rows", _mut_mask_strict), ("_attend_rows", _mut_no_mask),
              ("query_positions", _mut_top_left), ("query_positions", _mut_reversed)]


@pytest.mark.parametrize("attr,mutant", MQ_MUTANTS, ids=[m.__name__ for _, m in MQ_MUTANTS])
def test_mq_planted_mistake_is_caught(monkeypatch, attr, mutant):
    assert not _some_pin_fails(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(orc, attr, mutant)
    assert _some_pin_fails(), f"no pin caught the planted mistake {mutant.__name__}"

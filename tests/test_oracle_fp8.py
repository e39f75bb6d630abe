"""Pins of the oracle's fp8 KV cache reading (R9 in the oracle's header; CPU).

The decoder follows the OCP FP8 E4M3 definition; it is pinned by torch's float8_e4m3fn
conversion of every code (a library routine), by closed-form values of the format
(largest normal 448, smallest subnormal 2^-9, smallest normal 2^-6, 1, -1, NaN), and by
planted mistakes (exponent bias 8, subnormals read as normals, an ignored sign).  Cache
scales act as the definition says: K scaled by c equals attention with its score scale
multiplied by c; V scaled by c scales O by c and leaves lse unchanged.
"""
import math

import numpy as np
import pytest
import torch

from oracle import dcp_oracle as orc

ALL = np.arange(256, dtype=np.uint8)


def _check_decoder():
    got = orc.fp8_e4m3_decode(ALL)
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.all(both_nan | (got == ref))
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x07] == 7 * 2.0 ** -9
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x00] == 0.0
    assert math.isnan(got[0x7F]) and math.isnan(got[0xFF])
    assert np.count_nonzero(np.isnan(got)) == 2
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_decoder_matches_format():
    _check_decoder()


@pytest.mark.parametrize("mutant", ["bias8", "subnormal_as_normal", "no_sign"])
def test_decoder_planted_mistake_is_caught(monkeypatch, mutant):
    real = orc.fp8_e4m3_decode

    def bad(codes):
        c = np.asarray(codes).astype(np.int64)
        v = real(codes)
        if mutant == "bias8":
            return v / 2.0
        if mutant == "subnormal_as_normal":
            e, m = (c >> 3) & 0xF, (c & 7).astype(np.float64)
            sub = np.where(c & 0x80, -1.0, 1.0) * (1 + m / 8) * 2.0 ** -7
            return np.where((e == 0) & (m > 0), sub, v)
        return np.abs(v)

    monkeypatch.setattr(orc, "fp8_e4m3_decode", bad)
    with pytest.raises(AssertionError):
        _check_decoder()


def test_scales_act_as_defined():
    rng = np.random.default_rng(91)
    L, B, G, D = 70, 16, 4, 16
    pages = (L + B - 1) // B
    kc = rng.integers(0, 256, size=(pages, 1, B, D), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(pages, 1, B, D), dtype=np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38   # no NaN codes in a cache
    vc[(vc & 0x7F) == 0x7F] = 0x38
    q = rng.standard_normal((G, D))
    row = np.arange(pages)
    k1, v1 = orc.fp8_kv_values(kc, 1.0), orc.fp8_kv_values(vc, 1.0)
    o1, l1 = orc.gqa_full(q, k1 * 0.01, v1, row, L, 0.25, B)
    # K scale c == score scale times c
    o2, l2 = orc.gqa_full(q, orc.fp8_kv_values(kc, 0.02), v1, row, L, 0.125, B)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)
    # V scale c scales O, not lse
    o3, l3 = orc.gqa_full(q, k1 * 0.01, orc.fp8_kv_values(vc, 3.0), row, L, 0.25, B)
    np.testing.assert_allclose(o3, 3.0 * o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l3, l1, rtol=1e-12, atol=1e-12)

"""The parity gates themselves, on the CPU: at the GQA share's shard size (16384 local
tokens, 8 query heads on one KV head, head dim 128, bf16 values) the relative-L2 row gate
must pass the error the kernels' bf16 rounding of P makes and must fail an output that
lost 1/8 of every tile's tokens, which the elementwise gate alone lets through (there |O|
is about 0.01-0.04 against its 2e-2 absolute term).  The mistakes are planted in oracle
results here; nothing runs on a GPU."""
import numpy as np
import pytest
import torch

from oracle import dcp_oracle as orc
from parity_helpers import REL_L2_BF16, TOL_BF16_O, assert_close, assert_rel_l2, row_errors

T, HQ, D = 16384, 8, 128


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def request_data():
    rng = np.random.default_rng(2024)
    q = _bf16(rng.standard_normal((HQ, D)))
    k = _bf16(rng.standard_normal((T, 1, D)))
    v = _bf16(rng.standard_normal((T, 1, D)))
    return q, k, v, 1.0 / np.sqrt(D)


def _p_rounded(q, k, v, scale):
    """Attention with the unnormalised weights exp(s - max) rounded to bf16 before P.V (the
    normaliser summed from the unrounded weights), as the matrix-core kernels compute it."""
    s = scale * (k[:, 0, :] @ q.T)                   # [T, HQ]
    w = np.exp(s - s.max(axis=0))
    return (_bf16(w).T @ v[:, 0, :]) / w.sum(axis=0)[:, None]


def test_gate_passes_bf16_p_rounding(request_data):
    q, k, v, scale = request_data
    o_ref, _ = orc.attend(q, k, v, scale)
    o = _p_rounded(q, k, v, scale)
    assert_close(o, o_ref, TOL_BF16_O, "bf16 P")
    assert_rel_l2(o, o_ref, REL_L2_BF16, "bf16 P")
    _, rl2 = row_errors(o, o_ref)
    assert rl2.max() < REL_L2_BF16 / 2


def test_gate_catches_dropped_tokens(request_data):
    q, k, v, scale = request_data
    o_ref, _ = orc.attend(q, k, v, scale)
    keep = (np.arange(T) % 64) < 56                 # 8 of every 64-token tile lost
    o_bad, _ = orc.attend(q, k[keep], v[keep], scale)
    assert_close(o_bad, o_ref, TOL_BF16_O, "dropped tokens, elementwise gate only")
    with pytest.raises(AssertionError, match="relative L2"):
        assert_rel_l2(o_bad, o_ref, REL_L2_BF16, "dropped tokens")
    _, rl2 = row_errors(o_bad, o_ref)
    assert rl2.min() > 0.2


def test_gate_catches_doubled_tile(request_data):
    """One 64-token tile counted twice (a split-combine or table-rebuild slip)."""
    q, k, v, scale = request_data
    o_ref, _ = orc.attend(q, k, v, scale)
    idx = np.concatenate([np.arange(T), np.arange(4096, 4160)])
    o_bad, _ = orc.attend(q, k[idx], v[idx], scale)
    with pytest.raises(AssertionError, match="relative L2"):
        assert_rel_l2(o_bad, o_ref, REL_L2_BF16, "doubled tile")

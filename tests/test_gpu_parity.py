"""Parity of the HIP shard kernels + LSE merge against the CPU oracle (GPU).

Small cases (the oracle checks every request, every rank, every head) cover several tiles,
ragged tails, one-token and empty shards, interleave sizes below, equal to, above and not
a multiple of the block size, every supported GQA group size and both dtypes.  The
full-size cases run the five workloads at their real shapes, in the launch configuration
the benchmark times, and check sampled requests exhaustively.
Tolerances: see tests/parity_helpers.py (2e-2 for bf16-input outputs, 1e-3 for fp32-input
outputs and every LSE, exact -inf for empty shards).
"""
import numpy as np
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from parity_helpers import check_requests, run_shards, scale_of

pytestmark = pytest.mark.gpu


def _run_and_check(w, requests=None, label=None, q_scale=None):
    torch.cuda.synchronize()
    print(f"[parity] {label or w.name}: batch={w.batch} C={w.cp_size} I={w.interleave} "
          f"B={w.block_size} q_scale={q_scale}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    if q_scale is not None:
        # the oracle reads the same (rescaled, re-rounded) query back from the device
        inp["q"] = (inp["q"].float() * q_scale).to(inp["q"].dtype)
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    o_parts, l_parts = run_shards(inp, kind, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    if requests is None:
        requests = range(w.batch)
    check_requests(inp, kind, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   list(requests), label or w.name)
    return inp


SMALL_GQA = [
    wl.TINY_GQA,
    wl.GQA_SHARE.with_(name="gqa_g8_ragged", batch=4, lengths=(1, 77, 1000, 5000), seed=11),
    wl.GQA_SHARE.with_(name="gqa_g4_b16_c3", batch=4, num_q_heads=8, num_kv_heads=2,
                       block_size=16, cp_size=3, interleave=16, lengths=(3, 64, 65, 2000),
                       seed=12),
    wl.GQA_SHARE.with_(name="gqa_g16_i1", batch=3, num_q_heads=16, num_kv_heads=1,
                       block_size=32, cp_size=4, interleave=1, lengths=(5, 129, 1500), seed=13),
    wl.TINY_GQA.with_(name="gqa_f32_g2_i3", batch=3, num_q_heads=4, num_kv_heads=2,
                      block_size=8, cp_size=2, interleave=3, lengths=(1, 10, 333), seed=14),
    wl.GQA_SHARE.with_(name="gqa_g1_c1", batch=2, num_q_heads=2, num_kv_heads=2, block_size=64,
                       cp_size=1, interleave=64, lengths=(700, 129), seed=15),
    wl.GQA_SHARE.with_(name="gqa_i_gt_b", batch=2, block_size=16, cp_size=2, interleave=48,
                       lengths=(1000, 96), seed=16),
]

SMALL_MLA = [
    wl.MLA_DECODE.with_(name="mla_c8_ragged", batch=3, lengths=(1, 130, 3000), seed=21),
    wl.MLA_DECODE.with_(name="mla_b16_i100_c3", batch=2, block_size=16, cp_size=3,
                        interleave=100, lengths=(64, 2500), seed=22),
    wl.MLA_DECODE.with_(name="mla_c1", batch=2, cp_size=1, lengths=(1000, 4097), seed=23),
    wl.MLA_DECODE.with_(name="mla_i1_c4", batch=2, cp_size=4, interleave=1,
                        lengths=(300, 701), seed=24),
    wl.MLA_LONG.with_(name="mla_i128_c4", batch=2, lengths=(9000, 513), seed=25),
]


@pytest.mark.parametrize("w", SMALL_GQA, ids=[w.name for w in SMALL_GQA])
def test_gqa_small(gpu_lib, w):
    _run_and_check(w)


@pytest.mark.parametrize("w", SMALL_MLA, ids=[w.name for w in SMALL_MLA])
def test_mla_small(gpu_lib, w):
    _run_and_check(w)


# Queries scaled by 30: score spreads of tens of log2 units, so the running max of every
# head jumps by more than the kernels' rescale slack many times per request and the
# softmax is nearly one-hot (the lazy-rescale and near-overflow paths).
LARGE_Q = [SMALL_GQA[1], SMALL_GQA[3], SMALL_GQA[4], SMALL_MLA[0], SMALL_MLA[3]]


@pytest.mark.parametrize("w", LARGE_Q, ids=[w.name + "_q30" for w in LARGE_Q])
def test_large_scores(gpu_lib, w):
    _run_and_check(w, label=w.name + "_q30", q_scale=30.0)


def test_gqa_full_share(gpu_lib):
    """64 x 32768 bf16 GQA share, C = 2, I = 128: requests 0, 31, 63 checked exhaustively."""
    _run_and_check(wl.GQA_SHARE, requests=[0, 31, 63])


def test_mla_full_decode(gpu_lib):
    """64 x 67584 MLA, C = 8, I = 64: requests 0 and 63 checked exhaustively."""
    _run_and_check(wl.MLA_DECODE, requests=[0, 63])


def test_mla_full_long(gpu_lib):
    """8 x 200000 MLA, C = 4, I = 128: all 4 shards and the merge; requests 0 and 5."""
    _run_and_check(wl.MLA_LONG, requests=[0, 5])


def test_mla_full_ragged(gpu_lib):
    """512 lognormal-length MLA requests, C = 8, I = 64, with injected edge lengths: every
    edge-length request (empty shards included) plus two lognormal ones."""
    w = wl.MLA_RAGGED
    lens = w.seq_lens()
    edge = [int(np.where(lens == L)[0][0]) for L in (1, 2, 63, 64, 65, 448, 449, 513, 262144)]
    rest = [i for i in range(w.batch) if i not in edge][:2]
    _run_and_check(w, requests=edge + rest)

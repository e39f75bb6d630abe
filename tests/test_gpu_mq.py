"""Parity of multi-token decode (q_len query positions per request, causally masked among
the request's draft tokens) against the CPU oracle (GPU).

Every case runs all ranks' shards through dcp_attn_shard_mq, merges them with dcp_merge
and compares every rank's partial and the merged output of the checked requests with the
oracle, elementwise (tolerances in parity_helpers).  The cases cover every q_len, GQA rows
per KV head from 1 to 64 (bf16 on the matrix cores, one workgroup up to 48 rows and
32-row slices past 48; fp32 on the vector ALUs), both dtypes, both
MLA tile paths (page-contiguous and token-granular), requests shorter than q_len (query
positions before the sequence start: empty rows), positions whose visible tokens end
inside or before an item, and the full-size GQA share and MLA decode shapes.
"""
import numpy as np
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from parity_helpers import check_requests, run_shards

pytestmark = pytest.mark.gpu


def _run_and_check(w, requests=None, q_scale=None):
    torch.cuda.synchronize()
    print(f"[mq] {w.name}: q_len={w.q_len} batch={w.batch} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} C={w.cp_size} I={w.interleave} B={w.block_size} "
          f"q_scale={q_scale}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    assert inp["q"].dim() == 4 and inp["q"].shape[1] == w.q_len
    if q_scale is not None:
        inp["q"] = (inp["q"].float() * q_scale).to(inp["q"].dtype)
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    o_parts, l_parts = run_shards(inp, kind, w.cp_size, w.interleave, w.scale)
    assert o_parts.shape == (w.cp_size, w.batch, w.q_len, w.num_q_heads, w.head_dim_v)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    check_requests(inp, kind, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   list(range(w.batch)) if requests is None else requests, w.name)


G = wl.GQA_SHARE
MQ_GQA = [
    # G = 8: 16, 24, 32 rows per KV head (2, 3, 4 rows per wave); items end at draft tokens
    G.with_(name="mq_gqa_g8_q2", batch=3, q_len=2, lengths=(2, 700, 3000), seed=51),
    G.with_(name="mq_gqa_g8_q3", batch=4, q_len=3, lengths=(1, 2, 129, 2050), seed=52),
    G.with_(name="mq_gqa_g8_q4_i1", batch=3, q_len=4, block_size=32, cp_size=4, interleave=1,
            lengths=(3, 515, 1800), seed=53),
    # G = 16, q_len 4 / 3: 64 rows per KV head (two 32-row slices) / 48 (one workgroup)
    G.with_(name="mq_gqa_g16_q4", batch=2, q_len=4, num_q_heads=16, lengths=(9, 1300),
            seed=54),
    G.with_(name="mq_gqa_g16_q3_h2_i1", batch=2, q_len=3, num_q_heads=32, num_kv_heads=2,
            block_size=32, cp_size=3, interleave=1, lengths=(2, 1500), seed=49),
    # G = 4, q_len 3: 12 rows (repeated rows past the end of the wave grid)
    G.with_(name="mq_gqa_g4_q3_c3", batch=3, q_len=3, num_q_heads=8, num_kv_heads=2,
            block_size=16, cp_size=3, interleave=16, lengths=(4, 65, 1000), seed=55),
    # matrix-core rows: G = 16, q_len 2 (32 rows, position = row / 16); two KV heads of
    # G = 4 at q_len 4 (16 rows) on page-contiguous tiles
    G.with_(name="mq_gqa_g16_q2", batch=2, q_len=2, num_q_heads=16, lengths=(5, 2600),
            seed=59),
    G.with_(name="mq_gqa_g4_q4_h2", batch=3, q_len=4, num_q_heads=8, num_kv_heads=2,
            block_size=64, interleave=64, lengths=(4, 130, 5000), seed=60),
    # G = 2, q_len 4: 8 rows on the matrix cores, position = row / 2
    G.with_(name="mq_gqa_g2_q4", batch=2, q_len=4, num_q_heads=4, num_kv_heads=2,
            lengths=(3, 1700), seed=50),
    # G = 1, q_len 3: 3 rows on 4 waves
    G.with_(name="mq_gqa_g1_q3", batch=2, q_len=3, num_q_heads=2, num_kv_heads=2,
            block_size=64, cp_size=1, interleave=64, lengths=(700, 66), seed=56),
    # f32, G = 2, q_len 3: 6 rows on 8 waves; interleave 3
    wl.TINY_GQA.with_(name="mq_gqa_f32_g2_q3_i3", batch=3, q_len=3, num_q_heads=4,
                      num_kv_heads=2, block_size=8, cp_size=2, interleave=3,
                      lengths=(2, 10, 333), seed=57),
]

M = wl.MLA_DECODE
MQ_MLA = [
    M.with_(name="mq_mla_q2_c8", batch=3, q_len=2, lengths=(1, 130, 3000), seed=61),
    M.with_(name="mq_mla_q3_c3_b16", batch=3, q_len=3, block_size=16, cp_size=3, interleave=100,
            lengths=(2, 64, 2500), seed=62),
    M.with_(name="mq_mla_q4_i1_c4", batch=2, q_len=4, cp_size=4, interleave=1,
            lengths=(3, 701), seed=63),
    M.with_(name="mq_mla_q4_c1", batch=2, q_len=4, cp_size=1, lengths=(1000, 4097), seed=64),
]


@pytest.mark.parametrize("w", MQ_GQA, ids=[w.name for w in MQ_GQA])
def test_mq_gqa_small(gpu_lib, w):
    _run_and_check(w)


@pytest.mark.parametrize("w", MQ_MLA, ids=[w.name for w in MQ_MLA])
def test_mq_mla_small(gpu_lib, w):
    _run_and_check(w)


@pytest.mark.parametrize("w", [MQ_GQA[1], MQ_MLA[0]], ids=["gqa_q30", "mla_q30"])
def test_mq_large_scores(gpu_lib, w):
    _run_and_check(w.with_(name=w.name + "_q30"), q_scale=30.0)


def test_mq_single_position_equals_decode(gpu_lib):
    """q_len = 1 through dcp_attn_shard_mq is bit-identical to dcp_attn_shard."""
    w = G.with_(name="mq_one", batch=3, lengths=(5, 900, 4000), seed=58)
    inp = wl.make_inputs(w, device="cuda")
    for r in range(w.cp_size):
        o1, l1, _ = dca.shard(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                              inp["seq_lens"], r, w.cp_size, w.interleave, w.scale)
        o4, l4, _ = dca.shard(inp["q"][:, None].contiguous(), inp["k_pages"], inp["v_pages"],
                              inp["block_table"], inp["seq_lens"], r, w.cp_size, w.interleave,
                              w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1, o4[:, 0]) and torch.equal(l1, l4[:, 0])


def test_mq_gqa_full_share(gpu_lib):
    """64 x 32768 GQA share with 4 query positions: requests 0 and 63 checked."""
    _run_and_check(G.with_(q_len=4), requests=[0, 63])


def test_mq_mla_full_decode(gpu_lib):
    """64 x 67584 MLA with 2 query positions, C = 8: requests 0 and 63 checked."""
    _run_and_check(M.with_(q_len=2), requests=[0, 63])

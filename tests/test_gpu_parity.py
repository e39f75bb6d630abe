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
from parity_helpers import (REL_L2_BF16, REL_L2_F32, TOL_F32, assert_close, assert_rel_l2,
                            check_requests, run_shards, scale_of)

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
    # fewer gathered heads (smaller DCP groups): 64, 32 and 16 heads
    wl.MLA_DECODE.with_(name="mla_h64_c4", batch=3, num_q_heads=64, cp_size=4,
                        lengths=(1, 700, 3000), seed=26),
    wl.MLA_DECODE.with_(name="mla_h32_i1_c2", batch=2, num_q_heads=32, cp_size=2, interleave=1,
                        lengths=(5, 900), seed=27),
    wl.MLA_DECODE.with_(name="mla_h16_q2_c2", batch=2, num_q_heads=16, cp_size=2, q_len=2,
                        lengths=(3, 2200), seed=28),
    wl.MLA_DECODE.with_(name="mla_h64_b16_i100_c3", batch=2, num_q_heads=64, block_size=16,
                        cp_size=3, interleave=100, lengths=(64, 2500), seed=29),
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
    """64 x 32768 bf16 GQA share, C = 2, I = 128: every request checked exhaustively."""
    _run_and_check(wl.GQA_SHARE)


def test_mla_full_decode(gpu_lib):
    """64 x 67584 MLA, C = 8, I = 64: requests 0 and 63 checked exhaustively."""
    _run_and_check(wl.MLA_DECODE, requests=[0, 63])


@pytest.fixture(scope="module")
def mla_long_run(gpu_lib):
    """8 x 200000 MLA, C = 4, I = 128: all 4 shards and the merge, run once for the
    per-request checks below."""
    w = wl.MLA_LONG
    print(f"[parity] {w.name}: batch={w.batch} C={w.cp_size} I={w.interleave}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    o_parts, l_parts = run_shards(inp, dca.MLA, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    return w, inp, o_parts, l_parts, o_m, l_m


@pytest.mark.parametrize("b", range(wl.MLA_LONG.batch))
def test_mla_full_long(mla_long_run, b):
    """Every request of the long-context workload, one test each (the oracle takes several
    seconds per 200000-token request)."""
    w, inp, o_parts, l_parts, o_m, l_m = mla_long_run
    check_requests(inp, dca.MLA, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   [b], w.name)


def test_mla_full_ragged(gpu_lib):
    """512 lognormal-length MLA requests, C = 8, I = 64, with injected edge lengths: every
    edge-length request (empty shards included) plus two lognormal ones."""
    w = wl.MLA_RAGGED
    lens = w.seq_lens()
    edge = [int(np.where(lens == L)[0][0]) for L in (1, 2, 63, 64, 65, 448, 449, 513, 262144)]
    rest = [i for i in range(w.batch) if i not in edge][:2]
    _run_and_check(w, requests=edge + rest)


def _plan_chunk(ws):
    """Tokens per work item of the plan a shard call left in its workspace (header[2])."""
    return int(ws[8:12].cpu().numpy().view(np.int32)[0])


SPLIT_CASES = [(wl.GQA_SHARE, dca.GQA, 17), (wl.MLA_DECODE, dca.MLA, 40)]


@pytest.mark.parametrize("w,kind,b", SPLIT_CASES, ids=[c[0].name for c in SPLIT_CASES])
def test_split_invariance(gpu_lib, w, kind, b):
    """One request of a full-size batch, run alone: the planner then cuts its shard into
    many more, shorter work items (a different split and split-combine), and the result
    must agree with the batched one and with the oracle."""
    print(f"[split] {w.name} request {b}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    one = dict(inp, q=inp["q"][b:b + 1].contiguous(),
               block_table=inp["block_table"][b:b + 1].contiguous(),
               seq_lens=inp["seq_lens"][b:b + 1].contiguous())
    rl2 = REL_L2_BF16 if inp["q"].dtype == torch.bfloat16 else REL_L2_F32
    o1_parts, l1_parts = [], []
    for r in range(w.cp_size):
        o_all, l_all, ws_all = dca.shard(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], r,
                                         w.cp_size, w.interleave, w.scale, kind=kind)
        o_one, l_one, ws_one = dca.shard(one["q"], kv, v, one["block_table"], one["seq_lens"],
                                         r, w.cp_size, w.interleave, w.scale, kind=kind)
        torch.cuda.synchronize()
        assert dca.read_device_errors(ws_all) == 0 and dca.read_device_errors(ws_one) == 0
        c_all, c_one = _plan_chunk(ws_all), _plan_chunk(ws_one)
        assert c_one < c_all, (c_one, c_all)
        assert_close(l_one[0].cpu().numpy(), l_all[b].cpu().numpy(), TOL_F32,
                     f"rank {r} lse alone vs batched")
        assert_rel_l2(o_one[0].cpu().numpy(), o_all[b].cpu().numpy(), rl2,
                      f"rank {r} O alone (items of {c_one}) vs batched (items of {c_all})")
        o1_parts.append(o_one)
        l1_parts.append(l_one)
    o_parts, l_parts = torch.stack(o1_parts), torch.stack(l1_parts)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    check_requests(one, kind, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   [0], f"{w.name} request {b} alone")


LONG_ITEM_CASES = [
    wl.GQA_SHARE.with_(name="gqa_long_items", batch=2, num_q_heads=16, num_kv_heads=16,
                       block_size=64, cp_size=1, interleave=64, lengths=(140000, 139001),
                       seed=61),
    wl.GQA_SHARE_FP8.with_(name="gqa_fp8_long_items", batch=2, num_q_heads=16,
                           num_kv_heads=16, block_size=64, cp_size=1, interleave=64,
                           lengths=(140000, 139001), seed=62),
]


@pytest.mark.parametrize("w", LONG_ITEM_CASES, ids=[w.name for w in LONG_ITEM_CASES])
def test_gqa_items_beyond_64_tiles(gpu_lib, w):
    """Work items longer than 64 tiles of 64 tokens: the GQA kernels rebuild their page
    table in LDS every 64 tiles (16 KV heads leave the planner 32 items per call, so
    279001 tokens give items of 8768 tokens, 137 tiles)."""
    print(f"[parity] {w.name}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    _, _, ws = dca.shard(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                         inp["seq_lens"], 0, w.cp_size, w.interleave, w.scale, kind=dca.GQA,
                         k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"))
    torch.cuda.synchronize()
    assert _plan_chunk(ws) > 64 * 64 * 2, _plan_chunk(ws)
    _run_and_check(w)


@pytest.mark.parametrize("heads", [8, 48, 96, 256])
def test_mla_rejects_head_counts(gpu_lib, heads):
    """MLA takes 16, 32, 64 or 128 gathered heads; other counts are refused before any
    launch."""
    w = wl.MLA_DECODE.with_(name=f"mla_h{heads}", batch=1, num_q_heads=heads, cp_size=2,
                            lengths=(100,), seed=30)
    inp = wl.make_inputs(w, device="cuda")
    with pytest.raises(dca.DCPError):
        dca.shard(inp["q"], inp["latent_pages"], None, inp["block_table"], inp["seq_lens"], 0,
                  w.cp_size, w.interleave, w.scale, kind=dca.MLA)

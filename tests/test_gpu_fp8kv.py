"""Parity of the fp8 KV cache shard call (dcp_attn_shard_fp8kv) against the CPU oracle (GPU).

K and V pages hold OCP FP8 E4M3 codes with one scale each; the oracle attends over the
values decode(code) * scale in float64 (its fp8 reading, pinned on the CPU).  Every rank's
partial and the merged output are compared elementwise with the bf16-input tolerance (the
queries are bf16 and every fp8 value is exact in bf16).  Cases: page-contiguous and
token-granular tiles, one and two 16-row tiles per wave (1, 2, 4, 8, 16, 24, 32, 48 and
64 query rows per KV head, multi-token decode), two KV heads, ragged and empty shards, the full-size GQA share
on sampled requests, bf16 partial outputs, and the shapes the call rejects.
"""
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from parity_helpers import check_requests, run_shards

pytestmark = pytest.mark.gpu

F = wl.GQA_SHARE_FP8
CASES = [
    F.with_(name="fp8_g8_ragged", batch=4, lengths=(1, 77, 1000, 5000), seed=101),
    F.with_(name="fp8_g8_i1_c4", batch=3, block_size=32, cp_size=4, interleave=1,
            lengths=(3, 515, 2100), seed=102),
    F.with_(name="fp8_g4_h2_q4_c3", batch=3, q_len=4, num_q_heads=8, num_kv_heads=2,
            block_size=16, cp_size=3, interleave=16, lengths=(2, 65, 1800), seed=103),
    F.with_(name="fp8_g16_q2", batch=2, q_len=2, num_q_heads=16, lengths=(5, 2600), seed=104),
    F.with_(name="fp8_g8_q3_b64", batch=3, q_len=3, block_size=64, interleave=64,
            lengths=(1, 129, 4000), seed=105),
    # fewer than 16 rows per KV head: 1 (G = 1), 2 (G = 2), 4 (G = 4) rows, padding lanes
    F.with_(name="fp8_g1", batch=2, num_q_heads=2, num_kv_heads=2, lengths=(90, 3000),
            seed=108),
    F.with_(name="fp8_g2_i3", batch=2, num_q_heads=4, num_kv_heads=2, block_size=16, cp_size=2,
            interleave=3, lengths=(7, 1100), seed=109),
    F.with_(name="fp8_g4_c4", batch=3, num_q_heads=8, num_kv_heads=2, cp_size=4, interleave=64,
            block_size=64, lengths=(1, 300, 2600), seed=110),
    # 48 rows per KV head: one workgroup (three row tiles per wave); 64: two 32-row slices
    F.with_(name="fp8_g16_q4", batch=2, q_len=4, num_q_heads=16, lengths=(3, 2000), seed=111),
    F.with_(name="fp8_g16_q3_h2_i3", batch=2, q_len=3, num_q_heads=32, num_kv_heads=2,
            block_size=16, interleave=3, lengths=(40, 900), seed=112),
]


def _run(w, requests=None):
    torch.cuda.synchronize()
    print(f"[fp8kv] {w.name}: q_len={w.q_len} batch={w.batch} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} C={w.cp_size} I={w.interleave} B={w.block_size}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    assert inp["k_pages"].dtype == torch.uint8
    o_parts, l_parts = run_shards(inp, dca.GQA, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    check_requests(inp, dca.GQA, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   list(range(w.batch)) if requests is None else requests, w.name)
    return inp


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_fp8kv_small(gpu_lib, w):
    _run(w)


def test_fp8kv_full_share(gpu_lib):
    """64 x 32768 GQA share with an fp8 cache: requests 0 and 63 checked."""
    _run(F, requests=[0, 63])


def test_fp8kv_bf16_partials(gpu_lib):
    """bf16 partial output = the float32 partial rounded to nearest even."""
    w = F.with_(name="fp8_bf16o", batch=3, lengths=(2, 900, 20000), seed=106)
    inp = wl.make_inputs(w, device="cuda")
    args = (inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"])
    for r in range(w.cp_size):
        kw = dict(max_seq_len=inp["max_seq_len"], k_scale=inp["k_scale"],
                  v_scale=inp["v_scale"])
        o32, l32, _ = dca.shard(*args, r, w.cp_size, w.interleave, w.scale, **kw)
        o16, l16, _ = dca.shard(*args, r, w.cp_size, w.interleave, w.scale,
                                out_dtype=torch.bfloat16, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
        assert torch.equal(l16, l32)


def test_fp8kv_rejects_unsupported(gpu_lib):
    """A group of 80 query heads per KV head (more than 64 rows), float32 queries, missing
    scales: refused before any launch."""
    w = F.with_(name="fp8_g80", batch=1, num_q_heads=80, lengths=(100,), seed=107)
    inp = wl.make_inputs(w, device="cuda")
    with pytest.raises(dca.DCPError):
        dca.shard(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                  inp["seq_lens"], 0, w.cp_size, w.interleave, w.scale,
                  k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    with pytest.raises(TypeError):
        dca.shard(inp["q"].float(), inp["k_pages"], inp["v_pages"], inp["block_table"],
                  inp["seq_lens"], 0, w.cp_size, w.interleave, w.scale,
                  k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    with pytest.raises(ValueError):
        dca.shard(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"],
                  inp["seq_lens"], 0, w.cp_size, w.interleave, w.scale)

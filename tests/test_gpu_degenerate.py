"""Degenerate inputs on the GPU: requests of length 0 (every shard empty: O = 0 and
lse = -inf for every rank and after the merge, never NaN), a batch of only empty requests,
and an empty batch (nothing launched, empty outputs)."""
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from parity_helpers import check_requests, run_shards

pytestmark = pytest.mark.gpu

CASES = [
    wl.GQA_SHARE.with_(name="zero_gqa_bf16", batch=4, lengths=(0, 1, 0, 300), seed=121),
    wl.TINY_GQA.with_(name="zero_gqa_f32", batch=3, lengths=(0, 70, 0), seed=122),
    wl.GQA_SHARE_FP8.with_(name="zero_gqa_fp8", batch=3, lengths=(0, 500, 0), seed=123),
    wl.MLA_DECODE.with_(name="zero_mla", batch=3, lengths=(0, 0, 130), seed=124),
    wl.GQA_SHARE.with_(name="zero_gqa_q2", batch=3, q_len=2, lengths=(0, 1, 200), seed=125),
    wl.MLA_DECODE.with_(name="zero_mla_q2_i1", batch=3, q_len=2, cp_size=4, interleave=1,
                        lengths=(0, 1, 90), seed=126),
    wl.GQA_SHARE.with_(name="all_zero_gqa", batch=2, lengths=(0, 0), seed=127),
    wl.MLA_DECODE.with_(name="all_zero_mla", batch=2, lengths=(0, 0), seed=128),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_zero_length_requests(gpu_lib, w):
    print(f"[degenerate] {w.name}: lengths={w.lengths} q_len={w.q_len}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    o_parts, l_parts = run_shards(inp, kind, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    check_requests(inp, kind, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   list(range(w.batch)), w.name)
    for b, L in enumerate(w.lengths):
        if L == 0:
            assert torch.all(o_m[b] == 0) and torch.all(torch.isneginf(l_m[b]))


@pytest.mark.parametrize("kind", ["gqa", "mla"])
def test_empty_batch(gpu_lib, kind):
    """batch = 0: every call returns at once with empty outputs."""
    w = (wl.GQA_SHARE if kind == "gqa" else wl.MLA_DECODE).with_(batch=1, lengths=(64,), seed=129)
    inp = wl.make_inputs(w, device="cuda")
    q = inp["q"][:0].contiguous()
    bt = inp["block_table"][:0].contiguous()
    lens = inp["seq_lens"][:0].contiguous()
    k = dca.GQA if kind == "gqa" else dca.MLA
    kv = inp["k_pages"] if k == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if k == dca.GQA else None
    o, l, _ = dca.shard(q, kv, v, bt, lens, 0, w.cp_size, w.interleave, w.scale, kind=k,
                        max_seq_len=64)
    assert o.shape[0] == 0 and l.shape[0] == 0
    om, lm = dca.merge(o[None].contiguous(), l[None].contiguous())
    torch.cuda.synchronize()
    assert om.shape[0] == 0 and lm.shape[0] == 0

"""dcp_attn_shard_noalloc: the shard call whose plan and split partials live in the
library's static device scratch.  Its outputs must be bit-identical to dcp_attn_shard_ex
(the same kernels and plan with a caller workspace) on two calls in a row, the second with a
smaller input, for GQA (bf16 and f32, multi-token, bf16 partial output) and MLA; a call whose
workspace would exceed the scratch is refused with DCP_ESCRATCH before any launch."""
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl

pytestmark = pytest.mark.gpu

DCP_ESCRATCH = -5

PAIRS = [
    (wl.GQA_SHARE.with_(name="na_gqa_big", batch=6, lengths=(1, 129, 5000, 20000, 33, 8000),
                        seed=91),
     wl.GQA_SHARE.with_(name="na_gqa_small", batch=2, lengths=(700, 3), seed=92)),
    (wl.TINY_GQA.with_(name="na_f32_q2", batch=3, q_len=2, lengths=(2, 900, 3000), seed=93),
     wl.TINY_GQA.with_(name="na_f32_q2_small", batch=1, q_len=2, lengths=(400,), seed=94)),
    (wl.MLA_DECODE.with_(name="na_mla_big", batch=4, cp_size=4, lengths=(1, 300, 9000, 20000),
                         seed=95),
     wl.MLA_DECODE.with_(name="na_mla_small", batch=2, cp_size=4, lengths=(2000, 65), seed=96)),
]


def _run(w, out_dtype):
    inp = wl.make_inputs(w, device="cuda")
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    res = []
    for r in range(w.cp_size):
        o_ref, l_ref, ws = dca.shard(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], r,
                                     w.cp_size, w.interleave, w.scale, kind=kind,
                                     max_seq_len=inp["max_seq_len"], out_dtype=out_dtype)
        o = torch.full_like(o_ref, float("nan"))
        l = torch.full_like(l_ref, float("nan"))
        dca.shard_noalloc(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], r, w.cp_size,
                          w.interleave, w.scale, o, l, kind=kind,
                          max_seq_len=inp["max_seq_len"])
        res.append((o_ref, l_ref, o, l))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("pair", PAIRS, ids=[p[0].name for p in PAIRS])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32o", "bf16o"])
def test_noalloc_matches_workspace_call(gpu_lib, pair, out_dtype):
    for w in pair:   # two calls in a row, the second smaller
        print(f"[noalloc] {w.name} {out_dtype}", flush=True)
        for o_ref, l_ref, o, l in _run(w, out_dtype):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                               o_ref.view(torch.int16) if o.dtype == torch.bfloat16 else o_ref), \
                f"{w.name}: O differs from dcp_attn_shard_ex"
            assert torch.equal(torch.isneginf(l), torch.isneginf(l_ref))
            fin = ~torch.isneginf(l_ref)
            assert torch.equal(l[fin], l_ref[fin]), f"{w.name}: lse differs"


def test_noalloc_rejects_beyond_scratch(gpu_lib):
    # 1024 MLA requests: the split partials alone need far more than the scratch
    print("[noalloc] oversize", flush=True)
    b = 1024
    q = torch.zeros(b, 128, 576, dtype=torch.bfloat16, device="cuda")
    lat = torch.zeros(1, 64, 576, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(b, 1, dtype=torch.int32, device="cuda")
    lens = torch.full((b,), 64, dtype=torch.int32, device="cuda")
    o = torch.zeros(b, 128, 512, dtype=torch.float32, device="cuda")
    l = torch.zeros(b, 128, dtype=torch.float32, device="cuda")
    desc = dca.make_desc(dca.MLA, q, lat, bt)
    assert dca.workspace_size(desc, b, 64, 1, 64) > dca.NOALLOC_SCRATCH_BYTES
    with pytest.raises(dca.DCPError) as e:
        dca.shard_noalloc(q, lat, None, bt, lens, 0, 1, 64, 0.07, o, l, kind=dca.MLA,
                          max_seq_len=64)
    assert e.value.status == DCP_ESCRATCH
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0   # nothing launched

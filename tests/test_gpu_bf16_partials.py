"""bf16 partial outputs (dcp_attn_shard_ex with o_dtype = DCP_BF16) and the merge of bf16
partials (dcp_merge_ex) on the GPU.

A bf16 partial must be exactly the float32 partial of the same call rounded to nearest
even (both come from the same float32 arithmetic; only the final store differs), for
requests written by the shard kernel directly and for requests combined from split items.
The merge of bf16 partials is checked against the oracle's merge of the same partials
(widened exactly) and, end to end, against the oracle's unsharded attention.
"""
import numpy as np
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from oracle import dcp_oracle as orc
from parity_helpers import (REL_L2_BF16, TOL_F32, assert_close, assert_rel_l2, oracle_full,
                            request_host)

pytestmark = pytest.mark.gpu

CASES = [
    wl.GQA_SHARE.with_(name="bf16o_gqa_ragged", batch=4, lengths=(1, 77, 1000, 20000), seed=71),
    wl.TINY_GQA.with_(name="bf16o_gqa_f32in_i3", batch=3, num_q_heads=4, num_kv_heads=2,
                      block_size=8, cp_size=2, interleave=3, lengths=(1, 10, 333), seed=72),
    wl.MLA_DECODE.with_(name="bf16o_mla_c8", batch=3, lengths=(1, 130, 30000), seed=73),
    wl.GQA_SHARE.with_(name="bf16o_gqa_q4", batch=3, q_len=4, lengths=(2, 900, 20000), seed=75),
    wl.MLA_DECODE.with_(name="bf16o_mla_q2_i1", batch=2, q_len=2, cp_size=4, interleave=1,
                        lengths=(3, 2100), seed=74),
]


def _shards(inp, w, kind, out_dtype):
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    os_, ls_ = [], []
    ws = None
    for r in range(w.cp_size):
        o, l, ws = dca.shard(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], r, w.cp_size,
                             w.interleave, w.scale, kind=kind, max_seq_len=inp["max_seq_len"],
                             workspace=ws, out_dtype=out_dtype)
        os_.append(o)
        ls_.append(l)
    torch.cuda.synchronize()
    assert dca.read_device_errors(ws) == 0
    return torch.stack(os_), torch.stack(ls_)


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_bf16_partials(gpu_lib, w):
    print(f"[bf16o] {w.name}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    o32, l32 = _shards(inp, w, kind, torch.float32)
    o16, l16 = _shards(inp, w, kind, torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16)), \
        "bf16 partial differs from the rounded float32 partial"
    assert torch.equal(l16.isinf(), l32.isinf())
    fin = ~l32.isinf()
    assert torch.equal(l16[fin], l32[fin])
    # merge of the bf16 partials: against the oracle's merge of the same (widened) values,
    # and end to end against unsharded attention
    o_m, l_m = dca.merge(o16, l16)
    torch.cuda.synchronize()
    ref_o, ref_l = orc.merge(o16.double().cpu().numpy(), l16.double().cpu().numpy())
    assert_close(o_m.cpu().numpy(), ref_o, (1e-5, 1e-5), f"{w.name} merge of bf16 partials O")
    assert_close(l_m.cpu().numpy(), ref_l, (1e-5, 1e-5), f"{w.name} merge of bf16 partials lse")
    tol = (2e-2, 2e-2)
    for b in range(w.batch):
        h = request_host(inp, kind, b)
        o_ref, l_ref = oracle_full(h, kind, w.scale)
        assert_close(o_m[b].cpu().numpy(), o_ref, tol, f"{w.name} b={b} merged O")
        assert_rel_l2(o_m[b].cpu().numpy(), o_ref, REL_L2_BF16, f"{w.name} b={b} merged O")
        assert_close(l_m[b].cpu().numpy(), l_ref, TOL_F32, f"{w.name} b={b} merged lse")


@pytest.mark.parametrize("c,b,h,dv", [(8, 5, 16, 512), (3, 7, 8, 128), (12, 3, 4, 512)])
def test_merge_bf16_poisoned(gpu_lib, c, b, h, dv):
    """bf16 partials with empty (-inf) partials holding NaN garbage, every partial of some
    rows empty, more partials than the one-round-trip path holds."""
    g = torch.Generator(device="cuda")
    g.manual_seed(c * 1000 + b)
    o = torch.randn(c, b, h, dv, device="cuda", generator=g).to(torch.bfloat16)
    lse = torch.randn(c, b, h, device="cuda", generator=g) * 5
    empty = torch.rand(c, b, h, device="cuda", generator=g) < 0.3
    empty[:, 0, 0] = True
    lse[empty] = float("-inf")
    o[empty] = float("nan")
    o_m, l_m = dca.merge(o, lse)
    ob, lb = dca.merge(o, lse, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref_o, ref_l = orc.merge(o.double().cpu().numpy(), lse.double().cpu().numpy())
    assert_close(o_m.cpu().numpy(), ref_o, (1e-5, 1e-5), "O")
    assert_close(l_m.cpu().numpy(), ref_l, (1e-5, 1e-5), "lse")
    assert np.all(o_m[0, 0].cpu().numpy() == 0) and np.isneginf(l_m[0, 0].item())
    assert torch.equal(ob.view(torch.int16), o_m.to(torch.bfloat16).view(torch.int16))

"""The shard and merge entry points do no host synchronisation and allocate nothing
themselves, so one decode step (every rank's shard call + the merge) can be captured in a
HIP graph and replayed (GQA, MLA at interleave 1, multi-token GQA over an fp8 cache, and
multi-token MLA on page-contiguous tiles).  Every replay must reproduce the eager result bit for bit (the
kernels are deterministic), with the program's own eager work and synchronisations between
the replays.
"""
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = [
    wl.GQA_SHARE.with_(name="graph_gqa", batch=4, lengths=(1, 77, 1000, 5000), seed=31),
    wl.MLA_DECODE.with_(name="graph_mla_i1", batch=3, cp_size=4, interleave=1,
                        lengths=(5, 300, 2100), seed=32),
    wl.GQA_SHARE_FP8.with_(name="graph_gqa_fp8kv_q2", batch=3, q_len=2, lengths=(3, 700, 4000),
                           seed=33),
    wl.MLA_DECODE.with_(name="graph_mla_i64_q2", batch=3, q_len=2, lengths=(5, 3000, 9000),
                        seed=34),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_graph_replay_matches_eager(gpu_lib, w):
    print(f"[graph] {w.name}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    C = w.cp_size
    rows = (w.batch,) + ((w.q_len,) if w.q_len > 1 else ()) + (w.num_q_heads,)
    o_parts = torch.empty((C,) + rows + (w.head_dim_v,), device="cuda")
    l_parts = torch.empty((C,) + rows, device="cuda")
    out = torch.empty(rows + (w.head_dim_v,), device="cuda")
    lse = torch.empty(rows, device="cuda")
    ws = dca.alloc_workspace(dca.make_desc(kind, inp["q"], kv, inp["block_table"]), w.batch,
                             inp["max_seq_len"], C, w.interleave, q_len=w.q_len)

    def step():
        for r in range(C):
            dca.shard(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], r, C, w.interleave,
                      w.scale, kind=kind, max_seq_len=inp["max_seq_len"], out=o_parts[r],
                      lse=l_parts[r], workspace=ws, k_scale=inp.get("k_scale"),
                      v_scale=inp.get("v_scale"))
        dca.merge(o_parts, l_parts, out=out, lse_out=lse)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # eager, on the stream the capture will use
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(float("nan"))     # eager work between the replays
        lse.fill_(float("nan"))
        o_parts.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"{w.name}: replay {rep} O differs"
        assert torch.equal(lse.isinf(), ref_l.isinf())
        fin = ~ref_l.isinf()
        assert torch.equal(lse[fin], ref_l[fin]), f"{w.name}: replay {rep} lse differs"
    assert dca.read_device_errors(ws) == 0

"""The work plan a shard call leaves in its workspace (GPU; integer, bit-exact).

The planner splits the tokens a rank owns into work items (request, local begin, local
end, partial index) and stores them in dispatch order.  Its layout in the workspace is the
one the library documents: int32 header[64] ([1] = item count, [2] = tokens per item),
int32 off[batch + 1] at byte 256, int4 items from the next 256-byte boundary.

Checked against the host walker (dcp_local_len) and the bounds the host sizes the
workspace with: the items of every request tile its local tokens [0, local_len) exactly,
in item-size pieces; a request's partial indices are off[b], off[b] + 1, ... in token
order; the item count is at most target + batch; the dispatch order never increases in
tile count (capped at 1023 tiles).
"""
import numpy as np
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = [
    # uniform GQA share (every item full size), ragged GQA, ragged MLA with empty shards,
    # token-granular interleave, one long request
    (wl.GQA_SHARE.with_(batch=64, lengths=(32768,) * 64), dca.GQA, 0),
    (wl.GQA_SHARE.with_(name="plan_gqa_ragged", batch=6, lengths=(1, 77, 128, 1000, 5000, 20001),
                        seed=81), dca.GQA, 1),
    # 64 query rows per KV head on two KV heads: two 32-row slices per item and KV head
    (wl.GQA_SHARE.with_(name="plan_gqa_g16_q4_h2", batch=5, q_len=4, num_q_heads=32,
                        num_kv_heads=2, lengths=(1, 65, 5000, 20001, 300), seed=84), dca.GQA, 1),
    # 48 query rows per KV head: one workgroup per item and KV head
    (wl.GQA_SHARE.with_(name="plan_gqa_g16_q3", batch=4, q_len=3, num_q_heads=16,
                        lengths=(2, 300, 9000, 20001), seed=86), dca.GQA, 1),
    # fp32 queries and cache (vector-ALU kernel)
    (wl.GQA_SHARE.with_(name="plan_gqa_f32", dtype="f32", head_dim_qk=64, head_dim_v=64,
                        batch=3, lengths=(1, 4000, 20001), seed=85), dca.GQA, 1),
    (wl.MLA_RAGGED, dca.MLA, 5),
    (wl.MLA_DECODE.with_(name="plan_mla_i1", batch=3, cp_size=4, interleave=1,
                         lengths=(3, 700, 9000), seed=82), dca.MLA, 3),
    (wl.MLA_LONG.with_(name="plan_mla_long", batch=1, lengths=(200000,), seed=83), dca.MLA, 0),
]


def _decode(ws, batch):
    raw = ws.cpu().numpy()
    hdr = raw[:256].view(np.int32)
    off = raw[256:256 + 4 * (batch + 1)].view(np.int32)
    items_at = 256 + (4 * (batch + 1) + 255) // 256 * 256
    n = int(hdr[1])
    items = raw[items_at:items_at + 16 * n].view(np.int32).reshape(n, 4)
    return hdr, off, items


@pytest.mark.parametrize("w,kind,rank", CASES, ids=[c[0].name for c in CASES])
def test_plan(gpu_lib, w, kind, rank):
    print(f"[plan] {w.name} rank {rank}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    _, _, ws = dca.shard(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], rank, w.cp_size,
                         w.interleave, w.scale, kind=kind, max_seq_len=inp["max_seq_len"])
    torch.cuda.synchronize()
    assert dca.read_device_errors(ws) == 0
    hdr, off, items = _decode(ws, w.batch)
    n, chunk = int(hdr[1]), int(hdr[2])
    tile = 64 if kind == dca.GQA else 32
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = w.q_len * (w.num_q_heads // w.num_kv_heads)
    slices = 2 if (kind == dca.GQA and w.dtype == "bf16" and rows > 48) else 1
    target = (max(1, cus * 2 // (w.num_kv_heads * slices)) if kind == dca.GQA
              else max(1, cus // w.q_len))
    assert chunk % tile == 0 and chunk > 0
    assert n <= target + w.batch
    lens = [int(x) for x in inp["seq_lens"].cpu()]
    loc = [dca.local_len(L, rank, w.cp_size, w.interleave) for L in lens]
    assert off[0] == 0 and int(off[w.batch]) == n
    # every request: items tile [0, loc) in chunk-size pieces, partial indices consecutive
    seen = np.zeros(n, dtype=bool)
    by_req = {}
    for k in range(n):
        b, j0, j1, p = (int(x) for x in items[k])
        assert 0 <= b < w.batch and 0 <= p < n and not seen[p]
        seen[p] = True
        by_req.setdefault(b, []).append((j0, j1, p))
    for b in range(w.batch):
        its = sorted(by_req.get(b, []))
        expect = [(j, min(j + chunk, loc[b])) for j in range(0, loc[b], chunk)]
        assert [(j0, j1) for j0, j1, _ in its] == expect, f"request {b}"
        assert [p for _, _, p in its] == list(range(int(off[b]), int(off[b + 1]))), f"request {b}"
    assert seen.all()
    # dispatch order: non-increasing tile count (capped)
    tiles = np.minimum((items[:, 2] - items[:, 1] + tile - 1) // tile, 1023)
    assert np.all(np.diff(tiles) <= 0)

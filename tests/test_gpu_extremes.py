"""GPU parity at the extremes of the layout parameters and of the merge's partial count:
one-token pages, pages of 512 and 1024 tokens, 16 to 64 ranks, an interleave longer than
every sequence (rank 0 owns everything), and merges of 9 to 100 partials (the streamed row
merge, lse over more than one 64-lane pass), each against the oracle."""
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from oracle import dcp_oracle as orc
from parity_helpers import assert_close, check_requests, run_shards

pytestmark = pytest.mark.gpu

G = wl.GQA_SHARE
M = wl.MLA_DECODE
F = wl.GQA_SHARE_FP8
T = wl.TINY_GQA

LAYOUT_CASES = [
    # one token per page: every tile gathers 64 (32) pages
    G.with_(name="x_gqa_b1", batch=3, block_size=1, cp_size=3, interleave=5,
            lengths=(1, 7, 300), seed=301),
    T.with_(name="x_f32_b1_i1", batch=2, block_size=1, cp_size=2, interleave=1,
            lengths=(2, 129), seed=302),
    M.with_(name="x_mla_b1_i1", batch=3, block_size=1, cp_size=2, interleave=1,
            lengths=(1, 65, 300), seed=303),
    F.with_(name="x_fp8_b1_i3", batch=2, block_size=1, cp_size=2, interleave=3,
            lengths=(1, 500), seed=304),
    # large pages on the page-contiguous tiles
    G.with_(name="x_gqa_b1024", batch=3, block_size=1024, cp_size=2, interleave=1024,
            lengths=(3000, 1025, 1), seed=305),
    M.with_(name="x_mla_b512", batch=2, block_size=512, cp_size=2, interleave=512,
            lengths=(3000, 1), seed=306),
    # many ranks: most shards of the short requests are empty
    G.with_(name="x_gqa_c64_i1", batch=3, block_size=16, cp_size=64, interleave=1,
            lengths=(100, 7, 64), seed=307),
    M.with_(name="x_mla_c16_i3", batch=2, block_size=16, cp_size=16, interleave=3,
            lengths=(100, 2), seed=308),
    # an interleave longer than every sequence: rank 0 owns all tokens, the others none
    G.with_(name="x_gqa_i_gt_l", batch=2, block_size=128, cp_size=4, interleave=100000,
            lengths=(5000, 1), seed=309),
    M.with_(name="x_mla_i_gt_l", batch=2, block_size=64, cp_size=3, interleave=70000,
            lengths=(4000, 33), seed=310),
]


@pytest.mark.parametrize("w", LAYOUT_CASES, ids=[w.name for w in LAYOUT_CASES])
def test_layout_extremes(gpu_lib, w):
    """Every rank's shard and the merged result of every request against the oracle."""
    print(f"[extreme] {w.name}: B={w.block_size} C={w.cp_size} I={w.interleave} "
          f"lens={w.lengths}", flush=True)
    kind = dca.MLA if w.kind == "mla" else dca.GQA
    inp = wl.make_inputs(w, device="cuda")
    o_parts, l_parts = run_shards(inp, kind, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    check_requests(inp, kind, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   range(w.batch), w.name)


@pytest.mark.parametrize("c,b,h,dv", [(9, 3, 4, 512), (16, 2, 8, 128), (64, 2, 3, 256),
                                      (100, 2, 2, 512), (100, 1, 3, 100)])
@pytest.mark.parametrize("in_bf16", [False, True], ids=["f32in", "bf16in"])
def test_merge_many_partials(gpu_lib, c, b, h, dv, in_bf16):
    """More partials than the one-round-trip merge takes: streamed in batches of 8, and past
    64 partials the lse reduction takes more than one pass over the lanes.  Some partials
    are empty (lse = -inf, rows of NaN), one row entirely."""
    print(f"[merge-many] C={c} b={b} H={h} Dv={dv} bf16 in={in_bf16}", flush=True)
    g = torch.Generator().manual_seed(400 + c + dv)
    o = torch.randn(c, b, h, dv, generator=g)
    if in_bf16:
        o = o.to(torch.bfloat16)
    lse = torch.randn(c, b, h, generator=g) * 6
    empty = torch.rand(c, b, h, generator=g) < 0.3
    lse[empty] = -float("inf")
    o[empty] = float("nan")
    lse[:, 0, 0] = -float("inf")
    o[:, 0, 0] = float("nan")
    out, lse_out = dca.merge(o.cuda(), lse.cuda())
    ref_o, ref_l = orc.merge(o.double().numpy(), lse.double().numpy())
    assert_close(lse_out.cpu().numpy(), ref_l, (1e-5, 1e-5), "merged lse")
    assert_close(out.cpu().numpy(), ref_o, (1e-5, 1e-5), "merged O")
    assert torch.all(out[0, 0] == 0)
    # bf16 output: the float32 result rounded to nearest even
    out_bf, _ = dca.merge(o.cuda(), lse.cuda(), out_dtype=torch.bfloat16, want_lse=False)
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


ITEM_CASES = [
    # one long request per call: the planner cuts it into hundreds of work items, so the
    # split combine merges more than 64 partials per row (GQA: one wave per row; MLA: one
    # wave per 256 columns, the first 32 partials loaded with the lse)
    G.with_(name="x_gqa_one_long", batch=1, cp_size=1, lengths=(100000,), seed=320),
    F.with_(name="x_fp8_one_long", batch=1, cp_size=1, lengths=(100000,), seed=321),
    M.with_(name="x_mla_one_long", batch=1, cp_size=1, lengths=(60000,), seed=322),
    M.with_(name="x_mla_one_long_q2", batch=1, cp_size=2, q_len=2, lengths=(61000,), seed=323),
    T.with_(name="x_f32_one_long", batch=1, cp_size=1, lengths=(50000,), seed=324),
]


@pytest.mark.parametrize("w", ITEM_CASES, ids=[w.name for w in ITEM_CASES])
def test_many_items_per_request(gpu_lib, w):
    """A single long request, split over many work items, against the oracle."""
    kind = dca.MLA if w.kind == "mla" else dca.GQA
    inp = wl.make_inputs(w, device="cuda")
    o_parts, l_parts = run_shards(inp, kind, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    _, _, ws = dca.shard(inp["q"], inp["k_pages"] if kind == dca.GQA else inp["latent_pages"],
                         inp["v_pages"] if kind == dca.GQA else None, inp["block_table"],
                         inp["seq_lens"], 0, w.cp_size, w.interleave, w.scale, kind=kind,
                         max_seq_len=inp["max_seq_len"], k_scale=inp.get("k_scale"),
                         v_scale=inp.get("v_scale"))
    torch.cuda.synchronize()
    n_items = int(ws[:8].cpu().numpy().view("int32")[1])   # plan header: item count
    print(f"[items] {w.name}: {n_items} work items on rank 0", flush=True)
    assert n_items > 64
    check_requests(inp, kind, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   range(w.batch), w.name)


WINDOW_CASES = [
    # per-token tile tables (interleave or block size not a multiple of 32) with items long
    # enough that the table windows (12 tiles each) are rebuilt several times inside an item
    M.with_(name="x_mla_i1_windows", batch=1, num_q_heads=16, cp_size=2, interleave=1,
            lengths=(600000,), seed=330),
    M.with_(name="x_mla_b16_i3_windows", batch=2, num_q_heads=32, block_size=16, cp_size=1,
            interleave=3, lengths=(300000, 5), seed=331),
    M.with_(name="x_mla_i1_q2_windows", batch=1, num_q_heads=16, cp_size=2, interleave=1,
            q_len=2, lengths=(400000,), seed=332),
]


@pytest.mark.parametrize("w", WINDOW_CASES, ids=[w.name for w in WINDOW_CASES])
def test_mla_table_windows_inside_items(gpu_lib, w):
    """MLA work items spanning several per-token table windows, against the oracle."""
    inp = wl.make_inputs(w, device="cuda")
    o_parts, l_parts = run_shards(inp, dca.MLA, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    _, _, ws = dca.shard(inp["q"], inp["latent_pages"], None, inp["block_table"],
                         inp["seq_lens"], 0, w.cp_size, w.interleave, w.scale, kind=dca.MLA,
                         max_seq_len=inp["max_seq_len"])
    torch.cuda.synchronize()
    chunk = int(ws[:16].cpu().numpy().view("int32")[2])   # plan header: item size (tokens)
    print(f"[windows] {w.name}: items of {chunk} tokens ({chunk // 32} tiles)", flush=True)
    assert chunk // 32 > 24
    check_requests(inp, dca.MLA, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   range(w.batch), w.name)

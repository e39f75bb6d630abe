"""GPU tests of the merge kernel alone, the exported block-table walk (bit-exact) and the
device error word."""
import numpy as np
import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from oracle import dcp_oracle as orc
from parity_helpers import (TOL_F32, assert_close, assert_rel_l2, o_rel_l2, o_tol,
                            oracle_tokens)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("c,b,h,dv", [(2, 3, 8, 128), (8, 5, 128, 512), (4, 2, 3, 64),
                                      (3, 4, 2, 100), (1, 2, 4, 256)])
def test_merge_poisoned_partials(gpu_lib, c, b, h, dv):
    """Merge kernel vs the oracle's merge on synthetic partials where some partials are
    empty (lse = -inf) and carry NaN garbage, and some rows are entirely empty."""
    print(f"[merge] C={c} b={b} H={h} Dv={dv}", flush=True)
    g = torch.Generator().manual_seed(100 + c + dv)
    o = torch.randn(c, b, h, dv, generator=g)
    lse = torch.randn(c, b, h, generator=g) * 6
    empty = torch.rand(c, b, h, generator=g) < 0.3
    lse[empty] = -float("inf")
    o[empty] = float("nan")
    lse[:, 0, 0] = -float("inf")            # a row with every partial empty
    o[:, 0, 0] = float("nan")
    out, lse_out = dca.merge(o.cuda(), lse.cuda())
    ref_o, ref_l = orc.merge(o.numpy(), lse.numpy())
    assert_close(lse_out.cpu().numpy(), ref_l, (1e-5, 1e-5), "merged lse")
    assert_close(out.cpu().numpy(), ref_o, (1e-5, 1e-5), "merged O")
    assert torch.all(out[0, 0] == 0)
    # bf16 output: the fp32 result rounded to nearest even
    out_bf, _ = dca.merge(o.cuda(), lse.cuda(), out_dtype=torch.bfloat16, want_lse=False)
    assert torch.equal(out_bf.cpu(), out.cpu().to(torch.bfloat16))


def _slots_case(bt, lens, B, nb, C, I, label):
    bt_d = torch.from_numpy(bt).cuda()
    lens_d = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    for r in range(C):
        slots, offs, ws = dca.shard_slots(bt_d, lens_d, B, nb, r, C, I, seq_lens_host=list(lens))
        assert dca.read_device_errors(ws) == 0
        slots = slots.cpu().numpy()
        offs = offs.cpu().numpy()
        for b, L in enumerate(lens):
            ref = orc.owned_slots(bt[b], L, B, r, C, I)
            got = slots[offs[b]:offs[b + 1]]
            assert np.array_equal(got, ref), f"{label}: rank {r} request {b} slots differ"


@pytest.mark.parametrize("w", list(wl.WORKLOADS.values()), ids=list(wl.WORKLOADS))
def test_slots_bit_exact_workloads(gpu_lib, w):
    """The walk the kernels use, exported, equals the oracle's filter over every position,
    for every rank of every workload's real block table."""
    print(f"[slots] {w.name}", flush=True)
    lens = w.seq_lens()
    B = w.block_size
    pages = [(int(n) + B - 1) // B for n in lens]
    nb = sum(pages)
    rng = np.random.default_rng(w.seed)
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((w.batch, max(pages)), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    _slots_case(bt, [int(x) for x in lens], B, nb, w.cp_size, w.interleave, w.name)


@pytest.mark.parametrize("B,C,I,lens", [
    (16, 2, 4, [1, 7, 16, 17, 100]),        # I < B
    (16, 3, 24, [1, 48, 95, 500]),          # B does not divide I
    (12, 2, 8, [1, 24, 25, 300]),           # I does not divide B
    (8, 4, 8, [32, 64, 96]),                # L = 0 mod I C
    (4, 5, 7, [1, 2, 3, 34, 35, 36]),
    (64, 8, 64, [1, 63, 64, 65, 511, 512, 513]),
    (1, 3, 5, [1, 2, 15, 16, 301]),         # one token per page
    (16, 64, 1, [1, 63, 64, 65, 200]),      # many ranks, most shards of short requests empty
    (128, 4, 100000, [1, 5000, 70000]),     # an interleave longer than every sequence
    (1024, 2, 1024, [1, 1024, 1025, 3000]), # large pages
])
def test_slots_bit_exact_edges(gpu_lib, B, C, I, lens):
    rng = np.random.default_rng(B * 100 + C * 10 + I)
    pages = [(n + B - 1) // B for n in lens]
    nb = sum(pages) + 3
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(lens), max(pages)), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    _slots_case(bt, lens, B, nb, C, I, f"B={B} C={C} I={I}")


ERR_CASES = [
    # (workload, rank, cp_size, interleave): page-contiguous and token-granular tiles of the
    # bf16 GQA, fp8 GQA and MLA kernels
    (wl.GQA_SHARE.with_(batch=2, lengths=(300, 200), seed=31), 0, 1, 128),
    (wl.GQA_SHARE.with_(batch=2, lengths=(300, 200), seed=31), 1, 2, 1),
    (wl.GQA_SHARE_FP8.with_(batch=2, lengths=(300, 200), seed=34), 0, 1, 128),
    (wl.GQA_SHARE_FP8.with_(batch=2, lengths=(300, 200), seed=34), 1, 2, 1),
    (wl.MLA_DECODE.with_(batch=2, lengths=(300, 200), seed=35), 0, 1, 64),
    (wl.MLA_DECODE.with_(batch=2, lengths=(300, 200), seed=35), 1, 2, 1),
]


def _check_survivors(inp, kind, bt, lens, rank, cp, il, scale, o, l, what):
    """Each request's partial against the oracle over its surviving tokens: owned by the
    rank, below min(seq_len, what the table row covers), on a page id inside the cache."""
    B = (inp["k_pages"].shape[2] if kind == dca.GQA else inp["latent_pages"].shape[1])
    bt_h = bt.cpu().numpy()
    num_blocks = inp["num_blocks"]
    o = o.cpu().numpy()
    l = l.cpu().numpy()
    tol = o_tol(kind, inp["q"].dtype)
    for b in range(bt_h.shape[0]):
        L = min(int(lens[b]), bt_h.shape[1] * B)
        t = orc.owned_tokens(L, rank, cp, il)
        pg = bt_h[b][t // B]
        t = t[(pg >= 0) & (pg < num_blocks)]
        good = inp["block_table"][b].cpu().numpy()
        # the surviving tokens' pages are the same in bt and in the input table
        assert np.array_equal(bt_h[b][t // B], good[t // B])
        o_ref, l_ref = oracle_tokens(inp, kind, b, t, scale)
        assert_close(l[b], l_ref, TOL_F32, f"{what}: b={b} lse")
        assert_close(o[b], o_ref, tol, f"{what}: b={b} O")
        assert_rel_l2(o[b], o_ref, o_rel_l2(inp["q"].dtype), f"{what}: b={b} O")


@pytest.mark.parametrize("w,rank,cp,il", ERR_CASES,
                         ids=["gqa", "gqa_i1", "gqa_fp8", "gqa_fp8_i1", "mla", "mla_i1"])
def test_device_error_word(gpu_lib, w, rank, cp, il):
    """Contract violations only the device sees are flagged, never fault, and leave the
    remaining tokens' attention intact: every request's partial equals the oracle's
    attention over the rank's tokens that lie inside the block table and on valid pages."""
    print(f"[deverr] {w.name} rank={rank} cp={cp} il={il}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    kw = dict(kind=kind, k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"))
    bt = inp["block_table"].clone()
    # request 1 claims more tokens than its block-table row covers
    lens = inp["seq_lens"].clone()
    lens[1] = bt.shape[1] * w.block_size + 50
    o, l, ws = dca.shard(inp["q"], kv, v, bt, lens, rank, cp, il, w.scale, **kw)
    assert dca.read_device_errors(ws) & dca.DEVERR_SEQ_LEN
    assert torch.isfinite(o).all() and torch.isfinite(l).all()
    _check_survivors(inp, kind, bt, lens, rank, cp, il, w.scale, o, l, "seq_len past table")
    # a block id outside the cache (logical page 1 of request 0; its other pages remain)
    bt2 = inp["block_table"].clone()
    bt2[0, 1] = 10 ** 6
    o, l, ws = dca.shard(inp["q"], kv, v, bt2, inp["seq_lens"], rank, cp, il, w.scale,
                         workspace=ws, **kw)
    assert dca.read_device_errors(ws) & dca.DEVERR_BLOCK_ID
    assert torch.isfinite(o).all() and torch.isfinite(l).all()
    _check_survivors(inp, kind, bt2, inp["seq_lens"], rank, cp, il, w.scale, o, l,
                     "block id outside the cache")
    # a clean call clears the word
    dca.shard(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], rank, cp, il, w.scale,
              workspace=ws, **kw)
    assert dca.read_device_errors(ws) == 0


def test_shard_is_deterministic(gpu_lib):
    w = wl.MLA_DECODE.with_(batch=2, lengths=(3000, 777), seed=41)
    inp = wl.make_inputs(w, device="cuda")
    a = dca.shard(inp["q"], inp["latent_pages"], None, inp["block_table"], inp["seq_lens"], 1,
                  8, 64, w.scale)
    b = dca.shard(inp["q"], inp["latent_pages"], None, inp["block_table"], inp["seq_lens"], 1,
                  8, 64, w.scale)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_argument_errors_launch_nothing(gpu_lib):
    w = wl.TINY_GQA
    inp = wl.make_inputs(w, device="cuda")
    with pytest.raises(dca.DCPError):
        dca.shard(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                  2, 2, 16, w.scale)   # rank >= cp_size
    with pytest.raises(dca.DCPError):
        dca.shard(inp["q"], inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                  0, 2, 0, w.scale)    # interleave 0

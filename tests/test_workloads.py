"""The seeded input generators: shapes, determinism and the ragged-length recipe (CPU)."""
import math

import numpy as np
import torch

from decode_attention_context_amd import workloads as wl
from oracle import dcp_oracle as orc


def test_small_inputs_shapes_and_determinism():
    w = wl.TINY_GQA
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    assert a["q"].shape == (1, 8, 64) and a["q"].dtype == torch.float32
    assert a["k_pages"].shape == (64, 2, 16, 64)
    assert torch.equal(a["k_pages"], b["k_pages"]) and torch.equal(a["q"], b["q"])
    bt = a["block_table"].numpy()
    assert sorted(bt[0].tolist()) == list(range(64))         # a permutation of the pages
    m = wl.make_inputs(wl.MLA_DECODE.with_(batch=2, lengths=(100, 65)))
    assert m["latent_pages"].shape == (4, 64, 576) and m["q"].shape == (2, 128, 576)
    assert m["block_table"][1, 1].item() >= 0 and m["block_table"][1].shape[0] == 2


def test_ragged_recipe():
    lens = wl.MLA_RAGGED.seq_lens()
    assert lens.shape == (512,) and lens.min() >= 1 and lens.max() <= 262144
    for e in wl.RAGGED_EDGE_LENGTHS:
        assert e in lens
    # lognormal around the trace median (about 67k) with sigma 0.8
    rest = np.setdiff1d(np.arange(512), [int(np.where(lens == e)[0][0]) for e in wl.RAGGED_EDGE_LENGTHS])
    z = np.log(lens[rest]) - math.log(67000)
    assert abs(np.median(z)) < 0.15 and 0.65 < z.std() < 0.95
    # short requests leave some of the 8 shards empty
    empties = sum(orc.owned_count(int(L), r, 8, 64) == 0 for L in lens for r in range(8))
    assert empties > 0


def test_workload_shards_match_the_pages_shapes():
    # per-rank shard of each workload
    assert orc.owned_count(32768, 0, 2, 128) == 16384
    assert orc.owned_count(67584, 5, 8, 64) == 8448
    assert [orc.owned_count(200000, r, 4, 128) for r in range(4)] == [50048, 50048, 49984, 49920]

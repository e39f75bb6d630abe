"""Seeded random parity sweep against the CPU oracle (GPU).

Each case draws a kernel (bf16 GQA, fp32 GQA, GQA over an fp8 cache, MLA), a group size
(any with q_len * G <= 64, non-powers of two included),
KV heads, q_len, cp_size, interleave, block size and ragged lengths (with edge values:
1, a block, a block + 1, an interleave period) from its own seed, runs every rank's shard
and the merge, and compares them elementwise with the oracle (tolerances in
parity_helpers).  Three classes: small, wide (longer sequences, more KV heads) and extreme
(odd block sizes from 1 to 1024 tokens, up to 64 ranks, interleaves past every sequence).
The draws are fixed by the seeds, so a failure names its case.
"""
import numpy as np
import pytest

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from parity_helpers import check_requests, run_shards

pytestmark = pytest.mark.gpu


def _draw(seed, wide=False):
    """wide: longer sequences (to 20000 tokens, items of many tiles), batches to 6, blocks to
    256, interleaves to 512, up to 8 KV heads."""
    rng = np.random.default_rng(seed)
    kind = ["gqa_bf16", "gqa_f32", "gqa_fp8", "mla"][seed % 4]
    q_len = int(rng.integers(1, 5))
    block = int(rng.choice([16, 32, 64, 128, 256] if wide else [16, 32, 64, 128]))
    cp = int(rng.integers(1, 9))
    il = int(rng.choice([1, 2, 3, 7, 16, 32, 64, 96, 128, 256, 512] if wide else
                        [1, 2, 3, 16, 32, 64, 100, 128, 256]))
    batch = int(rng.integers(1, 7 if wide else 4))
    edges = [1, block, block + 1, il * cp, il * cp + 1] + ([2, 4096, 8193] if wide else [])
    lengths = tuple(int(rng.choice(edges)) if rng.random() < 0.3 else
                    int(rng.integers(1, 20000 if wide else 2500)) for _ in range(batch))
    if kind == "mla":
        heads = int(rng.choice([16, 32, 64, 128]))
        return wl.MLA_DECODE.with_(name=f"rand{seed}_mla", batch=batch, q_len=q_len,
                                   num_q_heads=heads,
                                   block_size=block, cp_size=cp, interleave=il,
                                   lengths=lengths, seed=seed)
    hkv = int(rng.choice([1, 2, 4, 8] if wide else [1, 2, 4]))
    # every group the GQA kernels take: q_len * G <= 64 rows per KV head
    groups = [g for g in (1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 21, 32, 64) if g * q_len <= 64]
    g = int(rng.choice(groups))
    base = wl.TINY_GQA if kind == "gqa_f32" else (wl.GQA_SHARE_FP8 if kind == "gqa_fp8"
                                                   else wl.GQA_SHARE)
    return base.with_(name=f"rand{seed}_{kind}", batch=batch, q_len=q_len,
                      num_q_heads=g * hkv, num_kv_heads=hkv, block_size=block, cp_size=cp,
                      interleave=il, lengths=lengths, seed=seed)


def _draw_extreme(seed):
    """Extreme layouts: blocks of 1 to 1024 tokens (odd sizes included), up to 64 ranks,
    interleaves to 70000 (past every sequence), batches to 8, up to 16 KV heads."""
    rng = np.random.default_rng(seed)
    kind = ["gqa_bf16", "gqa_f32", "gqa_fp8", "mla"][seed % 4]
    q_len = int(rng.integers(1, 5))
    block = int(rng.choice([1, 3, 5, 16, 48, 64, 100, 128, 512, 1024]))
    cp = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 32, 64]))
    il = int(rng.choice([1, 2, 5, 31, 64, 100, 128, 1000, 70000]))
    batch = int(rng.integers(1, 9))
    top = 12000 if kind == "mla" else 30000
    edges = [1, 2, block, block + 1, il, il + 1, min(il * cp, top), min(il * cp + 1, top), q_len]
    lengths = tuple(int(rng.choice(edges)) if rng.random() < 0.35 else
                    int(rng.integers(1, top)) for _ in range(batch))
    if kind == "mla":
        heads = int(rng.choice([16, 32, 64, 128]))
        return wl.MLA_DECODE.with_(name=f"ext{seed}_mla", batch=batch, q_len=q_len,
                                   num_q_heads=heads, block_size=block, cp_size=cp,
                                   interleave=il, lengths=lengths, seed=seed)
    hkv = int(rng.choice([1, 2, 4, 8, 16]))
    groups = [g for g in (1, 2, 3, 5, 7, 8, 11, 16, 24, 32, 48, 64) if g * q_len <= 64]
    g = int(rng.choice(groups))
    base = wl.TINY_GQA if kind == "gqa_f32" else (wl.GQA_SHARE_FP8 if kind == "gqa_fp8"
                                                   else wl.GQA_SHARE)
    return base.with_(name=f"ext{seed}_{kind}", batch=batch, q_len=q_len, num_q_heads=g * hkv,
                      num_kv_heads=hkv, block_size=block, cp_size=cp, interleave=il,
                      lengths=lengths, seed=seed)


SEEDS = list(range(2000, 2096))


WIDE_SEEDS = list(range(5000, 5048))


EXTREME_SEEDS = list(range(9000, 9024))


def _check(w):
    print(f"[rand] {w.name}: q_len={w.q_len} batch={w.batch} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} C={w.cp_size} I={w.interleave} B={w.block_size} "
          f"lengths={w.lengths}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    o_parts, l_parts = run_shards(inp, kind, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    check_requests(inp, kind, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   list(range(w.batch)), w.name)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case(gpu_lib, seed):
    _check(_draw(seed))


@pytest.mark.parametrize("seed", WIDE_SEEDS)
def test_random_wide_case(gpu_lib, seed):
    _check(_draw(seed, wide=True))


@pytest.mark.parametrize("seed", EXTREME_SEEDS)
def test_random_extreme_case(gpu_lib, seed):
    _check(_draw_extreme(seed))

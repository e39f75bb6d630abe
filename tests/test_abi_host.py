"""CPU-side tests of the C-ABI library: it loads, exports every symbol include/dcp_attn.h
declares, and its host-only functions agree with the oracle.  No GPU call is made."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import decode_attention_context_amd as dca
from oracle import dcp_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcp_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+(dcp_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = dca.load()
    names = _declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in dcp_attn.h but not exported"
    # and nothing declared is missing from the binding's signature table
    assert set(names) <= set(dca._SIGS), set(names) - set(dca._SIGS)


def test_local_len_matches_oracle():
    rng = np.random.default_rng(0)
    for _ in range(300):
        L = int(rng.integers(0, 5000))
        C = int(rng.integers(1, 9))
        I = int(rng.choice([1, 2, 3, 16, 64, 100, 128]))
        for r in range(C):
            assert dca.local_len(L, r, C, I) == orc.owned_count(L, r, C, I)
    # the blog's 200K-token, four-GPU example and the workloads' own shards
    assert [dca.local_len(200000, r, 4, 50000) for r in range(4)] == [50000] * 4
    assert [dca.local_len(200000, r, 4, 128) for r in range(4)] == [50048, 50048, 49984, 49920]
    assert dca.local_len(67584, 3, 8, 64) == 8448
    assert dca.local_len(32768, 1, 2, 128) == 16384


def test_local_len_large_and_invalid():
    lib = dca.load()
    L = 2 ** 31 - 1
    for C, I in [(8, 64), (3, 1000), (1, 1)]:
        tot = sum(lib.dcp_local_len(L, r, C, I) for r in range(C))
        assert tot == L
    assert lib.dcp_local_len(10, 2, 2, 4) == -1      # rank >= cp_size
    assert lib.dcp_local_len(10, 0, 0, 4) == -1
    assert lib.dcp_local_len(10, 0, 2, 0) == -1
    assert lib.dcp_local_len(-1, 0, 2, 4) == -1


def test_check_parallel_matches_page_examples():
    with open(os.path.join(ROOT, "tests", "golden", "dcp_size_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert dca.check_parallel(c["tp"], c["dcp"], c["num_kv_heads"], c["is_mla"]) == c["ok"], c
    for tp in range(1, 17):
        for dcp in range(1, 17):
            for kvh in (1, 2, 4, 8):
                for mla in (0, 1):
                    assert dca.check_parallel(tp, dcp, kvh, mla) == orc.check_parallel(tp, dcp, kvh, mla)


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        s = dca.status_string(code)
        assert s.startswith("DCP_")


def test_argument_errors_are_host_side():
    """Invalid arguments are rejected before any device work (no GPU needed here)."""
    lib = dca.load()
    d = dca.Desc(dca.GQA, dca.BF16, 8, 1, 128, 128, 128, 256, 1024)
    null = ctypes.c_void_p(0)
    args = lambda rank, cp, il, desc=d: (ctypes.byref(desc), null, null, null, null, null, 4,
                                         32768, rank, cp, il, 0.1, null, null, null, 0, null)
    assert lib.dcp_attn_shard(*args(2, 2, 128)) == -1          # rank >= cp_size
    assert lib.dcp_attn_shard(*args(0, 0, 128)) == -1          # cp_size 0
    assert lib.dcp_attn_shard(*args(0, 2, 0)) == -1            # interleave 0
    assert lib.dcp_attn_shard(*args(0, 2, 128)) == -1          # null pointers
    bad = dca.Desc(dca.GQA, dca.BF16, 8, 3, 128, 128, 128, 256, 1024)     # Hq % Hkv != 0
    assert lib.dcp_attn_shard(*args(0, 2, 128, bad)) == -1
    uns = dca.Desc(dca.GQA, dca.BF16, 8, 1, 96, 96, 128, 256, 1024)       # head dim 96
    assert lib.dcp_attn_shard(*args(0, 2, 128, uns)) == -2
    mla_bad = dca.Desc(dca.MLA, dca.BF16, 96, 1, 576, 512, 64, 256, 1024)  # 96 heads
    assert lib.dcp_attn_shard(*args(0, 2, 64, mla_bad)) == -2
    assert lib.dcp_merge(null, null, 0, 1, 1, 1, null, 0, null, null) == -1
    assert lib.dcp_merge(null, null, 2, 1, 1, 1, null, 5, null, null) == -1
    assert lib.dcp_shard_slots(null, null, 1, 1, 16, 1, 3, 2, 16, null, null, null, null) == -1

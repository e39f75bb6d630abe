"""The GQA shape contract of include/dcp_attn.h, walked through the C ABI (GPU).

Supported: bf16 with head_dim 128 or f32 with head_dim 64, and any group G = Hq / Hkv with
q_len * G <= 64 query rows per KV head ("GQA backend" of the blog names the Qwen3 and Llama
families, whose groups include 3, 5, 6 and 7).  Every supported (dtype, G, q_len) runs a
small ragged two-rank case checked against the oracle (every request, rank and head, and
the merge), for bf16 and f32 caches and for an fp8 cache (bf16 queries); every unsupported
(dtype, head_dim, G, q_len) must return DCP_EUNSUPPORTED from dcp_attn_shard_mq without
launching (the outputs keep their sentinel values)."""
import ctypes

import pytest
import torch

import decode_attention_context_amd as dca
from decode_attention_context_amd import workloads as wl
from parity_helpers import check_requests, run_shards

pytestmark = pytest.mark.gpu

GROUPS = (1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 21, 24, 32, 48, 64)
SUPPORTED_D = {"bf16": 128, "f32": 64}


def supported(dtype, d, g, q_len):
    return SUPPORTED_D[dtype] == d and 1 <= q_len <= 4 and g * q_len <= 64


CASES = [(dt, g, ql) for dt in ("bf16", "f32") for g in GROUPS for ql in (1, 2, 3, 4)
         if supported(dt, SUPPORTED_D[dt], g, ql)]


@pytest.mark.parametrize("dtype,g,q_len", CASES,
                         ids=[f"{dt}-g{g}-q{ql}" for dt, g, ql in CASES])
def test_supported_shape_parity(gpu_lib, dtype, g, q_len):
    hkv = 2 if g <= 8 else 1
    base = wl.GQA_SHARE if dtype == "bf16" else wl.TINY_GQA
    w = base.with_(name=f"shape_{dtype}_g{g}_q{q_len}", batch=2, num_q_heads=g * hkv,
                   num_kv_heads=hkv, block_size=16, cp_size=2, interleave=16,
                   lengths=(q_len + 1, 700), q_len=q_len, seed=300 + g * 8 + q_len)
    print(f"[shapes] {w.name}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    o_parts, l_parts = run_shards(inp, dca.GQA, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    check_requests(inp, dca.GQA, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   range(w.batch), w.name)


FP8_CASES = [(g, ql) for g in (3, 5, 7, 12, 21, 32, 64) for ql in (1, 2, 3, 4) if g * ql <= 64]


@pytest.mark.parametrize("g,q_len", FP8_CASES, ids=[f"fp8-g{g}-q{ql}" for g, ql in FP8_CASES])
def test_supported_shape_parity_fp8_cache(gpu_lib, g, q_len):
    """The fp8 KV cache takes the same group contract (bf16 queries, head_dim 128)."""
    hkv = 2 if g <= 8 else 1
    w = wl.GQA_SHARE_FP8.with_(name=f"shape_fp8_g{g}_q{q_len}", batch=2, num_q_heads=g * hkv,
                               num_kv_heads=hkv, block_size=16, cp_size=2, interleave=16,
                               lengths=(q_len + 1, 700), q_len=q_len, seed=500 + g * 8 + q_len)
    print(f"[shapes] {w.name}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    o_parts, l_parts = run_shards(inp, dca.GQA, w.cp_size, w.interleave, w.scale)
    o_m, l_m = dca.merge(o_parts, l_parts)
    torch.cuda.synchronize()
    check_requests(inp, dca.GQA, w.cp_size, w.interleave, w.scale, o_parts, l_parts, o_m, l_m,
                   range(w.batch), w.name)


UNSUPPORTED = [(dt, d, g, ql) for dt in ("bf16", "f32") for d in (32, 64, 96, 128, 256)
               for g in (1, 3, 8, 16, 32, 65) for ql in (1, 2, 3, 5)
               if not supported(dt, d, g, ql)]


def test_unsupported_shapes_refused_without_launch(gpu_lib):
    lib = dca.load()
    print(f"[shapes] {len(UNSUPPORTED)} unsupported shapes", flush=True)
    for dt, d, g, ql in UNSUPPORTED:
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        batch, hkv, bs = 2, 1, 16
        q = torch.zeros(batch, ql, g * hkv, d, dtype=tdt, device="cuda")
        k = torch.zeros(4, hkv, bs, d, dtype=tdt, device="cuda")
        bt = torch.zeros(batch, 2, dtype=torch.int32, device="cuda")
        lens = torch.full((batch,), 20, dtype=torch.int32, device="cuda")
        o = torch.full((batch, ql, g * hkv, d), 7.0, dtype=torch.float32, device="cuda")
        lse = torch.full((batch, ql, g * hkv), 7.0, dtype=torch.float32, device="cuda")
        ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
        desc = dca.Desc(dca.GQA, dca.BF16 if dt == "bf16" else dca.F32, g * hkv, hkv, d, d, bs,
                        2, 4)
        st = lib.dcp_attn_shard_mq(ctypes.byref(desc), ql, ctypes.c_void_p(q.data_ptr()),
                                   ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                   ctypes.c_void_p(bt.data_ptr()),
                                   ctypes.c_void_p(lens.data_ptr()), batch, 32, 0, 2, 16, 0.1,
                                   ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                                   ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == -2, (dt, d, g, ql, st)
        assert lib.dcp_workspace_size_mq(ctypes.byref(desc), ql, batch, 32, 2, 16) == 0
    torch.cuda.synchronize()
    # nothing was launched: the sentinels of the last call are intact
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)

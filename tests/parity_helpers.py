"""Shared helpers of the GPU parity tests: run the HIP path through the binding, fetch the
exact inputs a request used, and compare against the CPU oracle elementwise.

Tolerances (written here once, used by every parity test):
  * outputs O computed from bf16 inputs: |x - x*| <= 2e-2 + 2e-2 |x*|
  * outputs O computed from fp32 inputs, and every LSE: |x - x*| <= 1e-3 + 1e-3 |x*|
  * an LSE of -inf (empty shard) must be exactly -inf, and its O exactly 0
  * the index mapping (physical slots of a rank's tokens) must be bit-exact
  * on top of the elementwise gate, every O row (one head of one partial or of the merged
    output) must satisfy ||x - x*||_2 <= REL_L2 * ||x*||_2: 1e-2 for bf16-input outputs
    (the kernels round P to bf16, about 2e-3, and bf16 outputs or split partials add about
    1e-3 each), 1e-3 for fp32-input outputs.  At long context |O| is small against the
    elementwise absolute term, so this is the gate that sees a dropped or doubled share of
    the tokens (dropping 1/8 of them moves a row by about 0.35 in relative L2).
"""
import math

import numpy as np
import torch

import decode_attention_context_amd as dca
from oracle import dcp_oracle as orc

TOL_BF16_O = (2e-2, 2e-2)
TOL_F32 = (1e-3, 1e-3)
REL_L2_BF16 = 1e-2
REL_L2_F32 = 1e-3


def row_errors(got, ref):
    """Per-row error figures of O over its last axis: (max abs, relative L2) for every row
    whose reference is not all zero (rows of empty shards are checked exactly elsewhere)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    rn = np.linalg.norm(r, axis=1)
    keep = rn > 0
    d = g[keep] - r[keep]
    return np.abs(d).max(axis=1), np.linalg.norm(d, axis=1) / rn[keep]


def assert_rel_l2(got, ref, bound, what):
    _, rl2 = row_errors(got, ref)
    if rl2.size and not np.all(rl2 <= bound):
        i = int(np.argmax(rl2))
        raise AssertionError(f"{what}: row relative L2 error {float(rl2[i]):.3e} > {bound:.0e} "
                             f"(row {i} of {rl2.size})")


def assert_close(got, ref, tol, what):
    atol, rtol = tol
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    ninf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf_ref), f"{what}: -inf pattern differs"
    fin = ~ninf_ref
    assert np.all(np.isfinite(got[fin])), f"{what}: non-finite values"
    err = np.abs(got[fin] - ref[fin])
    bound = atol + rtol * np.abs(ref[fin])
    if err.size and not np.all(err <= bound):
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: max excess {float((err - bound)[i]):.3e} "
                             f"(err {float(err[i]):.3e}, ref {float(ref[fin][i]):.4f}); "
                             f"max abs err {float(err.max()):.3e}")


def o_tol(kind, dtype):
    return TOL_BF16_O if dtype == torch.bfloat16 else TOL_F32


def o_rel_l2(dtype):
    return REL_L2_BF16 if dtype == torch.bfloat16 else REL_L2_F32


def run_shards(inp, kind, cp_size, interleave, scale, ranks=None):
    """Every rank's (O_r, lse_r) on the GPU, stacked: [C, b, H, Dv], [C, b, H]."""
    q = inp["q"]
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    os_, ls_ = [], []
    ws = None
    for r in (range(cp_size) if ranks is None else ranks):
        o, l, ws = dca.shard(q, kv, v, inp["block_table"], inp["seq_lens"], r, cp_size,
                             interleave, scale, kind=kind, max_seq_len=inp["max_seq_len"],
                             workspace=ws, k_scale=inp.get("k_scale"),
                             v_scale=inp.get("v_scale"))
        os_.append(o)
        ls_.append(l)
        assert dca.read_device_errors(ws) == 0
    return torch.stack(os_), torch.stack(ls_)


def request_host(inp, kind, b):
    """Exact float64 copies of what request b reads: its query, its pages (compacted) and a
    block-table row that addresses the compact copy."""
    L = int(inp["seq_lens"][b].item())
    bt = inp["block_table"]
    if kind == dca.GQA:
        B = inp["k_pages"].shape[2]
    else:
        B = inp["latent_pages"].shape[1]
    npages = (L + B - 1) // B
    pages = bt[b, :npages].long()
    q = inp["q"][b].float().cpu().numpy().astype(np.float64)
    row = np.arange(npages, dtype=np.int64)
    if kind == dca.GQA:
        if inp["k_pages"].dtype == torch.uint8:   # fp8 cache: the values its codes stand for
            k = orc.fp8_kv_values(inp["k_pages"][pages].cpu().numpy(), inp["k_scale"])
            v = orc.fp8_kv_values(inp["v_pages"][pages].cpu().numpy(), inp["v_scale"])
        else:
            k = inp["k_pages"][pages].float().cpu().numpy().astype(np.float64)
            v = inp["v_pages"][pages].float().cpu().numpy().astype(np.float64)
        return dict(q=q, k=k, v=v, row=row, L=L, B=B)
    lat = inp["latent_pages"][pages].float().cpu().numpy().astype(np.float64)
    return dict(q=q, lat=lat, row=row, L=L, B=B)


def oracle_shard(h, kind, rank, cp_size, interleave, scale):
    """One request's rank partial; a [q_len, Hq, D] query is multi-token decode."""
    mq = h["q"].ndim == 3
    if kind == dca.GQA:
        f = orc.gqa_shard_mq if mq else orc.gqa_shard
        return f(h["q"], h["k"], h["v"], h["row"], h["L"], rank, cp_size, interleave, scale,
                 h["B"])
    f = orc.mla_shard_mq if mq else orc.mla_shard
    return f(h["q"], h["lat"], h["row"], h["L"], rank, cp_size, interleave, scale, h["B"])


def oracle_full(h, kind, scale):
    mq = h["q"].ndim == 3
    if kind == dca.GQA:
        f = orc.gqa_full_mq if mq else orc.gqa_full
        return f(h["q"], h["k"], h["v"], h["row"], h["L"], scale, h["B"])
    f = orc.mla_full_mq if mq else orc.mla_full
    return f(h["q"], h["lat"], h["row"], h["L"], scale, h["B"])


def oracle_tokens(inp, kind, b, tokens, scale):
    """Oracle attention of request b's query over an explicit set of its global token
    positions (pages looked up in the input block table): for calls where some tokens must
    be skipped, e.g. those of a page id outside the cache."""
    tokens = np.asarray(tokens, dtype=np.int64)
    kvp = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    B = kvp.shape[2] if kind == dca.GQA else kvp.shape[1]
    pages = inp["block_table"][b].long().cpu().numpy()[tokens // B]
    pg = torch.from_numpy(pages).to(kvp.device)
    sl = torch.from_numpy(tokens % B).to(kvp.device)
    q = inp["q"][b].float().cpu().numpy().astype(np.float64)
    if kind == dca.GQA:
        k = inp["k_pages"][pg, :, sl, :]
        v = inp["v_pages"][pg, :, sl, :]
        if k.dtype == torch.uint8:
            k = orc.fp8_kv_values(k.cpu().numpy(), inp["k_scale"])
            v = orc.fp8_kv_values(v.cpu().numpy(), inp["v_scale"])
        else:
            k = k.float().cpu().numpy().astype(np.float64)
            v = v.float().cpu().numpy().astype(np.float64)
        return orc.attend(q, k, v, scale)
    rows = inp["latent_pages"][pg, sl, :].float().cpu().numpy().astype(np.float64)
    return orc.attend(q, rows[:, None, :], rows[:, None, :orc.MLA_DV], scale)


def check_requests(inp, kind, cp_size, interleave, scale, o_parts, l_parts, o_merged,
                   l_merged, requests, label):
    """Compare every rank's partial and the merged output of the sampled requests:
    elementwise, and by relative L2 per head row."""
    tol = o_tol(kind, inp["q"].dtype)
    rl2 = o_rel_l2(inp["q"].dtype)
    o_parts = o_parts.cpu().numpy()
    l_parts = l_parts.cpu().numpy()
    o_merged = o_merged.cpu().numpy()
    l_merged = l_merged.cpu().numpy()
    for b in requests:
        h = request_host(inp, kind, b)
        for r in range(cp_size):
            o_ref, l_ref = oracle_shard(h, kind, r, cp_size, interleave, scale)
            assert_close(l_parts[r, b], l_ref, TOL_F32, f"{label} b={b} rank={r} lse")
            assert_close(o_parts[r, b], o_ref, tol, f"{label} b={b} rank={r} O")
            assert_rel_l2(o_parts[r, b], o_ref, rl2, f"{label} b={b} rank={r} O")
            empty = np.isneginf(l_ref)
            assert np.all(o_parts[r, b][empty] == 0), f"{label} b={b} rank={r}: empty row O != 0"
        o_ref, l_ref = oracle_full(h, kind, scale)
        assert_close(l_merged[b], l_ref, TOL_F32, f"{label} b={b} merged lse")
        assert_close(o_merged[b], o_ref, tol, f"{label} b={b} merged O")
        assert_rel_l2(o_merged[b], o_ref, rl2, f"{label} b={b} merged O")


def scale_of(d):
    return 1.0 / math.sqrt(d)

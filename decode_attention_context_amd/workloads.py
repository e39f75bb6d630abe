"""Seeded synthetic inputs for DCP shard attention and the LSE merge.

This module only builds inputs: query tensors, paged KV caches, block tables and
sequence lengths.  It holds none of the attention or merge arithmetic, so both the HIP
path and the CPU oracle can be fed from it without sharing any of the method's code.

Workloads follow the shapes of the decode-context-parallel pages: a small GQA case, a
GQA per-GPU share shaped like Qwen3-235B, MLA decode shaped like DeepSeek-V3 / Kimi
(128 gathered heads, 576-wide latent key, 512-wide value), a 200K-token MLA case and a
ragged batch whose lengths are lognormal around the agentic trace's median of about 67k
input tokens.  The trace itself is not available; the lognormal lengths stand in for it.

Queries: [batch][Hq][Dk], or [batch][q_len][Hq][Dk] for multi-token decode (q_len > 1:
the request's last q_len cache tokens are its draft tokens, each verified by one query row).
Cache layouts:
  GQA  k_pages, v_pages: [num_blocks][Hkv][block_size][D]   (fp32 or bf16; or uint8 fp8
       codes with k_scale / v_scale when kv_dtype is "fp8")
  MLA  latent_pages:     [num_blocks][block_size][576]      (bf16)
  block_table: int32 [batch][max_blocks_per_seq], physical page per logical page,
               padded with -1;  seq_lens: int32 [batch], global context lengths.
Physical pages are a seeded random permutation, so consecutive logical pages of a
sequence land on scattered physical pages.
"""

from dataclasses import dataclass, field, replace
import math

import numpy as np
import torch

MLA_DK = 576
MLA_DV = 512
MLA_HEADS = 128

# Edge lengths overwritten into the ragged batch so that some shards are empty or hold a
# single token, whatever the lognormal draw gives.
RAGGED_EDGE_LENGTHS = (1, 2, 63, 64, 65, 127, 128, 129, 447, 448, 449, 511, 512, 513,
                       4096, 262144)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "gqa" or "mla"
    dtype: str                # "f32" or "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    block_size: int
    cp_size: int
    interleave: int
    scale: float
    seed: int
    seq_len: int = 0          # fixed length for every request (0: use `lengths`)
    lengths: tuple = field(default=())
    ragged: dict = field(default=None)   # lognormal recipe, see ragged_lengths()
    q_len: int = 1            # query positions per request (multi-token decode when > 1)
    kv_dtype: str = ""        # "" = dtype; "fp8": GQA K / V pages of OCP FP8 E4M3 codes
    kv_scales: tuple = (0.5, 0.25)   # fp8 cache: (k_scale, v_scale), value = code * scale

    def seq_lens(self):
        if self.ragged is not None:
            return ragged_lengths(self.batch, **self.ragged)
        if self.lengths:
            assert len(self.lengths) == self.batch
            return np.asarray(self.lengths, dtype=np.int64)
        return np.full(self.batch, self.seq_len, dtype=np.int64)

    def with_(self, **kw):
        return replace(self, **kw)


def ragged_lengths(batch, median, sigma, lo, hi, seed, edges=RAGGED_EDGE_LENGTHS):
    """Lognormal lengths: L = clip(rint(exp(ln median + sigma z)), lo, hi) with z from
    numpy's default_rng(seed); then `edges` overwrite len(edges) seeded positions."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(batch)
    lens = np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)
    if edges:
        pos = rng.choice(batch, size=min(len(edges), batch), replace=False)
        lens[pos] = np.asarray(edges[:len(pos)], dtype=np.int64)
    return lens


def _scale(d):
    return 1.0 / math.sqrt(d)


# The five workloads of the pages' shapes (tiny GQA, GQA share, MLA, long MLA, ragged MLA).
TINY_GQA = Workload("tiny_gqa_fp32", "gqa", "f32", batch=1, num_q_heads=8, num_kv_heads=2,
                    head_dim_qk=64, head_dim_v=64, block_size=16, cp_size=2, interleave=16,
                    scale=_scale(64), seed=1001, seq_len=1024)
GQA_SHARE = Workload("gqa_qwen3_235b_share", "gqa", "bf16", batch=64, num_q_heads=8,
                     num_kv_heads=1, head_dim_qk=128, head_dim_v=128, block_size=128,
                     cp_size=2, interleave=128, scale=_scale(128), seed=1002,
                     seq_len=32768)
MLA_DECODE = Workload("mla_deepseek_v3_decode", "mla", "bf16", batch=64,
                      num_q_heads=MLA_HEADS, num_kv_heads=1, head_dim_qk=MLA_DK,
                      head_dim_v=MLA_DV, block_size=64, cp_size=8, interleave=64,
                      scale=_scale(192), seed=1003, seq_len=67584)
MLA_LONG = Workload("mla_long_200k", "mla", "bf16", batch=8, num_q_heads=MLA_HEADS,
                    num_kv_heads=1, head_dim_qk=MLA_DK, head_dim_v=MLA_DV, block_size=64,
                    cp_size=4, interleave=128, scale=_scale(192), seed=1004,
                    seq_len=200000)
MLA_RAGGED = Workload("mla_ragged_512", "mla", "bf16", batch=512, num_q_heads=MLA_HEADS,
                      num_kv_heads=1, head_dim_qk=MLA_DK, head_dim_v=MLA_DV, block_size=64,
                      cp_size=8, interleave=64, scale=_scale(192), seed=1005,
                      ragged=dict(median=67000, sigma=0.8, lo=1, hi=262144, seed=1005))

# the GQA share with its K / V cache in fp8 (the lower-byte cache variant)
GQA_SHARE_FP8 = replace(GQA_SHARE, name="gqa_qwen3_235b_share_fp8kv", kv_dtype="fp8")
WORKLOADS = {w.name: w for w in (TINY_GQA, GQA_SHARE, MLA_DECODE, MLA_LONG, MLA_RAGGED,
                                 GQA_SHARE_FP8)}


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _fill_normal(t, gen, chunk_elems=1 << 28):
    """Fill `t` with N(0,1) draws in its own dtype, chunk by chunk (bounded scratch)."""
    flat = t.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        flat[s:s + chunk_elems].normal_(generator=gen)
    return t


def _fill_fp8(shape, gen, scale, device, chunk_elems=1 << 26):
    """fp8 cache pages: N(0,1) float32 draws divided by `scale`, rounded to OCP FP8 E4M3 by
    torch's float8_e4m3fn conversion (nearest, saturating to the largest finite value is not
    needed: |x| / scale stays far below 448), stored as uint8 codes."""
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        n = min(chunk_elems, flat.numel() - s)
        x = torch.empty(n, dtype=torch.float32, device=device).normal_(generator=gen)
        flat[s:s + n] = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def make_inputs(w, device="cpu", seed=None):
    """Build every input tensor of workload `w` on `device` from its seed."""
    seed = w.seed if seed is None else seed
    lens = w.seq_lens()
    bsz = w.block_size
    pages_per_seq = [(int(n) + bsz - 1) // bsz for n in lens]
    num_blocks = max(1, sum(pages_per_seq))
    max_blocks = max(1, max(pages_per_seq))
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((w.batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        bt[b, :n] = perm[off:off + n]
        off += n

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = torch_dtype(w.dtype)
    out = dict(block_table=torch.from_numpy(bt).to(device),
               seq_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
               num_blocks=num_blocks, max_blocks_per_seq=max_blocks,
               max_seq_len=int(lens.max()) if len(lens) else 0)
    qshape = (w.batch,) + ((w.q_len,) if w.q_len > 1 else ()) + (w.num_q_heads, w.head_dim_qk)
    if w.kind == "gqa":
        out["q"] = _fill_normal(torch.empty(qshape, dtype=dt, device=device), gen)
        shape = (num_blocks, w.num_kv_heads, bsz, w.head_dim_qk)
        if w.kv_dtype == "fp8":
            ks, vs = w.kv_scales
            out["k_pages"] = _fill_fp8(shape, gen, ks, device)
            out["v_pages"] = _fill_fp8(shape, gen, vs, device)
            out["k_scale"], out["v_scale"] = float(ks), float(vs)
        else:
            out["k_pages"] = _fill_normal(torch.empty(shape, dtype=dt, device=device), gen)
            out["v_pages"] = _fill_normal(torch.empty(shape, dtype=dt, device=device), gen)
    else:
        out["q"] = _fill_normal(torch.empty(qshape, dtype=dt, device=device), gen)
        out["latent_pages"] = _fill_normal(
            torch.empty(num_blocks, bsz, w.head_dim_qk, dtype=dt, device=device), gen)
    return out

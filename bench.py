"""Benchmark of the DCP decode-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: every DCP rank's shard attention
(virtual ranks of one paged cache on this GPU) followed by the LSE merge of their partials,
which yields exact unsharded attention for every request.  The default workload is the
GQA per-GPU share shaped like Qwen3-235B: 64 decode requests x 32768 tokens, 8 query heads
on 1 KV head, head dim 128, bf16 cache in 128-token pages, DCP size 2 with interleave 128.

Printed: one JSON line with the throughput (KV tokens of context attended per second), the
roofline of the dominant kernel (the GQA shard kernel, timed with HIP events recorded on
its own stream around every launch), the CPU oracle timed on a bounded sample of the
same workload, and `accuracy`: the oracle's comparison with sampled requests of every timed
workload, read back from the outputs of the timed launches themselves (both oracle legs
are skipped with --no-cpu-baseline).  `secondary` adds the MLA shard kernel (MFMA utilisation) and the 8-way
merge on the MLA decode workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def _src_hash(name):
    """sha256[:16] of a kernel source together with the headers every kernel includes."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_context_amd", "csrc")
    for path in [os.path.join(csrc, n) for n in (name, "common.h", "launch.h", "host_rules.h",
                                                 "walker.h")] + \
            [os.path.join(ROOT, "include", "dcp_attn.h")]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gqa_kernel_name(w):
    """The GQA shard kernel variant the library launches for workload w."""
    rows = w.q_len * (w.num_q_heads // w.num_kv_heads)
    rt = 1 if rows <= 16 else 2
    if w.kv_dtype == "fp8":
        return f"gqa_fp8_kernel<RT={rt}>"
    if w.dtype == "bf16":
        return f"gqa_shard_kernel<bf16, matrix cores, RT={rt}>"
    return f"gqa_shard_kernel<f32, vector ALUs, {rows} rows>"


def owned_tokens_count(L, rank, cp, il):
    """Tokens of an L-token sequence stored by `rank` (the library's host walker)."""
    import decode_attention_context_amd as dca
    return dca.local_len(L, rank, cp, il)


def owned_pages_count(L, rank, cp, il, bs):
    """Cache pages holding at least one token the rank stores (each block-table entry the
    shard kernel needs)."""
    pages = set()
    g = rank
    while g * il < L:
        lo, hi = g * il, min(g * il + il, L)
        pages.update(range(lo // bs, (hi - 1) // bs + 1))
        g += cp
    return len(pages)


def gqa_launch_bytes(w, lens, rank):
    """Algorithmic HBM bytes of one GQA shard launch: the K and V rows the rank owns, the
    queries, the block-table entries of owned pages, and the O / lse written."""
    elem = 2 if w.dtype == "bf16" else 4
    kv_elem = 1 if w.kv_dtype == "fp8" else elem
    tok = sum(owned_tokens_count(int(L), rank, w.cp_size, w.interleave) for L in lens)
    pages = sum(owned_pages_count(int(L), rank, w.cp_size, w.interleave, w.block_size)
                for L in lens)
    kv = tok * 2 * w.num_kv_heads * w.head_dim_qk * kv_elem
    q = w.batch * w.num_q_heads * w.head_dim_qk * elem
    out = w.batch * w.num_q_heads * (w.head_dim_v + 1) * 4
    return kv + q + out + pages * 4, tok


def mla_launch_cost(w, lens, rank):
    tok = sum(owned_tokens_count(int(L), rank, w.cp_size, w.interleave) for L in lens)
    pages = sum(owned_pages_count(int(L), rank, w.cp_size, w.interleave, w.block_size)
                for L in lens)
    byts = tok * w.head_dim_qk * 2 + w.batch * w.num_q_heads * (w.head_dim_qk * 2 +
                                                                (w.head_dim_v + 1) * 4) + pages * 4
    flops = tok * 2 * w.num_q_heads * (w.head_dim_qk + w.head_dim_v)
    return byts, flops, tok


def load_counters(kernel_key, src_name, workload):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel on this workload,
    if recorded against the current source of the kernel (else None)."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(kernel_key)
    if not e or e.get("source_sha") != _src_hash(src_name) or e.get("workload") != workload:
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, seconds_target=12.0, max_requests=8, max_passes=200):
    """The oracle, as it stands, on the first requests of the same workload: every shard of a
    request plus their merge, in float64 numpy on the host's cores.  The sample is converted
    to float64 once and the passes over it are repeated until about `seconds_target` seconds
    of oracle time have accumulated."""
    import numpy as np
    from oracle import dcp_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    B = w.block_size
    sample = []
    for b in range(min(max_requests, w.batch)):
        L = int(inp["seq_lens"][b].item())
        npages = (L + B - 1) // B
        pages = inp["block_table"][b, :npages].long()
        q = inp["q"][b].float().cpu().numpy().astype(np.float64)
        if w.kind == "gqa":
            kv = (inp["k_pages"][pages].float().cpu().numpy().astype(np.float64),
                  inp["v_pages"][pages].float().cpu().numpy().astype(np.float64))
        else:
            kv = (inp["latent_pages"][pages].float().cpu().numpy().astype(np.float64),)
        sample.append((L, q, kv, np.arange(npages)))
    done_tokens = 0
    passes = 0
    t_total = 0.0
    while passes < max_passes and t_total < seconds_target:
        for L, q, kv, row in sample:
            t0 = time.perf_counter()
            parts = []
            for r in range(w.cp_size):
                if w.kind == "gqa":
                    parts.append(orc.gqa_shard(q, kv[0], kv[1], row, L, r, w.cp_size,
                                               w.interleave, w.scale, B))
                else:
                    parts.append(orc.mla_shard(q, kv[0], row, L, r, w.cp_size, w.interleave,
                                               w.scale, B))
            orc.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            t_total += time.perf_counter() - t0
            done_tokens += L
        passes += 1
    return {"value": done_tokens / t_total, "unit": "KV tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"first {len(sample)} of {w.batch} requests of the same workload, "
                      f"{passes} passes: all {w.cp_size} shard partials + merge of each "
                      f"request in float64 numpy ({t_total:.1f} s of oracle time)"}


def oracle_leg(w, inp, samples):
    """The benchmark's one use of the CPU oracle, after all GPU timing: its own throughput
    on a bounded sample of the workload (cpu_baseline) and its verdict on the kept outputs
    of the timed launches (accuracy)."""
    return cpu_baseline(w, inp), accuracy(samples)


def keep_sample(samples, w, inp, bufs, requests):
    """Host copies of what sampled requests read (query, their pages compacted, a block-table
    row addressing the copy) and of what the timed path wrote for them (every rank's
    partial and the merged output), for the oracle comparison after the timed work."""
    import numpy as np
    if samples is None:
        return
    o_parts, l_parts, o, lse = bufs
    B = w.block_size
    rows = []
    for b in requests:
        L = int(inp["seq_lens"][b].item())
        npages = (L + B - 1) // B
        pages = inp["block_table"][b, :npages].long()
        h = {"b": int(b), "L": L, "row": np.arange(npages),
             "q": inp["q"][b].float().cpu().numpy().astype(np.float64),
             "o_parts": o_parts[:, b].float().cpu().numpy(),
             "l_parts": l_parts[:, b].float().cpu().numpy(),
             "o": o[b].float().cpu().numpy(), "lse": lse[b].float().cpu().numpy()}
        if w.kind == "gqa":
            h["k"] = inp["k_pages"][pages].float().cpu().numpy().astype(np.float64)
            h["v"] = inp["v_pages"][pages].float().cpu().numpy().astype(np.float64)
        else:
            h["lat"] = inp["latent_pages"][pages].float().cpu().numpy().astype(np.float64)
        rows.append(h)
    samples[w.name] = (w, rows)


def accuracy(samples):
    """Error of the timed path's outputs against the oracle on the kept requests, per
    workload: merged O (max abs; max over head rows of max|err| / max|ref|; max over head
    rows and over the whole sample of the relative L2 error), merged LSE (max abs), and the
    largest per-row relative L2 error of any rank's partial O."""
    import numpy as np
    from oracle import dcp_oracle as orc
    out = {}
    for name, (w, rows) in samples.items():
        t0 = time.perf_counter()
        ea = er = el = 0.0
        pl2 = 0.0
        num = den = 0.0
        for h in rows:
            if w.kind == "gqa":
                full = orc.gqa_full(h["q"], h["k"], h["v"], h["row"], h["L"], w.scale,
                                    w.block_size)
                shard = [orc.gqa_shard(h["q"], h["k"], h["v"], h["row"], h["L"], r, w.cp_size,
                                       w.interleave, w.scale, w.block_size)
                         for r in range(w.cp_size)]
            else:
                full = orc.mla_full(h["q"], h["lat"], h["row"], h["L"], w.scale, w.block_size)
                shard = [orc.mla_shard(h["q"], h["lat"], h["row"], h["L"], r, w.cp_size,
                                       w.interleave, w.scale, w.block_size)
                         for r in range(w.cp_size)]
            o_ref, l_ref = full
            d = h["o"] - o_ref
            ea = max(ea, float(np.abs(d).max()))
            rn = np.linalg.norm(o_ref, axis=-1)
            m = rn > 0                       # rows with tokens (an empty request has O = 0)
            if m.any():
                er = max(er, float((np.abs(d).max(axis=-1)[m] / np.abs(o_ref).max(axis=-1)[m])
                                   .max()))
                el = max(el, float((np.linalg.norm(d, axis=-1)[m] / rn[m]).max()))
            num += float((d * d).sum())
            den += float((o_ref * o_ref).sum())
            fin = np.isfinite(l_ref)
            lse_err = float(np.abs(h["lse"][fin] - l_ref[fin]).max()) if fin.any() else 0.0
            out.setdefault(name, {"lse_max_abs": 0.0})
            out[name]["lse_max_abs"] = max(out[name]["lse_max_abs"], lse_err)
            for r, (po, _) in enumerate(shard):
                pn = np.linalg.norm(po, axis=-1)
                m = pn > 0
                if m.any():
                    pd = np.linalg.norm(h["o_parts"][r] - po, axis=-1)[m] / pn[m]
                    pl2 = max(pl2, float(pd.max()))
        out[name].update({
            "requests": [h["b"] for h in rows], "o_max_abs": float(f"{ea:.3e}"),
            "o_max_rel": float(f"{er:.3e}"), "o_rel_l2_row_max": float(f"{el:.3e}"),
            "o_rel_l2": float(f"{np.sqrt(num / den):.3e}"),
            "partial_o_rel_l2_row_max": float(f"{pl2:.3e}"),
            "oracle_s": round(time.perf_counter() - t0, 1)})
        out[name]["lse_max_abs"] = float(f"{out[name]['lse_max_abs']:.3e}")
    return out


def run_step_fns(dca, w, inp, kind):
    import torch
    q = inp["q"]
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    C = w.cp_size
    o_parts = torch.empty(C, w.batch, w.num_q_heads, w.head_dim_v, device="cuda")
    l_parts = torch.empty(C, w.batch, w.num_q_heads, device="cuda")
    o = torch.empty(w.batch, w.num_q_heads, w.head_dim_v, device="cuda")
    lse = torch.empty(w.batch, w.num_q_heads, device="cuda")
    ws = dca.alloc_workspace(dca.make_desc(kind, q, kv, inp["block_table"]), w.batch,
                             inp["max_seq_len"], C, w.interleave)
    shard_events, merge_events = [], []

    def step(record):
        for r in range(C):
            ev = None
            if record:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                shard_events.append(ev)
            dca.shard(q, kv, v, inp["block_table"], inp["seq_lens"], r, C, w.interleave,
                      w.scale, kind=kind, max_seq_len=inp["max_seq_len"], out=o_parts[r],
                      lse=l_parts[r], workspace=ws, events=ev, k_scale=inp.get("k_scale"),
                      v_scale=inp.get("v_scale"))
        ev = None
        if record:
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            merge_events.append(ev)
        dca.merge(o_parts, l_parts, out=o, lse_out=lse, events=ev)

    step.bufs = (o_parts, l_parts, o, lse)
    return step, shard_events, merge_events, ws


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa_qwen3_235b_share")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only the main workload's step (no interleave-1 pass, no other "
                         "workloads): a kernel trace of it then holds only the step's launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the other DCP "
              "ranks are virtual shards of one cache); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_context_amd as dca
    from decode_attention_context_amd import workloads as wl

    if args.copy_calibration:
        n = 1 << 30
        x = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(5):
            y.copy_(x)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / 5
        print(json.dumps({"copy_calibration_bytes_each_way": n, "launches": 8,
                          "copy_us": round(ms * 1e3, 2),
                          "copy_gbs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}))
        return

    dca.load()
    w = wl.WORKLOADS[args.workload]
    kind = dca.GQA if w.kind == "gqa" else dca.MLA
    inp = wl.make_inputs(w, device="cuda")
    lens = w.seq_lens()
    step, shard_ev, merge_ev, ws = run_step_fns(dca, w, inp, kind)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    # eager pass: every launch stamped by its own kernel's start / end (kernel durations)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed_eager = time.perf_counter() - t0
    assert dca.read_device_errors(ws) == 0
    # timed pass: the same step (every shard launch + the merge) captured once in a HIP
    # graph and replayed, so the launches follow each other without host dispatch gaps
    graph = capture_step(torch, step)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert dca.read_device_errors(ws) == 0
    samples = None if args.no_cpu_baseline else {}
    keep_sample(samples, w, inp, step.bufs, sorted({0, w.batch // 3, 2 * w.batch // 3,
                                                    w.batch - 1}))

    shard_ms = [a.elapsed_time(b) for a, b in shard_ev]
    merge_ms = [a.elapsed_time(b) for a, b in merge_ev]
    C = w.cp_size
    # per-rank average kernel duration; algorithmic bytes per launch averaged over ranks
    per_rank_ms = [sum(shard_ms[r::C]) / len(shard_ms[r::C]) for r in range(C)]
    tokens_per_step = int(sum(int(L) for L in lens))
    ms_per_step = elapsed * 1e3 / args.steps
    value = tokens_per_step * args.steps / elapsed

    if kind == dca.GQA:
        costs = [gqa_launch_bytes(w, lens, r) for r in range(C)]
        bytes_avg = sum(c[0] for c in costs) / C
        dur_s = sum(per_rank_ms) / C / 1e3
        achieved = bytes_avg / dur_s / 1e9
        fp8 = w.kv_dtype == "fp8"
        traffic = (load_counters("gqa_fp8", "gqa_fp8.hip", w.name) if fp8
                   else load_counters("gqa_shard", "gqa_shard.hip", w.name))
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": gqa_kernel_name(w),
                "algorithmic_bytes_per_launch": int(bytes_avg),
                "avg_launch_us": round(dur_s * 1e6, 2)}
        kernel_name = "gqa_shard"
    else:
        costs = [mla_launch_cost(w, lens, r) for r in range(C)]
        flops_avg = sum(c[1] for c in costs) / C
        dur_s = sum(per_rank_ms) / C / 1e3
        achieved = flops_avg / dur_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": load_counters("mla_shard", "mla_shard.hip", w.name),
                "kernel": "mla_shard_kernel",
                "algorithmic_flops_per_launch": int(flops_avg),
                "hbm_gbs": round(sum(c[0] for c in costs) / C / dur_s / 1e9, 1),
                "avg_launch_us": round(dur_s * 1e6, 2)}
        kernel_name = "mla_shard"

    merge_us = sum(merge_ms) / len(merge_ms) * 1e3
    merge_bytes = C * w.batch * w.num_q_heads * (w.head_dim_v + 1) * 4 + \
        w.batch * w.num_q_heads * (w.head_dim_v + 1) * 4
    line = {
        "metric": "shard decode attn: HBM GB/s (% peak), KV tokens/s; MLA MFMA util; merge GB/s",
        "value": round(value, 1), "unit": "KV tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_eager": round(elapsed_eager * 1e3 / args.steps, 4),
        "step_launch": "hip_graph_replay", "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": int(max(lens)),
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim_qk": w.head_dim_qk, "head_dim_v": w.head_dim_v,
                   "block_size": w.block_size, "cp_size": C, "interleave": w.interleave,
                   "step": f"{C} virtual-rank shard launches + 1 merge"},
        "roofline": roof,
        "kernels": {f"{kernel_name}_us_per_rank": [round(x * 1e3, 2) for x in per_rank_ms],
                    "merge_us": round(merge_us, 2),
                    "merge_gbs": round(merge_bytes / (merge_us * 1e-6) / 1e9, 1)},
    }
    copy_gbs = device_copy_gbs(torch)
    line["device_copy_gbs"] = copy_gbs
    if roof["unit"] == "GB/s":
        roof["frac_of_device_copy"] = round(roof["achieved"] / copy_gbs, 4)
    elif "hbm_gbs" in roof:
        roof["hbm_frac_of_device_copy"] = round(roof["hbm_gbs"] / copy_gbs, 4)
    if not args.no_secondary:
        line["kernels"][f"{kernel_name}_interleave1_us"] = fine_interleave_us(dca, torch, w, inp,
                                                                             kind)
        line["kernels"][f"{kernel_name}_cold_us"] = cold_shard_us(dca, torch, w, inp, kind)
    if not args.no_secondary and kind == dca.GQA:
        line["secondary"] = secondary_mla(dca, wl, torch, samples=samples)
        line["secondary_ragged"] = secondary_ragged(dca, wl, torch, samples=samples)
        line["secondary_long"] = secondary_long(dca, wl, torch, samples=samples)
        line["secondary_fp8kv"] = secondary_fp8kv(dca, wl, torch)
        line["secondary_tiny"] = secondary_tiny(dca, wl, torch, samples=samples)
        line["secondary_multi_token"] = secondary_multi_token(dca, wl, torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["accuracy"] = oracle_leg(w, inp, samples)
    print(json.dumps(line), flush=True)


def capture_step(torch, step):
    """A HIP graph of one step (all launches recorded once on a side stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(False)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(False)
    return g


def fine_interleave_us(dca, torch, w, inp, kind, steps=10):
    """Median shard-kernel time of the same workload and inputs with interleave 1 (every
    token owned round-robin: the token-granular path instead of page-contiguous tiles)."""
    step, shard_ev, _, _ = run_step_fns(dca, w.with_(interleave=1), inp, kind)
    for _ in range(3):
        step(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in shard_ev)
    return round(ms[len(ms) // 2] * 1e3, 2)


def device_copy_gbs(torch, nbytes=1 << 30, reps=5):
    """Rate of a plain device-to-device copy of `nbytes` (bytes read + bytes written per
    second, median of `reps`): the practical HBM ceiling the kernels are also compared with."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    ms = []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        y.copy_(x)
        ev[1].record()
        torch.cuda.synchronize()
        ms.append(ev[0].elapsed_time(ev[1]))
    del x, y
    return round(2 * nbytes / (sorted(ms)[reps // 2] * 1e-3) / 1e9, 1)


def cold_shard_us(dca, torch, w, inp, kind, steps=10):
    """Median rank-0 shard kernel duration with the last-level cache (256 MB MALL) and the
    L2s flushed before each launch by a 1 GiB read: the cache holds nothing of the step's
    inputs (the KV cache itself is several times larger than the MALL either way)."""
    flush = torch.ones(1 << 28, device="cuda")
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    ws = None
    ms = []
    for i in range(steps + 2):
        flush.sum()
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        _, _, ws = dca.shard(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], 0, w.cp_size,
                             w.interleave, w.scale, kind=kind, max_seq_len=inp["max_seq_len"],
                             workspace=ws, events=ev, k_scale=inp.get("k_scale"),
                             v_scale=inp.get("v_scale"))
        torch.cuda.synchronize()
        if i >= 2:
            ms.append(ev[0].elapsed_time(ev[1]))
    del flush
    return round(sorted(ms)[len(ms) // 2] * 1e3, 2)


def secondary_mla(dca, wl, torch, steps=20, samples=None):
    """MLA decode workload (64 x 67584, 128 heads, C = 8): rank-0 shard kernel MFMA
    utilisation and HBM rate, and the 8-partial merge rate."""
    w = wl.MLA_DECODE
    inp = wl.make_inputs(w, device="cuda")
    lens = w.seq_lens()
    step, shard_ev, merge_ev, ws = run_step_fns(dca, w, inp, dca.MLA)
    for _ in range(3):
        step(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    C = w.cp_size
    shard_ms = [a.elapsed_time(b) for a, b in shard_ev]
    dur = sum(shard_ms) / len(shard_ms) / 1e3
    costs = [mla_launch_cost(w, lens, r) for r in range(C)]
    byts = sum(c[0] for c in costs) / C
    flops = sum(c[1] for c in costs) / C
    merge_us = sum(a.elapsed_time(b) for a, b in merge_ev) / len(merge_ev) * 1e3
    merge_bytes = (C + 1) * w.batch * w.num_q_heads * (w.head_dim_v + 1) * 4
    # The same merge with its 134 MB of partials evicted from L2 and the 256 MB MALL by a
    # 1 GiB read before each launch (HBM rate), and with them just read by the previous
    # merge (cached rate).  In the step above the partials of the later ranks may still be
    # cached, those of the first ranks are not.
    o_parts, l_parts, o, lse = step.bufs
    flush = torch.ones(1 << 28, device="cuda")

    def merge_median(prep, reps=12):
        ms = []
        for _ in range(reps):
            prep()
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            dca.merge(o_parts, l_parts, out=o, lse_out=lse, events=ev)
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]) * 1e3)
        return sorted(ms)[len(ms) // 2]

    keep_sample(samples, w, inp, step.bufs, [0, w.batch - 1])
    mla_i1_us = fine_interleave_us(dca, torch, w, inp, dca.MLA)
    mla_cold_us = cold_shard_us(dca, torch, w, inp, dca.MLA)
    merge_hbm_us = merge_median(lambda: flush.sum())
    merge_cached_us = merge_median(lambda: None)
    del inp, flush
    torch.cuda.empty_cache()
    return {"workload": w.name, "mla_shard_avg_us": round(dur * 1e6, 2),
            "mla_mfma_util": round(flops / dur / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "mla_tflops": round(flops / dur / 1e12, 1),
            "mla_hbm_gbs": round(byts / dur / 1e9, 1),
            "mla_hbm_frac": round(byts / dur / 1e9 / HBM_PEAK_GBS, 4),
            "mla_traffic": load_counters("mla_shard", "mla_shard.hip", w.name),
            "mla_kv_tokens_per_s": round(sum(c[2] for c in costs) / C / dur, 1),
            "merge8_us": round(merge_us, 2),
            "merge8_gbs": round(merge_bytes / (merge_us * 1e-6) / 1e9, 1),
            "merge8_hbm_us": round(merge_hbm_us, 2),
            "merge8_hbm_gbs": round(merge_bytes / (merge_hbm_us * 1e-6) / 1e9, 1),
            "merge8_cached_us": round(merge_cached_us, 2),
            "merge8_cached_gbs": round(merge_bytes / (merge_cached_us * 1e-6) / 1e9, 1),
            "merge8_traffic": load_counters("merge_small", "merge.hip", w.name),
            "mla_interleave1_shard_us": mla_i1_us,
            "mla_shard_cold_us": mla_cold_us}


def shard_kernel_us(dca, torch, w, inp, kind, steps=10):
    """Median duration of the rank-0 shard kernel (its own start / end stamps)."""
    kv = inp["k_pages"] if kind == dca.GQA else inp["latent_pages"]
    v = inp["v_pages"] if kind == dca.GQA else None
    ws = None
    ms = []
    for i in range(steps + 3):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        _, _, ws = dca.shard(inp["q"], kv, v, inp["block_table"], inp["seq_lens"], 0, w.cp_size,
                             w.interleave, w.scale, kind=kind, max_seq_len=inp["max_seq_len"],
                             workspace=ws, events=ev, k_scale=inp.get("k_scale"),
                             v_scale=inp.get("v_scale"))
        torch.cuda.synchronize()
        if i >= 3:
            ms.append(ev[0].elapsed_time(ev[1]))
    assert dca.read_device_errors(ws) == 0
    return sorted(ms)[len(ms) // 2] * 1e3


def secondary_multi_token(dca, wl, torch):
    """Multi-token decode (q_len query positions per request, e.g. speculative decoding):
    the rank-0 shard kernel of the GQA share at q_len 2 and 4 (HBM rate; every K / V row is
    read once for all positions) and of the MLA decode workload at q_len 2 (MFMA
    utilisation); and the MLA decode workload with 64 and 32 gathered heads."""
    res = {}
    for nq in (2, 4):
        w = wl.GQA_SHARE.with_(q_len=nq)
        inp = wl.make_inputs(w, device="cuda")
        us = shard_kernel_us(dca, torch, w, inp, dca.GQA)
        byts, tok = gqa_launch_bytes(w, w.seq_lens(), 0)
        byts += (nq - 1) * w.batch * w.num_q_heads * (w.head_dim_qk * 2 + (w.head_dim_v + 1) * 4)
        flops = tok * 4 * w.num_q_heads * w.head_dim_qk * nq
        res[f"gqa_share_q{nq}"] = {"shard_us": round(us, 2),
                                   "hbm_gbs": round(byts / us / 1e3, 1),
                                   "hbm_frac": round(byts / us / 1e3 / HBM_PEAK_GBS, 4),
                                   "tflops": round(flops / us / 1e6, 2)}
        del inp
    w = wl.MLA_DECODE.with_(q_len=2)
    inp = wl.make_inputs(w, device="cuda")
    us = shard_kernel_us(dca, torch, w, inp, dca.MLA)
    byts, flops, tok = mla_launch_cost(w, w.seq_lens(), 0)
    flops *= 2
    res["mla_decode_q2"] = {"shard_us": round(us, 2),
                            "mfma_util": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                            "tflops": round(flops / us / 1e6, 1),
                            "hbm_gbs": round(byts / us / 1e3, 1)}
    del inp
    # fewer gathered heads (smaller DCP groups), same cache: 64 and 32 heads
    for h in (64, 32):
        w = wl.MLA_DECODE.with_(num_q_heads=h)
        inp = wl.make_inputs(w, device="cuda")
        us = shard_kernel_us(dca, torch, w, inp, dca.MLA)
        byts, flops, tok = mla_launch_cost(w, w.seq_lens(), 0)
        res[f"mla_decode_h{h}"] = {"shard_us": round(us, 2),
                                   "mfma_util": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                                   "tflops": round(flops / us / 1e6, 1),
                                   "hbm_gbs": round(byts / us / 1e3, 1)}
        del inp
    torch.cuda.empty_cache()
    return res


def secondary_ragged(dca, wl, torch, steps=5, samples=None):
    """Ragged MLA batch (512 requests, lognormal lengths around 67000 plus injected edge
    lengths, C = 8, I = 64): all 8 shard kernels (sum of their durations, MFMA utilisation,
    HBM rate) and the merge of 8 partials per (request, head) row, the largest merge of the
    workloads (1.21 GB).  Also the whole step replayed as a HIP graph."""
    w = wl.MLA_RAGGED
    inp = wl.make_inputs(w, device="cuda")
    lens = w.seq_lens()
    step, shard_ev, merge_ev, ws = run_step_fns(dca, w, inp, dca.MLA)
    for _ in range(2):
        step(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    assert dca.read_device_errors(ws) == 0
    # sampled: requests of lengths 1, 65 and 4096 (edge lengths) and the first lognormal one
    edge = [int(next(i for i, L in enumerate(lens) if L == e)) for e in (1, 65, 4096)]
    keep_sample(samples, w, inp, step.bufs,
                edge + [next(i for i in range(w.batch) if i not in edge and lens[i] < 150000)])
    C = w.cp_size
    shard_ms = [a.elapsed_time(b) for a, b in shard_ev]
    shards_s = sum(shard_ms) / steps / 1e3            # all C shard kernels of one step
    costs = [mla_launch_cost(w, lens, r) for r in range(C)]
    byts = sum(c[0] for c in costs)
    flops = sum(c[1] for c in costs)
    merge_s = sorted(a.elapsed_time(b) for a, b in merge_ev)[len(merge_ev) // 2] / 1e3
    merge_bytes = (C + 1) * w.batch * w.num_q_heads * (w.head_dim_v + 1) * 4
    # the same merge over bf16 partials (what shards called with a bf16 output write): the
    # float32 partials rounded once, caches flushed before each launch
    o_parts, l_parts, o, lse = step.bufs
    o16 = o_parts.to(torch.bfloat16)
    flush = torch.ones(1 << 28, device="cuda")
    ms16 = []
    for _ in range(9):
        flush.sum()
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        dca.merge(o16, l_parts, out=o, lse_out=lse, events=ev)
        torch.cuda.synchronize()
        ms16.append(ev[0].elapsed_time(ev[1]))
    merge16_s = sorted(ms16)[len(ms16) // 2] / 1e3
    merge16_bytes = w.batch * w.num_q_heads * (C * (w.head_dim_v * 2 + 4) + (w.head_dim_v + 1) * 4)
    del o16, flush
    graph = capture_step(torch, step)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    empty = sum(1 for L in lens for r in range(C)
                if owned_tokens_count(int(L), r, C, w.interleave) == 0)
    del inp, graph
    torch.cuda.empty_cache()
    return {"workload": w.name, "kv_tokens": int(lens.sum()), "empty_shards": empty,
            "mla_shards_us": round(shards_s * 1e6, 1),
            "mla_mfma_util": round(flops / shards_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "mla_hbm_gbs": round(byts / shards_s / 1e9, 1),
            "merge8_us": round(merge_s * 1e6, 2),
            "merge8_bytes": merge_bytes,
            "merge8_gbs": round(merge_bytes / merge_s / 1e9, 1),
            "merge8_hbm_frac": round(merge_bytes / merge_s / 1e9 / HBM_PEAK_GBS, 4),
            "merge8_bf16_partials_us": round(merge16_s * 1e6, 2),
            "merge8_bf16_partials_bytes": merge16_bytes,
            "merge8_bf16_partials_gbs": round(merge16_bytes / merge16_s / 1e9, 1),
            "step_ms": round(step_s * 1e3, 3),
            "kv_tokens_per_s": round(int(lens.sum()) / step_s, 1)}


def secondary_tiny(dca, wl, torch, steps=200, samples=None):
    """The tiny fp32 case (1 request x 1024 tokens, 8 query heads on 2 KV heads, D 64,
    C = 2, I = 16): latency-bound, so reported as latency: the graph-replayed step (both
    shard calls + the merge) and each shard kernel's own duration."""
    w = wl.TINY_GQA
    inp = wl.make_inputs(w, device="cuda")
    step, shard_ev, merge_ev, ws = run_step_fns(dca, w, inp, dca.GQA)
    for _ in range(5):
        step(False)
    for _ in range(20):
        step(True)
    torch.cuda.synchronize()
    assert dca.read_device_errors(ws) == 0
    keep_sample(samples, w, inp, step.bufs, [0])
    shard_us = sorted(a.elapsed_time(b) for a, b in shard_ev)[len(shard_ev) // 2] * 1e3
    merge_us = sorted(a.elapsed_time(b) for a, b in merge_ev)[len(merge_ev) // 2] * 1e3
    graph = capture_step(torch, step)
    for _ in range(10):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    step_us = (time.perf_counter() - t0) / steps * 1e6
    del inp, graph
    return {"workload": w.name, "step_us": round(step_us, 2),
            "shard_kernel_us_median": round(shard_us, 2), "merge_us_median": round(merge_us, 2)}


def secondary_fp8kv(dca, wl, torch):
    """The GQA share with its K / V cache in fp8 (OCP E4M3 codes, one scale each): the
    rank-0 shard kernel at q_len 1 and 4 (HBM rate on half the cache bytes, KV tokens/s)."""
    res = {"workload": wl.GQA_SHARE_FP8.name}
    for nq in (1, 4):
        w = wl.GQA_SHARE_FP8.with_(q_len=nq)
        inp = wl.make_inputs(w, device="cuda")
        us = shard_kernel_us(dca, torch, w, inp, dca.GQA)
        byts, tok = gqa_launch_bytes(w, w.seq_lens(), 0)
        byts += (nq - 1) * w.batch * w.num_q_heads * (w.head_dim_qk * 2 + (w.head_dim_v + 1) * 4)
        res[f"q{nq}"] = {"shard_us": round(us, 2), "algorithmic_bytes": int(byts),
                         "hbm_gbs": round(byts / us / 1e3, 1),
                         "hbm_frac": round(byts / us / 1e3 / HBM_PEAK_GBS, 4),
                         "kv_tokens_per_s": round(tok / us * 1e6, 1)}
        del inp
    torch.cuda.empty_cache()
    return res


def secondary_long(dca, wl, torch, steps=30, samples=None):
    """Long-context MLA (8 requests x 200000 tokens, C = 4, I = 128): all 4 shard kernels of
    a step (sum of their durations, MFMA utilisation, HBM rate), the merge of 4 partials per
    (request, head) row (10.5 MB: latency-bound), and the whole step replayed as a HIP
    graph."""
    w = wl.MLA_LONG
    inp = wl.make_inputs(w, device="cuda")
    lens = w.seq_lens()
    step, shard_ev, merge_ev, ws = run_step_fns(dca, w, inp, dca.MLA)
    for _ in range(3):
        step(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    assert dca.read_device_errors(ws) == 0
    keep_sample(samples, w, inp, step.bufs, [w.batch - 1])
    C = w.cp_size
    shard_ms = [a.elapsed_time(b) for a, b in shard_ev]
    shards_s = sum(shard_ms) / steps / 1e3
    costs = [mla_launch_cost(w, lens, r) for r in range(C)]
    byts = sum(c[0] for c in costs)
    flops = sum(c[1] for c in costs)
    merge_s = sorted(a.elapsed_time(b) for a, b in merge_ev)[len(merge_ev) // 2] / 1e3
    merge_bytes = (C + 1) * w.batch * w.num_q_heads * (w.head_dim_v + 1) * 4
    graph = capture_step(torch, step)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    del inp, graph
    torch.cuda.empty_cache()
    return {"workload": w.name, "kv_tokens": int(lens.sum()),
            "mla_shards_us": round(shards_s * 1e6, 1),
            "mla_shard_us_per_rank": [round(sum(shard_ms[r::C]) / steps * 1e3, 2)
                                      for r in range(C)],
            "mla_mfma_util": round(flops / shards_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "mla_hbm_gbs": round(byts / shards_s / 1e9, 1),
            "merge4_us": round(merge_s * 1e6, 2), "merge4_bytes": merge_bytes,
            "step_ms": round(step_s * 1e3, 3),
            "kv_tokens_per_s": round(int(lens.sum()) / step_s, 1)}


if __name__ == "__main__":
    main()

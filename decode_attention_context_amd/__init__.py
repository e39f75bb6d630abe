"""MI355X (gfx950) decode-context-parallel attention: Python binding of libdcpattn.so.

A thin ctypes layer over the C ABI declared in include/dcp_attn.h: it checks tensor
shapes, dtypes and devices, passes raw device pointers and the current HIP stream, and
returns torch tensors.  Every step of the computation runs in the library's HIP kernels;
PyTorch only provides device memory and streams.  There is no fallback: if the library
is missing or fails to load, every call raises.

Entry points (same names as the C ABI, without the dcp_ prefix):
  shard(...)          partial decode attention over one DCP rank's shard -> (O_r, lse_r)
  shard_noalloc(...)  the same with the library's static scratch instead of a workspace
  merge(...)          LSE-weighted merge of cp_size partials -> (O, lse)
  shard_slots(...)    the block-table walk: physical slots of a rank's tokens
  local_len(...)      tokens of a sequence a rank stores (host)
  check_parallel(...) the DCP size constraints (host)
  workspace_size(...) bytes of scratch a shard call needs
  read_device_errors(workspace)  the device error word of the latest call
"""
import ctypes
import os

import torch

__all__ = ["load", "lib_path", "GQA", "MLA", "F32", "BF16", "DCPError", "workspace_size",
           "shard", "shard_noalloc", "merge", "shard_slots", "local_len", "check_parallel",
           "read_device_errors", "status_string", "DEVERR_SEQ_LEN", "DEVERR_BLOCK_ID"]

GQA, MLA = 0, 1
F32, BF16 = 0, 1
DEVERR_SEQ_LEN, DEVERR_BLOCK_ID = 1, 2

_LIB = None


def lib_path():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdcpattn.so")


class DCPError(RuntimeError):
    def __init__(self, fn, status):
        msg = status_string(status) if _LIB is not None else str(status)
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float

_SIGS = {
    "dcp_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Desc), _I, _I64, _I, _I]),
    "dcp_workspace_size_mq": (ctypes.c_size_t, [ctypes.POINTER(Desc), _I, _I, _I64, _I, _I]),
    "dcp_attn_shard_mq": (_I, [ctypes.POINTER(Desc), _I, _P, _P, _P, _P, _P, _I, _I64, _I, _I,
                               _I, _F, _P, _P, _P, ctypes.c_size_t, _P]),
    "dcp_attn_shard_mq_timed": (_I, [ctypes.POINTER(Desc), _I, _P, _P, _P, _P, _P, _I, _I64, _I,
                                     _I, _I, _F, _P, _P, _P, ctypes.c_size_t, _P, _P, _P]),
    "dcp_attn_shard": (_I, [ctypes.POINTER(Desc), _P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _F,
                            _P, _P, _P, ctypes.c_size_t, _P]),
    "dcp_attn_shard_timed": (_I, [ctypes.POINTER(Desc), _P, _P, _P, _P, _P, _I, _I64, _I, _I, _I,
                                  _F, _P, _P, _P, ctypes.c_size_t, _P, _P, _P]),
    "dcp_attn_shard_ex": (_I, [ctypes.POINTER(Desc), _I, _I, _P, _P, _P, _P, _P, _I, _I64, _I,
                               _I, _I, _F, _P, _P, _P, ctypes.c_size_t, _P, _P, _P]),
    "dcp_attn_shard_fp8kv": (_I, [ctypes.POINTER(Desc), _I, _I, _P, _P, _P, _F, _F, _P, _P, _I,
                                  _I64, _I, _I, _I, _F, _P, _P, _P, ctypes.c_size_t, _P, _P,
                                  _P]),
    "dcp_attn_shard_noalloc": (_I, [ctypes.POINTER(Desc), _I, _I, _P, _P, _P, _P, _P, _I,
                                    _I64, _I, _I, _I, _F, _P, _P, _P]),
    "dcp_merge_ex": (_I, [_P, _I, _P, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P]),
    "dcp_merge": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P]),
    "dcp_merge_timed": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P]),
    "dcp_shard_slots": (_I, [_P, _P, _I, _I, _I, _I64, _I, _I, _I, _P, _P, _P, _P]),
    "dcp_local_len": (_I64, [_I64, _I, _I, _I]),
    "dcp_check_parallel": (_I, [_I, _I, _I, _I]),
    "dcp_status_string": (ctypes.c_char_p, [_I]),
    "dcp_read_device_errors": (_I, [_P, _P, ctypes.POINTER(ctypes.c_int32)]),
}


def load():
    """Load libdcpattn.so (built in-tree by __graft_entry__.build()); raises if absent."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(the HIP library is required; there is no fallback)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def status_string(status):
    return load().dcp_status_string(int(status)).decode()


def _check(fn, status):
    if status != 0:
        raise DCPError(fn, status)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt):
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {dt}")


def _need(t, name, dtype=None, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {tuple(t.shape)}")


def make_desc(kind, q, kv_pages, block_table):
    """Descriptor from the query ([b, Hq, D], or [b, q_len, Hq, D] for multi-token decode),
    the cache pages and the block table.
    GQA kv_pages: [num_blocks, Hkv, B, D]; MLA kv_pages: [num_blocks, B, Dk]."""
    dtype = _dtype_code(q.dtype)
    hq = q.shape[-2]
    if kind == GQA:
        nb, hkv, bs, d = kv_pages.shape
        return Desc(GQA, dtype, hq, hkv, d, d, bs, block_table.shape[1], nb)
    if kind == MLA:
        nb, bs, dk = kv_pages.shape
        return Desc(MLA, dtype, hq, 1, dk, 512, bs, block_table.shape[1], nb)
    raise ValueError("kind must be GQA or MLA")


def workspace_size(desc, batch, max_seq_len, cp_size, interleave, q_len=1):
    n = load().dcp_workspace_size_mq(ctypes.byref(desc), q_len, batch, max_seq_len, cp_size,
                                     interleave)
    if n == 0:
        raise DCPError("dcp_workspace_size_mq", -1)
    return int(n)


def alloc_workspace(desc, batch, max_seq_len, cp_size, interleave, device=None, q_len=1):
    n = workspace_size(desc, batch, max_seq_len, cp_size, interleave, q_len)
    return torch.empty(n, dtype=torch.uint8, device=device or torch.device("cuda"))


def shard(q, kv_pages, v_pages, block_table, seq_lens, rank, cp_size, interleave, scale, *,
          kind=None, max_seq_len=None, out=None, lse=None, workspace=None, stream=None,
          events=None, out_dtype=torch.float32, k_scale=None, v_scale=None):
    """Partial attention of the gathered queries over rank `rank`'s shard.

    GQA: q [b, Hq, D], kv_pages = K pages [nb, Hkv, B, D], v_pages = V pages (same shape).
    MLA: q [b, H, 576] bf16 with H = 16, 32, 64 or 128 gathered heads, kv_pages = latent
    pages [nb, B, 576], v_pages None.
    Multi-token decode: q [b, q_len, Hq, D] (q_len <= 4), query position i of request b at
    global position seq_len - q_len + i, causally masked (dcp_attn_shard_mq).
    block_table int32 [b, max_blocks]; seq_lens int32 [b] (global lengths).
    Returns (O_r [b, Hq, Dv] or [b, q_len, Hq, Dv], lse_r float32 [b, Hq] or [b, q_len, Hq],
    workspace); O_r is float32, or bf16 (rounded to nearest even) with
    out_dtype=torch.bfloat16 (dcp_attn_shard_ex).
    `events` = (begin, end) torch.cuda.Event pair that takes the attention kernel's own start
    and end time stamps.
    fp8 KV cache (GQA, bf16 q): K and V pages of dtype uint8 or torch.float8_e4m3fn holding
    OCP FP8 E4M3 codes, with the float scales k_scale and v_scale (dcp_attn_shard_fp8kv)."""
    lib = load()
    if kind is None:
        kind = MLA if v_pages is None else GQA
    _need(q, "q")
    if q.dim() not in (3, 4):
        raise ValueError(f"q must be [b, Hq, D] or [b, q_len, Hq, D], got {tuple(q.shape)}")
    q_len = q.shape[1] if q.dim() == 4 else 1
    fp8 = kind == GQA and kv_pages.dtype in (torch.uint8, torch.float8_e4m3fn)
    if fp8:
        if k_scale is None or v_scale is None:
            raise ValueError("an fp8 KV cache needs k_scale and v_scale")
        if q.dtype != torch.bfloat16:
            raise TypeError("an fp8 KV cache takes bf16 queries")
    elif k_scale is not None or v_scale is not None:
        raise ValueError("k_scale / v_scale apply to an fp8 KV cache only")
    kv_dtype = kv_pages.dtype if fp8 else q.dtype
    _need(kv_pages, "kv_pages", dtype=kv_dtype)
    if kind == GQA:
        _need(v_pages, "v_pages", dtype=kv_dtype)
        if v_pages.shape != kv_pages.shape:
            raise ValueError("K and V pages must have the same shape")
    elif v_pages is not None:
        raise ValueError("MLA takes no v_pages")
    _need(block_table, "block_table", dtype=torch.int32, dim=2)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1)
    batch = q.shape[0]
    if block_table.shape[0] != batch or seq_lens.shape[0] != batch:
        raise ValueError("q, block_table and seq_lens disagree on the batch size")
    desc = make_desc(kind, q, kv_pages, block_table)
    if q.shape[-1] != desc.head_dim_qk:
        raise ValueError("q head dim does not match the cache")
    if max_seq_len is None:
        max_seq_len = desc.max_blocks_per_seq * desc.block_size
    dv = desc.head_dim_v
    rows = (batch,) + ((q_len,) if q.dim() == 4 else ()) + (desc.num_q_heads,)
    if out is None:
        out = torch.empty(rows + (dv,), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=q.device)
    _need(out, "out", dtype=out_dtype)
    _need(lse, "lse", dtype=torch.float32)
    if tuple(out.shape) != rows + (dv,) or tuple(lse.shape) != rows:
        raise ValueError("out / lse have the wrong shape")
    need = workspace_size(desc, batch, max_seq_len, cp_size, interleave, q_len)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    args = (_ptr(q), _ptr(kv_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), batch,
            int(max_seq_len), rank, cp_size, interleave, float(scale), _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream(stream))
    if fp8:
        evs = (ctypes.c_void_p(0), ctypes.c_void_p(0))
        if events is not None:
            for ev in events:
                if not ev.cuda_event:   # torch creates the HIP event on its first record
                    ev.record(stream)
            evs = tuple(ctypes.c_void_p(ev.cuda_event) for ev in events)
        _check("dcp_attn_shard_fp8kv",
               lib.dcp_attn_shard_fp8kv(ctypes.byref(desc), q_len, _dtype_code(out_dtype),
                                        _ptr(q), _ptr(kv_pages), _ptr(v_pages), float(k_scale),
                                        float(v_scale), *args[3:], *evs))
    elif out_dtype != torch.float32:
        evs = (ctypes.c_void_p(0), ctypes.c_void_p(0))
        if events is not None:
            for ev in events:
                if not ev.cuda_event:   # torch creates the HIP event on its first record
                    ev.record(stream)
            evs = tuple(ctypes.c_void_p(ev.cuda_event) for ev in events)
        _check("dcp_attn_shard_ex",
               lib.dcp_attn_shard_ex(ctypes.byref(desc), q_len, _dtype_code(out_dtype), *args,
                                     *evs))
    elif events is None:
        if q.dim() == 3:
            _check("dcp_attn_shard", lib.dcp_attn_shard(ctypes.byref(desc), *args))
        else:
            _check("dcp_attn_shard_mq", lib.dcp_attn_shard_mq(ctypes.byref(desc), q_len, *args))
    else:
        ev0, ev1 = events
        for ev in (ev0, ev1):
            if not ev.cuda_event:       # torch creates the HIP event on its first record
                ev.record(stream)
        evs = (ctypes.c_void_p(ev0.cuda_event), ctypes.c_void_p(ev1.cuda_event))
        if q.dim() == 3:
            _check("dcp_attn_shard_timed",
                   lib.dcp_attn_shard_timed(ctypes.byref(desc), *args, *evs))
        else:
            _check("dcp_attn_shard_mq_timed",
                   lib.dcp_attn_shard_mq_timed(ctypes.byref(desc), q_len, *args, *evs))
    return out, lse, workspace


NOALLOC_SCRATCH_BYTES = 64 << 20   # DCP_NOALLOC_SCRATCH_BYTES of include/dcp_attn.h


def shard_noalloc(q, kv_pages, v_pages, block_table, seq_lens, rank, cp_size, interleave,
                  scale, out, lse, *, kind=None, max_seq_len=None, stream=None):
    """dcp_attn_shard_noalloc: the shard call with the plan and split partials in the
    library's static device scratch (no workspace, nothing allocated by the call).  The
    caller passes the outputs: out [b, Hq, Dv] or [b, q_len, Hq, Dv] (float32 or bf16) and
    lse float32 [b, Hq] or [b, q_len, Hq].  Calls on one device must not overlap."""
    lib = load()
    if kind is None:
        kind = MLA if v_pages is None else GQA
    _need(q, "q")
    if q.dim() not in (3, 4):
        raise ValueError(f"q must be [b, Hq, D] or [b, q_len, Hq, D], got {tuple(q.shape)}")
    q_len = q.shape[1] if q.dim() == 4 else 1
    _need(kv_pages, "kv_pages", dtype=q.dtype)
    if kind == GQA:
        _need(v_pages, "v_pages", dtype=q.dtype)
        if v_pages.shape != kv_pages.shape:
            raise ValueError("K and V pages must have the same shape")
    elif v_pages is not None:
        raise ValueError("MLA takes no v_pages")
    _need(block_table, "block_table", dtype=torch.int32, dim=2)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1)
    batch = q.shape[0]
    if block_table.shape[0] != batch or seq_lens.shape[0] != batch:
        raise ValueError("q, block_table and seq_lens disagree on the batch size")
    desc = make_desc(kind, q, kv_pages, block_table)
    if max_seq_len is None:
        max_seq_len = desc.max_blocks_per_seq * desc.block_size
    rows = (batch,) + ((q_len,) if q.dim() == 4 else ()) + (desc.num_q_heads,)
    _need(out, "out")
    _need(lse, "lse", dtype=torch.float32)
    if tuple(out.shape) != rows + (desc.head_dim_v,) or tuple(lse.shape) != rows:
        raise ValueError("out / lse have the wrong shape")
    _check("dcp_attn_shard_noalloc",
           lib.dcp_attn_shard_noalloc(ctypes.byref(desc), q_len, _dtype_code(out.dtype),
                                      _ptr(q), _ptr(kv_pages), _ptr(v_pages), _ptr(block_table),
                                      _ptr(seq_lens), batch, int(max_seq_len), rank, cp_size,
                                      interleave, float(scale), _ptr(out), _ptr(lse),
                                      _stream(stream)))
    return out, lse


def merge(o_partials, lse_partials, *, out_dtype=torch.float32, out=None, lse_out=None,
          want_lse=True, stream=None, events=None):
    """LSE merge of o_partials [C, b, H, Dv] (float32, or bf16 through dcp_merge_ex) /
    lse_partials [C, b, H] -> (O, lse).  Partials
    of multi-token decode, [C, b, q_len, H, Dv] / [C, b, q_len, H], merge the same way (rows
    b x q_len*H).  `events` = (begin, end) torch.cuda.Event pair that takes the merge
    kernel's own start and end time stamps."""
    lib = load()
    _need(o_partials, "o_partials")
    in_dtype = _dtype_code(o_partials.dtype)
    _need(lse_partials, "lse_partials", dtype=torch.float32)
    if o_partials.dim() not in (4, 5) or lse_partials.dim() != o_partials.dim() - 1:
        raise ValueError("o_partials must be [C, b, H, Dv] or [C, b, q_len, H, Dv]")
    if tuple(lse_partials.shape) != tuple(o_partials.shape[:-1]):
        raise ValueError("lse_partials shape does not match o_partials")
    c, b, dv = o_partials.shape[0], o_partials.shape[1], o_partials.shape[-1]
    rows_shape = tuple(o_partials.shape[1:-1])
    h = 1
    for n in rows_shape[1:]:
        h *= n
    if out is None:
        out = torch.empty(rows_shape + (dv,), dtype=out_dtype, device=o_partials.device)
    _need(out, "out", dtype=out_dtype)
    if tuple(out.shape) != rows_shape + (dv,):
        raise ValueError("out has the wrong shape")
    if want_lse and lse_out is None:
        lse_out = torch.empty(rows_shape, dtype=torch.float32, device=o_partials.device)
    if in_dtype != F32:
        evs = (ctypes.c_void_p(0), ctypes.c_void_p(0))
        if events is not None:
            for ev in events:
                if not ev.cuda_event:
                    ev.record(stream)
            evs = tuple(ctypes.c_void_p(ev.cuda_event) for ev in events)
        _check("dcp_merge_ex",
               lib.dcp_merge_ex(_ptr(o_partials), in_dtype, _ptr(lse_partials), c, b, h, dv,
                                _ptr(out), _dtype_code(out_dtype), _ptr(lse_out),
                                _stream(stream), *evs))
    elif events is None:
        st = lib.dcp_merge(_ptr(o_partials), _ptr(lse_partials), c, b, h, dv, _ptr(out),
                           _dtype_code(out_dtype), _ptr(lse_out), _stream(stream))
        _check("dcp_merge", st)
    else:
        ev0, ev1 = events
        for ev in (ev0, ev1):
            if not ev.cuda_event:       # torch creates the HIP event on its first record
                ev.record(stream)
        st = lib.dcp_merge_timed(_ptr(o_partials), _ptr(lse_partials), c, b, h, dv, _ptr(out),
                                 _dtype_code(out_dtype), _ptr(lse_out), _stream(stream),
                                 ctypes.c_void_p(ev0.cuda_event), ctypes.c_void_p(ev1.cuda_event))
        _check("dcp_merge_timed", st)
    return out, lse_out


def local_len(seq_len, rank, cp_size, interleave):
    n = load().dcp_local_len(int(seq_len), rank, cp_size, interleave)
    if n < 0:
        raise DCPError("dcp_local_len", -1)
    return int(n)


def check_parallel(tp, dcp, num_kv_heads, is_mla):
    return bool(load().dcp_check_parallel(tp, dcp, num_kv_heads, int(bool(is_mla))))


def shard_slots(block_table, seq_lens, block_size, num_blocks, rank, cp_size, interleave, *,
                seq_lens_host=None, stream=None):
    """Physical slots of the tokens `rank` owns, per request, ascending position.
    Returns (slots int64 [sum of local lengths], offsets int64 [b + 1], workspace)."""
    lib = load()
    _need(block_table, "block_table", dtype=torch.int32, dim=2)
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1)
    lens = seq_lens_host if seq_lens_host is not None else seq_lens.cpu().tolist()
    cap = block_table.shape[1] * block_size
    counts = [local_len(min(max(int(n), 0), cap), rank, cp_size, interleave) for n in lens]
    offs = [0]
    for n in counts:
        offs.append(offs[-1] + n)
    dev = block_table.device
    offsets = torch.tensor(offs, dtype=torch.int64, device=dev)
    slots = torch.empty(max(1, offs[-1]), dtype=torch.int64, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    st = lib.dcp_shard_slots(_ptr(block_table), _ptr(seq_lens), block_table.shape[0],
                             block_table.shape[1], block_size, int(num_blocks), rank, cp_size,
                             interleave, _ptr(offsets), _ptr(slots), _ptr(ws), _stream(stream))
    _check("dcp_shard_slots", st)
    return slots[:offs[-1]], offsets, ws


def read_device_errors(workspace, stream=None):
    """The DCP_DEVERR_* bits of the latest shard / slots call on `workspace` (syncs)."""
    out = ctypes.c_int32(0)
    st = load().dcp_read_device_errors(_ptr(workspace), _stream(stream), ctypes.byref(out))
    _check("dcp_read_device_errors", st)
    return int(out.value)

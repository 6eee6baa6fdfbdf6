"""Python binding of libdbsa.so (argument marshalling only).

Every function passes torch tensors' device pointers and the current HIP
stream to the C ABI declared in include/dbsa.h; all computation happens in the
library's gfx950 kernels.  If the library is missing, calls raise: there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "DbsaError", "load", "dbsa_prefill", "dbsa_prefill_layers", "dbsa_append_block",
    "dbsa_gather_rope",
    "dbsa_query_attn", "dbsa_query_attn_gathered", "dbsa_query_attn_gathered_noalloc",
    "dbsa_workspace_bytes", "dbsa_version",
    "OP_PREFILL", "OP_APPEND", "OP_GATHER", "OP_QUERY", "OP_QUERY_GATHERED", "OP_GATHER_SPANS",
    "OP_QUERY_SPANS", "OP_QUERY_BATCHED", "SYMBOLS", "dbsa_query_attn_batched", "dbsa_gather_rope_spans", "dbsa_query_attn_spans",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdbsa.so")

OK, EINVAL, EUNSUPPORTED, ENOSPC, EHIP = 0, -1, -2, -3, -4
BF16, F32 = 0, 1
OP_PREFILL, OP_APPEND, OP_GATHER, OP_QUERY, OP_QUERY_GATHERED = 0, 1, 2, 3, 4
OP_GATHER_SPANS, OP_QUERY_SPANS, OP_QUERY_BATCHED = 5, 6, 7
SYMBOLS = ("dbsa_prefill", "dbsa_prefill_layers", "dbsa_append_block", "dbsa_gather_rope", "dbsa_query_attn",
           "dbsa_query_attn_gathered", "dbsa_query_attn_gathered_noalloc",
           "dbsa_query_attn_batched", "dbsa_gather_rope_spans", "dbsa_query_attn_spans",
           "dbsa_workspace_bytes", "dbsa_last_error", "dbsa_version")
NOALLOC_SCRATCH_BYTES = 32 << 20


class DbsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dbsa error {code}: {msg}")
        self.code = code


class AttnT(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("rope_inv_freq", ctypes.c_void_p)]  # const double*


class BlocksT(ctypes.Structure):
    _fields_ = [("block_lens", ctypes.c_void_p), ("n_blocks", ctypes.c_int32),  # const int32_t*
                ("sink", ctypes.c_int32), ("j", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libdbsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise DbsaError(EHIP, f"{LIB_PATH} not built (run python -m "
                              "block_sparse_attention_sink_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pa, pb = ctypes.POINTER(AttnT), ctypes.POINTER(BlocksT)
    # Host arrays (const int32_t* / const int64_t*) go as plain addresses.
    p32 = p64 = vp
    lib.dbsa_prefill.argtypes = [pa, pb, vp, vp, vp, vp, vp, sz, vp]
    lib.dbsa_prefill_layers.argtypes = [pa, pb, i32, vp, i64, vp, vp, i64, vp, i64, vp, sz, vp]
    lib.dbsa_append_block.argtypes = [pa, pb, i32, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp]
    lib.dbsa_gather_rope.argtypes = [pa, pb, p32, i32, i32, vp, vp, vp, vp, i64, p64, vp, sz, vp]
    lib.dbsa_query_attn.argtypes = [pa, i32, i32, vp, vp, vp, vp, vp, p64, i64, vp, vp, sz, vp]
    lib.dbsa_query_attn_gathered.argtypes = [pa, pb, p32, i32, i32, vp, vp, i32, vp, vp, vp, vp,
                                             vp, p64, i64, vp, vp, sz, vp]
    lib.dbsa_query_attn_batched.argtypes = [pa, pb, p32, i32, i32, vp, vp, i32, vp, vp, vp, vp,
                                            vp, p64, i64, vp, vp, sz, vp]
    lib.dbsa_query_attn_gathered_noalloc.argtypes = [pa, pb, p32, i32, i32, vp, vp, i32, vp, vp,
                                                     vp, vp, vp, p64, i64, vp, vp]
    lib.dbsa_gather_rope_spans.argtypes = [pa, p32, p32, i32, i32, i64, vp, vp, vp, vp, i64,
                                           p64, vp, sz, vp]
    lib.dbsa_query_attn_spans.argtypes = [pa, p32, p32, i32, i32, i64, vp, vp, i32, vp, vp, vp,
                                          vp, vp, p64, i64, vp, vp, sz, vp]
    lib.dbsa_workspace_bytes.argtypes = [ctypes.c_int, pa, pb, i64, i32, i32, i64]
    lib.dbsa_workspace_bytes.restype = sz
    lib.dbsa_last_error.restype = ctypes.c_char_p
    lib.dbsa_version.restype = ctypes.c_char_p
    for name in ("dbsa_prefill", "dbsa_append_block", "dbsa_gather_rope", "dbsa_query_attn",
                 "dbsa_query_attn_gathered", "dbsa_query_attn_gathered_noalloc",
                 "dbsa_query_attn_batched", "dbsa_gather_rope_spans", "dbsa_query_attn_spans"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def dbsa_version() -> str:
    return load().dbsa_version().decode()


def _check(rc: int):
    if rc != OK:
        raise DbsaError(rc, load().dbsa_last_error().decode())


def attn_t(n_q_heads, n_kv_heads, head_dim, dtype, theta, scale=None) -> AttnT:
    """`theta` is the RoPE base, or an array of head_dim/2 angular frequencies
    (radians per position) used instead of theta^(-2i/d)."""
    sc = 0.0 if scale is None else float(scale)
    if np.ndim(theta) == 0:
        return AttnT(n_q_heads, n_kv_heads, head_dim, dtype, float(theta), sc, None)
    w = np.ascontiguousarray(np.asarray(theta, dtype=np.float64).reshape(-1))
    if w.size != head_dim // 2:
        raise DbsaError(EINVAL, f"rope frequency table has {w.size} entries, "
                                f"head_dim / 2 = {head_dim // 2} needed")
    a = AttnT(n_q_heads, n_kv_heads, head_dim, dtype, 1.0e4, sc, _addr(w))
    a._keep = w  # the table must outlive the call
    return a


class Blocks:
    """Keeps the host block_lens array alive for the call."""

    def __init__(self, block_lens, sink: int, j: int):
        self.lens = np.ascontiguousarray(np.asarray(block_lens, dtype=np.int32))
        self.t = BlocksT(_addr(self.lens), int(self.lens.size), int(sink), int(j))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise DbsaError(EUNSUPPORTED, f"dtype {t.dtype} not supported (bfloat16 or float32)")


def _ptr(t, name: str, dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise DbsaError(EINVAL, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise DbsaError(EINVAL, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise DbsaError(EINVAL, f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _addr(arr: np.ndarray) -> int:
    """Address of a host array's data (the array must outlive the call)."""
    return arr.__array_interface__["data"][0]


def _stream(device) -> int:
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


_ws_cache = {}


def _workspace(nbytes: int, device, stream: int):
    """Workspace of at least `nbytes` (and 1 MiB) for calls on `stream`.

    One workspace per (device, stream): calls on one stream are ordered, so
    they may share it, while calls on two streams may overlap and must not.
    The buffer is allocated on that stream (the current one), so when a
    larger one replaces it the caching allocator reuses the old memory only
    for work ordered after the calls that used it."""
    import torch
    key = (str(device), int(stream))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _run(device, stream, call, need):
    """call(ws_ptr, ws_bytes) with the cached workspace of (device, stream).

    DBSA_ENOSPC means nothing was enqueued.  Only when the workspace itself
    is too small (need() exceeds it) does it grow and the call run once more;
    every other ENOSPC (cache, context or output capacity) is raised."""
    ws = _workspace(0, device, stream)
    rc = call(ws.data_ptr(), ws.numel())
    if rc == ENOSPC:
        n = need()
        if n > ws.numel():
            ws = _workspace(n, device, stream)
            rc = call(ws.data_ptr(), ws.numel())
    _check(rc)


def _need(op, a, b, rows=0, batch=1, n_ids=0, max_ctx=0) -> int:
    lib = load()
    n = lib.dbsa_workspace_bytes(op, ctypes.byref(a), None if b is None else ctypes.byref(b.t),
                                 int(rows), int(batch), int(n_ids), int(max_ctx))
    if n == 0 and lib.dbsa_last_error():
        _check(EINVAL)
    return int(n)


def _max_selected(block_lens, ids: np.ndarray) -> int:
    """Largest total length of one row's selected blocks."""
    lens = np.asarray(block_lens, dtype=np.int64)
    return int(lens[np.clip(ids, 0, lens.size - 1)].sum(axis=1).max())


def dbsa_workspace_bytes(op, n_q_heads, n_kv_heads, head_dim, dtype, theta=1e4, block_lens=None,
                         sink=1, j=2, rows=0, batch=1, n_ids=0, max_ctx=0) -> int:
    lib = load()
    a = attn_t(n_q_heads, n_kv_heads, head_dim, dtype, theta)
    b = Blocks(block_lens if block_lens is not None else [1], sink, j)
    n = lib.dbsa_workspace_bytes(op, ctypes.byref(a), ctypes.byref(b.t), int(rows), int(batch),
                                 int(n_ids), int(max_ctx))
    if n == 0:
        msg = lib.dbsa_last_error().decode()
        if msg:
            raise DbsaError(EINVAL, msg)
    return int(n)


def _shape(t, name: str, want) -> None:
    """Raise EINVAL (before anything reaches the library) unless tensor `t`
    has len(want) dimensions and every entry of `want` that is not None."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        shown = ", ".join("*" if w is None else str(w) for w in want)
        raise DbsaError(EINVAL, f"{name} has shape {list(got)}, expected [{shown}]")


def _total_tokens(block_lens) -> int:
    return int(np.sum(np.asarray(block_lens, dtype=np.int64)))


def _pool_shape(k_pool, v_pool, hkv: int, d: int, min_tokens: int) -> None:
    _shape(k_pool, "k_pool", (None, hkv, d))
    _shape(v_pool, "v_pool", tuple(k_pool.shape))
    if k_pool.shape[0] < min_tokens:
        raise DbsaError(EINVAL, f"k_pool holds {k_pool.shape[0]} tokens, the blocks need "
                                f"{min_tokens}")


def dbsa_prefill(q, k, v, block_lens, sink: int, j: int, theta, scale=None, out=None):
    """Stage-1 block-sparse prefill of one layer: q [N, Hq, d], k, v [N, Hkv, d]
    with N = sum(block_lens); returns O [N, Hq, d]."""
    import torch
    lib = load()
    _shape(q, "q", (_total_tokens(block_lens), None, None))
    n, hq, d = q.shape
    _shape(k, "k", (n, None, d))
    hkv = k.shape[1]
    _shape(v, "v", (n, hkv, d))
    if out is not None:
        _shape(out, "out", (n, hq, d))
    dt = _dtype_code(q)
    a = attn_t(hq, hkv, d, dt, theta, scale)
    b = Blocks(block_lens, sink, j)
    if out is None:
        out = torch.empty_like(q)
    args = (ctypes.byref(a), ctypes.byref(b.t), _ptr(q, "q"), _ptr(k, "k", q.dtype),
            _ptr(v, "v", q.dtype), _ptr(out, "out", q.dtype))
    st = _stream(q.device)
    _run(q.device, st, lambda wp, wn: lib.dbsa_prefill(*args, wp, wn, st),
         lambda: _need(OP_PREFILL, a, b))
    return out


def dbsa_prefill_layers(q, k, v, block_lens, sink: int, j: int, theta, scale=None, out=None):
    """Stage-1 prefill of every layer: q [L, N, Hq, d] (or [N, Hq, d], shared
    by all layers), k, v [L, N, Hkv, d] (or [N, Hkv, d], shared); returns O
    [L, N, Hq, d]."""
    import torch
    lib = load()
    n_layers = max(t.shape[0] if t.dim() == 4 else 1 for t in (q, k, v))
    ql = q if q.dim() == 4 else q.unsqueeze(0)
    kl = k if k.dim() == 4 else k.unsqueeze(0)
    vl = v if v.dim() == 4 else v.unsqueeze(0)
    n = _total_tokens(block_lens)
    _shape(ql, "q", (None, n, None, None))
    _, _, hq, d = ql.shape
    _shape(kl, "k", (None, n, None, d))
    hkv = kl.shape[2]
    _shape(vl, "v", (kl.shape[0], n, hkv, d))
    for name, t in (("q", ql), ("k", kl), ("v", vl)):
        if t.shape[0] not in (1, n_layers) or not t.is_contiguous():
            raise DbsaError(EINVAL, f"{name}: {n_layers} layers (or one shared), contiguous")
    if out is not None:
        _shape(out, "out", (n_layers, n, hq, d))
    dt = _dtype_code(q)
    a = attn_t(hq, hkv, d, dt, theta, scale)
    b = Blocks(block_lens, sink, j)
    if out is None:
        out = torch.empty((n_layers, n, hq, d), dtype=q.dtype, device=q.device)
    stride = lambda t: 0 if t.shape[0] == 1 else t[0].numel()
    args = (ctypes.byref(a), ctypes.byref(b.t), n_layers, _ptr(ql, "q"), stride(ql),
            _ptr(kl, "k", q.dtype), _ptr(vl, "v", q.dtype), stride(kl), _ptr(out, "out", q.dtype),
            out[0].numel())
    st = _stream(q.device)
    _run(q.device, st, lambda wp, wn: lib.dbsa_prefill_layers(*args, wp, wn, st),
         lambda: _need(OP_PREFILL, a, b))
    return out


def dbsa_append_block(q_new, k_new, v_new, k_cache, v_cache, block_lens, sink: int, j: int,
                      theta: float, scale=None, out=None):
    """Encode one new block onto the pool (block_lens = the existing blocks):
    q_new [L, Hq, d], k_new, v_new [L, Hkv, d]; k_cache, v_cache [cap, Hkv, d]
    holding the pool's sum(block_lens) tokens (the new ones are written after
    them); returns O [L, Hq, d]."""
    import torch
    lib = load()
    _shape(q_new, "q_new", (None, None, None))
    new_len, hq, d = q_new.shape
    _shape(k_new, "k_new", (new_len, None, d))
    hkv = k_new.shape[1]
    _shape(v_new, "v_new", (new_len, hkv, d))
    _shape(k_cache, "k_cache", (None, hkv, d))
    _shape(v_cache, "v_cache", tuple(k_cache.shape))
    if out is not None:
        _shape(out, "out", (new_len, hq, d))
    dt = _dtype_code(q_new)
    a = attn_t(hq, hkv, d, dt, theta, scale)
    b = Blocks(block_lens, sink, j)
    if out is None:
        out = torch.empty_like(q_new)
    args = (ctypes.byref(a), ctypes.byref(b.t), int(new_len), _ptr(q_new, "q_new"),
            _ptr(k_new, "k_new", q_new.dtype), _ptr(v_new, "v_new", q_new.dtype),
            _ptr(k_cache, "k_cache", q_new.dtype), _ptr(v_cache, "v_cache", q_new.dtype),
            int(k_cache.shape[0]), _ptr(out, "out", q_new.dtype))
    st = _stream(q_new.device)
    _run(q_new.device, st, lambda wp, wn: lib.dbsa_append_block(*args, wp, wn, st),
         lambda: _need(OP_APPEND, a, b, rows=new_len))
    return out


def _ids2d(ids) -> np.ndarray:
    return np.ascontiguousarray(np.atleast_2d(np.asarray(ids, dtype=np.int32)))


def dbsa_gather_rope(k_pool, v_pool, block_lens, ids, theta: float, n_q_heads: Optional[int] = None,
                     capacity: Optional[int] = None, k_out=None, v_out=None, sink: int = 1,
                     j: int = 0):
    """Gather the selected blocks (ids [batch, n_ids], anchor first) of the pool
    k_pool, v_pool [N, Hkv, d] and re-rotate K.

    Returns (k_out, v_out, ctx_len) with k_out/v_out [batch, capacity, Hkv, d].
    """
    import torch
    lib = load()
    _shape(k_pool, "k_pool", (None, None, None))
    _, hkv, d = k_pool.shape
    _pool_shape(k_pool, v_pool, hkv, d, _total_tokens(block_lens))
    dt = _dtype_code(k_pool)
    a = attn_t(n_q_heads or hkv, hkv, d, dt, theta)
    b = Blocks(block_lens, sink, j)
    ids = _ids2d(ids)
    batch, n_ids = ids.shape
    if k_out is None:
        if capacity is None:
            capacity = _max_selected(block_lens, ids)
        k_out = torch.empty((batch, capacity, hkv, d), dtype=k_pool.dtype, device=k_pool.device)
        v_out = torch.empty_like(k_out)
    _shape(k_out, "k_out", (batch, None, hkv, d))
    _shape(v_out, "v_out", tuple(k_out.shape))
    ctx = np.zeros(batch, dtype=np.int64)
    args = (ctypes.byref(a), ctypes.byref(b.t), _addr(ids), n_ids, batch, _ptr(k_pool, "k_pool"),
            _ptr(v_pool, "v_pool", k_pool.dtype), _ptr(k_out, "k_out", k_pool.dtype),
            _ptr(v_out, "v_out", k_pool.dtype), int(k_out.shape[1]), _addr(ctx))
    st = _stream(k_pool.device)
    _run(k_pool.device, st, lambda wp, wn: lib.dbsa_gather_rope(*args, wp, wn, st),
         lambda: _need(OP_GATHER, a, b, batch=batch, n_ids=n_ids))
    return k_out, v_out, ctx


def _query_shapes(q, k_new, v_new, k_buf, v_buf, buf_name):
    """Shapes of a Stage-2 call: q [B, n, Hq, d], k_new, v_new [B, n, Hkv, d],
    context/tail buffers [B, cap, Hkv, d]; returns (B, n, Hq, Hkv, d)."""
    _shape(q, "q", (None, None, None, None))
    batch, n_new, hq, d = q.shape
    _shape(k_new, "k_new", (batch, n_new, None, d))
    hkv = k_new.shape[2]
    _shape(v_new, "v_new", (batch, n_new, hkv, d))
    _shape(k_buf, "k_" + buf_name, (batch, None, hkv, d))
    _shape(v_buf, "v_" + buf_name, tuple(k_buf.shape))
    return batch, n_new, hq, hkv, d


def dbsa_query_attn(q, k_new, v_new, k_ctx, v_ctx, ctx_len: Sequence[int], theta: float,
                    scale=None, out=None):
    """Query tokens q [batch, n_new, Hq, d] over the gathered cache k_ctx/v_ctx
    [batch, cap, Hkv, d] holding ctx_len[b] rotated tokens.  Appends the new
    tokens' K/V to the cache; the caller advances ctx_len by n_new."""
    import torch
    lib = load()
    batch, n_new, hq, hkv, d = _query_shapes(q, k_new, v_new, k_ctx, v_ctx, "ctx")
    if out is not None:
        _shape(out, "out", tuple(q.shape))
    dt = _dtype_code(q)
    a = attn_t(hq, hkv, d, dt, theta, scale)
    ctx = np.ascontiguousarray(np.asarray(ctx_len, dtype=np.int64).reshape(batch))
    if out is None:
        out = torch.empty_like(q)
    if n_new == 0:
        return out
    args = (ctypes.byref(a), batch, n_new, _ptr(q, "q"), _ptr(k_new, "k_new", q.dtype),
            _ptr(v_new, "v_new", q.dtype), _ptr(k_ctx, "k_ctx", q.dtype),
            _ptr(v_ctx, "v_ctx", q.dtype), _addr(ctx), int(k_ctx.shape[1]),
            _ptr(out, "out", q.dtype))
    st = _stream(q.device)
    _run(q.device, st, lambda wp, wn: lib.dbsa_query_attn(*args, wp, wn, st),
         lambda: _need(OP_QUERY, a, Blocks([1], 1, 0), rows=n_new, batch=batch,
                       max_ctx=int(ctx.max()) + n_new))
    return out


def dbsa_query_attn_gathered(q, k_new, v_new, k_pool, v_pool, block_lens, ids, k_tail, v_tail,
                             tail_len: Sequence[int], theta: float, scale=None, out=None):
    """Query tokens over the selected pool blocks, gathered and re-rotated inside
    the attention's loads, followed by the row's tail buffer (query/decoded
    tokens, rotated).  Appends the new tokens to the tail; the caller advances
    tail_len by n_new."""
    import torch
    lib = load()
    batch, n_new, hq, hkv, d = _query_shapes(q, k_new, v_new, k_tail, v_tail, "tail")
    _pool_shape(k_pool, v_pool, hkv, d, _total_tokens(block_lens))
    if out is not None:
        _shape(out, "out", tuple(q.shape))
    dt = _dtype_code(q)
    a = attn_t(hq, hkv, d, dt, theta, scale)
    b = Blocks(block_lens, 1, 0)
    ids = _ids2d(ids)
    if ids.shape[0] != batch:
        raise DbsaError(EINVAL, f"ids has {ids.shape[0]} rows, q has batch {batch}")
    n_ids = ids.shape[1]
    tl = np.ascontiguousarray(np.asarray(tail_len, dtype=np.int64).reshape(batch))
    if out is None:
        out = torch.empty_like(q)
    if n_new == 0:
        return out
    args = (ctypes.byref(a), ctypes.byref(b.t), _addr(ids), n_ids, batch,
            _ptr(k_pool, "k_pool", q.dtype), _ptr(v_pool, "v_pool", q.dtype), n_new, _ptr(q, "q"),
            _ptr(k_new, "k_new", q.dtype), _ptr(v_new, "v_new", q.dtype),
            _ptr(k_tail, "k_tail", q.dtype), _ptr(v_tail, "v_tail", q.dtype), _addr(tl),
            int(k_tail.shape[1]), _ptr(out, "out", q.dtype))
    st = _stream(q.device)
    _run(q.device, st, lambda wp, wn: lib.dbsa_query_attn_gathered(*args, wp, wn, st),
         lambda: _need(OP_QUERY_GATHERED, a, b, rows=n_new, batch=batch, n_ids=n_ids,
                       max_ctx=_max_selected(block_lens, ids) + int(tl.max()) + n_new))
    return out


def dbsa_query_attn_batched(q, k_new, v_new, k_pool, v_pool, block_lens, ids, k_tail, v_tail,
                            tail_len: Sequence[int], theta: float, scale=None, out=None):
    """dbsa_query_attn_gathered with the shared-block schedule: each selected
    pool block's K/V is loaded once for all the batch rows that chose it.
    Same arguments and results (up to rounding)."""
    import torch
    lib = load()
    batch, n_new, hq, hkv, d = _query_shapes(q, k_new, v_new, k_tail, v_tail, "tail")
    _pool_shape(k_pool, v_pool, hkv, d, _total_tokens(block_lens))
    if out is not None:
        _shape(out, "out", tuple(q.shape))
    dt = _dtype_code(q)
    a = attn_t(hq, hkv, d, dt, theta, scale)
    b = Blocks(block_lens, 1, 0)
    ids = _ids2d(ids)
    if ids.shape[0] != batch:
        raise DbsaError(EINVAL, f"ids has {ids.shape[0]} rows, q has batch {batch}")
    n_ids = ids.shape[1]
    tl = np.ascontiguousarray(np.asarray(tail_len, dtype=np.int64).reshape(batch))
    if out is None:
        out = torch.empty_like(q)
    if n_new == 0:
        return out
    args = (ctypes.byref(a), ctypes.byref(b.t), _addr(ids), n_ids, batch,
            _ptr(k_pool, "k_pool", q.dtype), _ptr(v_pool, "v_pool", q.dtype), n_new, _ptr(q, "q"),
            _ptr(k_new, "k_new", q.dtype), _ptr(v_new, "v_new", q.dtype),
            _ptr(k_tail, "k_tail", q.dtype), _ptr(v_tail, "v_tail", q.dtype), _addr(tl),
            int(k_tail.shape[1]), _ptr(out, "out", q.dtype))
    st = _stream(q.device)
    _run(q.device, st, lambda wp, wn: lib.dbsa_query_attn_batched(*args, wp, wn, st),
         lambda: _need(OP_QUERY_BATCHED, a, b, rows=n_new, batch=batch, n_ids=n_ids,
                       max_ctx=int(tl.max()) + n_new))
    return out


def dbsa_query_attn_gathered_noalloc(q, k_new, v_new, k_pool, v_pool, block_lens, ids, k_tail,
                                     v_tail, tail_len: Sequence[int], theta: float, scale=None,
                                     out=None):
    """dbsa_query_attn_gathered without a workspace: the library's fixed
    scratch array is used instead (nothing is allocated by the call except an
    `out` tensor when none is given).  Calls that may overlap on one GPU must
    not be issued."""
    import torch
    lib = load()
    batch, n_new, hq, hkv, d = _query_shapes(q, k_new, v_new, k_tail, v_tail, "tail")
    _pool_shape(k_pool, v_pool, hkv, d, _total_tokens(block_lens))
    if out is not None:
        _shape(out, "out", tuple(q.shape))
    dt = _dtype_code(q)
    a = attn_t(hq, hkv, d, dt, theta, scale)
    b = Blocks(block_lens, 1, 0)
    ids = _ids2d(ids)
    if ids.shape[0] != batch:
        raise DbsaError(EINVAL, f"ids has {ids.shape[0]} rows, q has batch {batch}")
    tl = np.ascontiguousarray(np.asarray(tail_len, dtype=np.int64).reshape(batch))
    if out is None:
        out = torch.empty_like(q)
    if n_new == 0:
        return out
    _check(lib.dbsa_query_attn_gathered_noalloc(
        ctypes.byref(a), ctypes.byref(b.t), _addr(ids), ids.shape[1], batch,
        _ptr(k_pool, "k_pool", q.dtype), _ptr(v_pool, "v_pool", q.dtype), n_new, _ptr(q, "q"),
        _ptr(k_new, "k_new", q.dtype), _ptr(v_new, "v_new", q.dtype),
        _ptr(k_tail, "k_tail", q.dtype), _ptr(v_tail, "v_tail", q.dtype), _addr(tl),
        int(k_tail.shape[1]), _ptr(out, "out", q.dtype), _stream(q.device)))
    return out


def _spans(span_src, span_len):
    src = np.ascontiguousarray(np.atleast_2d(np.asarray(span_src, dtype=np.int32)))
    ln = np.ascontiguousarray(np.atleast_2d(np.asarray(span_len, dtype=np.int32)))
    if src.shape != ln.shape:
        raise DbsaError(EINVAL, f"span_src {src.shape} and span_len {ln.shape} differ")
    return src, ln


def dbsa_gather_rope_spans(k_pool, v_pool, span_src, span_len, theta,
                           n_q_heads: Optional[int] = None, capacity: Optional[int] = None,
                           k_out=None, v_out=None):
    """Gather pool token spans ([batch, n_spans] sources and lengths, in
    placement order) and re-rotate K at 0..T'-1.  Returns (k_out, v_out,
    ctx_len) like dbsa_gather_rope."""
    import torch
    lib = load()
    _shape(k_pool, "k_pool", (None, None, None))
    n_pool, hkv, d = k_pool.shape
    _pool_shape(k_pool, v_pool, hkv, d, 0)
    dt = _dtype_code(k_pool)
    a = attn_t(n_q_heads or hkv, hkv, d, dt, theta)
    src, ln = _spans(span_src, span_len)
    batch, n_spans = src.shape
    if k_out is None:
        if capacity is None:
            capacity = int(max(1, ln.clip(min=0).sum(axis=1).max()))
        k_out = torch.empty((batch, capacity, hkv, d), dtype=k_pool.dtype, device=k_pool.device)
        v_out = torch.empty_like(k_out)
    _shape(k_out, "k_out", (batch, None, hkv, d))
    _shape(v_out, "v_out", tuple(k_out.shape))
    ctx = np.zeros(batch, dtype=np.int64)
    args = (ctypes.byref(a), _addr(src), _addr(ln), n_spans, batch, int(n_pool),
            _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool", k_pool.dtype),
            _ptr(k_out, "k_out", k_pool.dtype), _ptr(v_out, "v_out", k_pool.dtype),
            int(k_out.shape[1]), _addr(ctx))
    st = _stream(k_pool.device)
    _run(k_pool.device, st, lambda wp, wn: lib.dbsa_gather_rope_spans(*args, wp, wn, st),
         lambda: _need(OP_GATHER_SPANS, a, None, batch=batch, n_ids=n_spans))
    return k_out, v_out, ctx


def dbsa_query_attn_spans(q, k_new, v_new, k_pool, v_pool, span_src, span_len, k_tail, v_tail,
                          tail_len: Sequence[int], theta, scale=None, out=None):
    """Query tokens over pool token spans gathered and re-rotated inside the
    attention's loads, then the row's tail buffer (see
    dbsa_query_attn_gathered)."""
    import torch
    lib = load()
    batch, n_new, hq, hkv, d = _query_shapes(q, k_new, v_new, k_tail, v_tail, "tail")
    _pool_shape(k_pool, v_pool, hkv, d, 0)
    if out is not None:
        _shape(out, "out", tuple(q.shape))
    dt = _dtype_code(q)
    a = attn_t(hq, hkv, d, dt, theta, scale)
    src, ln = _spans(span_src, span_len)
    if src.shape[0] != batch:
        raise DbsaError(EINVAL, f"spans have {src.shape[0]} rows, q has batch {batch}")
    n_spans = src.shape[1]
    tl = np.ascontiguousarray(np.asarray(tail_len, dtype=np.int64).reshape(batch))
    if out is None:
        out = torch.empty_like(q)
    if n_new == 0:
        return out
    args = (ctypes.byref(a), _addr(src), _addr(ln), n_spans, batch, int(k_pool.shape[0]),
            _ptr(k_pool, "k_pool", q.dtype), _ptr(v_pool, "v_pool", q.dtype), n_new, _ptr(q, "q"),
            _ptr(k_new, "k_new", q.dtype), _ptr(v_new, "v_new", q.dtype),
            _ptr(k_tail, "k_tail", q.dtype), _ptr(v_tail, "v_tail", q.dtype), _addr(tl),
            int(k_tail.shape[1]), _ptr(out, "out", q.dtype))
    st = _stream(q.device)
    _run(q.device, st, lambda wp, wn: lib.dbsa_query_attn_spans(*args, wp, wn, st),
         lambda: _need(OP_QUERY_SPANS, a, None, rows=n_new, batch=batch, n_ids=n_spans,
                       max_ctx=int(ln.clip(min=0).sum(axis=1).max()) + int(tl.max()) + n_new))
    return out

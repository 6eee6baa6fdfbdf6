"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects malformed arguments on the host before any HIP
call (with the documented status codes)."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from block_sparse_attention_sink_amd import dbsa
from block_sparse_attention_sink_amd.inputs import llama31_inv_freq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# Aligned, never dereferenced: every call below fails a check before anything
# is enqueued.  A call that must pass the argument checks gets a workspace too
# small to hold it, so that it stops at the workspace check (the last one, and
# still before any launch): on a GPU machine a launch would read and write
# these fake addresses.
FAKE = 0x100000


@pytest.fixture(scope="module")
def lib():
    return dbsa.load()


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "dbsa.h")).read()
    declared = set(re.findall(r"\b(dbsa_[a-z_]+)\s*\(", header))
    assert declared == set(dbsa.SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    assert "gfx950" in dbsa.dbsa_version()


def test_exports_nothing_else_with_c_linkage():
    """Host helpers stay internal: the only unmangled functions the library
    exports are the declared entry points."""
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", dbsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    plain = {ln.split()[-1] for ln in out.splitlines()
             if ln.split()[1:2] == ["T"] and not ln.split()[-1].startswith("_Z")}
    assert plain == set(dbsa.SYMBOLS)


def test_no_host_staging_or_host_waits():
    """Per-call tables go in kernel arguments or through copy kernels on the
    caller's stream: the library neither allocates (host or device) nor waits
    on the host, so none of those runtime calls is even linked."""
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", dbsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    used = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in ("hipHostMalloc", "hipHostAlloc", "hipMalloc", "hipMallocAsync", "hipFree",
                 "hipEventSynchronize", "hipStreamSynchronize", "hipDeviceSynchronize",
                 "hipEventCreate", "hipEventCreateWithFlags", "hipHostRegister"):
        assert name not in used, name
    assert "hipLaunchKernel" in used or any(u.startswith("hipLaunch") for u in used)


def _attn(hq=4, hkv=2, d=128, dt=dbsa.BF16, theta=1e4):
    return dbsa.attn_t(hq, hkv, d, dt, theta)


def _prefill(lib, attn, blocks, ptrs=(FAKE,) * 4, ws=FAKE, ws_bytes=1 << 40):
    return lib.dbsa_prefill(ctypes.byref(attn), ctypes.byref(blocks.t) if blocks else None,
                            *ptrs, ws, ws_bytes, None)


def _err(lib):
    return lib.dbsa_last_error().decode()


def test_prefill_validation(lib):
    ok_blocks = dbsa.Blocks([5, 7, 9], 1, 2)
    assert _prefill(lib, _attn(), dbsa.Blocks([5, 0, 9], 1, 2)) == dbsa.EINVAL
    assert "length 0" in _err(lib)
    assert _prefill(lib, _attn(), dbsa.Blocks([5, 7], 1, -1)) == dbsa.EINVAL
    assert _prefill(lib, _attn(), dbsa.Blocks([5, 7], 2, 1)) == dbsa.EINVAL
    assert _prefill(lib, _attn(), dbsa.Blocks(np.zeros(0, np.int32), 1, 1)) == dbsa.EINVAL
    assert _prefill(lib, _attn(), None) == dbsa.EINVAL
    assert _prefill(lib, _attn(d=96), ok_blocks) == dbsa.EUNSUPPORTED
    assert _prefill(lib, _attn(hq=6, hkv=4), ok_blocks) == dbsa.EUNSUPPORTED
    assert _prefill(lib, _attn(dt=7), ok_blocks) == dbsa.EUNSUPPORTED
    assert _prefill(lib, _attn(theta=-1.0), ok_blocks) == dbsa.EINVAL
    assert _prefill(lib, _attn(), ok_blocks, ptrs=(FAKE, 0, FAKE, FAKE)) == dbsa.EINVAL
    assert _prefill(lib, _attn(), ok_blocks, ptrs=(FAKE + 8, FAKE, FAKE, FAKE)) == dbsa.EINVAL
    assert _prefill(lib, _attn(), ok_blocks, ws=0) == dbsa.EINVAL
    assert _prefill(lib, _attn(), ok_blocks, ws=FAKE + 64) == dbsa.EINVAL  # alignment
    assert _prefill(lib, _attn(), ok_blocks, ws_bytes=16) == dbsa.ENOSPC
    assert "workspace too small" in _err(lib)
    big = dbsa.Blocks(np.full(3, 1 << 30, np.int32), 1, 2)
    assert _prefill(lib, _attn(), big) == dbsa.EINVAL


def test_prefill_layers_validation(lib):
    blocks = dbsa.Blocks([5, 7, 9], 1, 2)
    a = _attn()
    q_ext, kv_ext = 21 * 4 * 128, 21 * 2 * 128

    def call(n, qs, kvs, os_, ws_bytes=1 << 40):
        return lib.dbsa_prefill_layers(ctypes.byref(a), ctypes.byref(blocks.t), n, FAKE, qs, FAKE,
                                       FAKE, kvs, FAKE, os_, FAKE, ws_bytes, None)
    assert call(0, q_ext, kv_ext, q_ext) == dbsa.EINVAL
    assert "n_layers" in _err(lib)
    assert call(2, q_ext, kv_ext, q_ext - 8) == dbsa.EINVAL  # outputs would overlap
    assert call(2, q_ext - 8, kv_ext, q_ext) == dbsa.EINVAL
    assert call(2, q_ext, kv_ext // 2, q_ext) == dbsa.EINVAL
    assert call(2, q_ext + 4, kv_ext, q_ext) == dbsa.EINVAL  # 8 bytes: misaligned layers
    assert "16 bytes" in _err(lib)
    # shared inputs (stride 0) and a single layer with any stride pass the
    # argument checks (and stop at the workspace check)
    assert call(3, 0, 0, q_ext, ws_bytes=16) == dbsa.ENOSPC and "workspace" in _err(lib)
    assert call(1, 3, 5, 7, ws_bytes=16) == dbsa.ENOSPC and "workspace" in _err(lib)


def test_rope_table_validation(lib):
    ok_blocks = dbsa.Blocks([5, 7, 9], 1, 2)
    table = llama31_inv_freq(5e5, 128)
    # a valid table passes the argument checks (and stops at the workspace check)
    assert _prefill(lib, dbsa.attn_t(4, 2, 128, dbsa.BF16, table), ok_blocks,
                    ws_bytes=16) == dbsa.ENOSPC
    assert "workspace" in _err(lib)
    for bad in (np.nan, -1.0, np.inf):
        t = table.copy()
        t[7] = bad
        assert _prefill(lib, dbsa.attn_t(4, 2, 128, dbsa.BF16, t), ok_blocks) == dbsa.EINVAL
        assert "rope_inv_freq[7]" in _err(lib)
    with pytest.raises(dbsa.DbsaError):
        dbsa.attn_t(4, 2, 128, dbsa.BF16, table[:10])


def _gather(lib, ids, n_blocks=6, cap=1 << 20, ws_bytes=1 << 30, ctx=True):
    ids = np.ascontiguousarray(np.atleast_2d(np.asarray(ids, np.int32)))
    blocks = dbsa.Blocks(np.full(n_blocks, 10, np.int32), 1, 2)
    out = np.zeros(ids.shape[0], np.int64)
    return lib.dbsa_gather_rope(ctypes.byref(_attn()), ctypes.byref(blocks.t),
                                ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ids.shape[1],
                                ids.shape[0], FAKE, FAKE, FAKE, FAKE, cap,
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)) if ctx else None,
                                FAKE, ws_bytes, None)


def test_gather_validation(lib):
    assert _gather(lib, [[1, 0, 2]]) == dbsa.EINVAL
    assert "anchor" in _err(lib)
    assert _gather(lib, [[0, 2, 2]]) == dbsa.EINVAL
    assert "repeats" in _err(lib)
    assert _gather(lib, [[0, 6]]) == dbsa.EINVAL
    assert _gather(lib, [[0, -1]]) == dbsa.EINVAL
    assert _gather(lib, [[0, 1], [0, 9]]) == dbsa.EINVAL
    assert _gather(lib, [[0, 1, 2]], cap=29) == dbsa.ENOSPC
    assert _gather(lib, [[0, 1, 2]], ws_bytes=8) == dbsa.ENOSPC
    assert _gather(lib, [[0, 1, 2]], ctx=False) == dbsa.EINVAL


def test_query_validation(lib):
    a = _attn()
    ctx = np.array([100, 50], np.int64)
    p64 = ctx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    args = lambda n_new, cap, ws_bytes=1 << 40: (ctypes.byref(a), 2, n_new, FAKE, FAKE, FAKE, FAKE,
                                                 FAKE, p64, cap, FAKE, FAKE, ws_bytes, None)
    assert lib.dbsa_query_attn(*args(16, 110)) == dbsa.ENOSPC
    assert lib.dbsa_query_attn(*args(-1, 1000)) == dbsa.EINVAL
    assert lib.dbsa_query_attn(*args(0, 1000)) == dbsa.OK  # no-op, nothing enqueued
    assert lib.dbsa_query_attn(*args(4, 1000, ws_bytes=4)) == dbsa.ENOSPC
    neg = np.array([-1, 5], np.int64)
    assert lib.dbsa_query_attn(ctypes.byref(a), 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE,
                               neg.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1000, FAKE,
                               FAKE, 1 << 40, None) == dbsa.EINVAL


def test_query_gathered_validation(lib):
    a = _attn()
    blocks = dbsa.Blocks([10, 20, 30], 1, 2)
    ids = np.array([[0, 3]], np.int32)
    tail = np.array([0], np.int64)
    rc = lib.dbsa_query_attn_gathered(ctypes.byref(a), ctypes.byref(blocks.t),
                                      ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, 1,
                                      FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      tail.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 8, FAKE,
                                      FAKE, 1 << 40, None)
    assert rc == dbsa.EINVAL and "out of range" in _err(lib)
    ids = np.array([[0, 2]], np.int32)
    rc = lib.dbsa_query_attn_gathered(ctypes.byref(a), ctypes.byref(blocks.t),
                                      ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, 1,
                                      FAKE, FAKE, 9, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      tail.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 8, FAKE,
                                      FAKE, 1 << 40, None)
    assert rc == dbsa.ENOSPC


def test_append_validation_and_constant_workspace(lib):
    a = _attn()
    blocks = dbsa.Blocks([64] * 10, 1, 2)
    rc = lib.dbsa_append_block(ctypes.byref(a), ctypes.byref(blocks.t), 64, FAKE, FAKE, FAKE, FAKE,
                               FAKE, 700, FAKE, FAKE, 1 << 40, None)
    assert rc == dbsa.ENOSPC and "cache" in _err(lib)
    rc = lib.dbsa_append_block(ctypes.byref(a), ctypes.byref(blocks.t), 0, FAKE, FAKE, FAKE, FAKE,
                               FAKE, 1 << 20, FAKE, FAKE, 1 << 40, None)
    assert rc == dbsa.EINVAL
    # Encoding one more block costs the same whatever the pool size
    # [Notes, Highlights]: the workspace holds only the anchor, the last j blocks
    # and the new block (plus the block-offset table).
    sizes = []
    for nb in (32, 64, 128):
        n = dbsa.dbsa_workspace_bytes(dbsa.OP_APPEND, 32, 8, 128, dbsa.BF16, 5e5, [1024] * nb, 1,
                                      2, rows=1024)
        sizes.append(n - nb * 4)
    assert max(sizes) - min(sizes) <= 1024, sizes


def test_workspace_sizes(lib):
    n1 = dbsa.dbsa_workspace_bytes(dbsa.OP_PREFILL, 32, 8, 128, dbsa.BF16, 1e4, [1024] * 30, 1, 2)
    # rotated K tile images: 8 KV heads x 480 tiles x 16 KiB (V is read in place)
    assert 8 * 480 * 64 * 128 * 2 <= n1 < 2 * 8 * 480 * 64 * 128 * 2
    assert dbsa.dbsa_workspace_bytes(dbsa.OP_PREFILL, 1, 1, 64, dbsa.F32, 1e4, [128] * 8) <= 4096
    with pytest.raises(dbsa.DbsaError):
        dbsa.dbsa_workspace_bytes(dbsa.OP_PREFILL, 3, 2, 128, dbsa.BF16, 1e4, [4])
    q = dbsa.dbsa_workspace_bytes(dbsa.OP_QUERY, 32, 8, 128, dbsa.BF16, rows=64, batch=1,
                                  max_ctx=28000)
    assert q > 0


def _span_call(lib, fn, src, ln, pool=100, cap=1 << 20, n_new=4, tail_cap=1 << 20,
               ws_bytes=1 << 40):
    src = np.ascontiguousarray(np.atleast_2d(np.asarray(src, np.int32)))
    ln = np.ascontiguousarray(np.atleast_2d(np.asarray(ln, np.int32)))
    p32 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    batch, n = src.shape
    a = _attn()
    out = np.zeros(batch, np.int64)
    if fn == "gather":
        return lib.dbsa_gather_rope_spans(ctypes.byref(a), p32(src), p32(ln), n, batch, pool,
                                          FAKE, FAKE, FAKE, FAKE, cap,
                                          out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                          FAKE, ws_bytes, None)
    return lib.dbsa_query_attn_spans(ctypes.byref(a), p32(src), p32(ln), n, batch, pool, FAKE,
                                     FAKE, n_new, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), tail_cap,
                                     FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("fn", ["gather", "query"])
def test_span_validation(lib, fn):
    assert _span_call(lib, fn, [[0, 95]], [[10, 6]]) == dbsa.EINVAL  # past the pool
    assert "outside the pool" in _err(lib)
    assert _span_call(lib, fn, [[-1, 5]], [[2, 3]]) == dbsa.EINVAL
    assert _span_call(lib, fn, [[0, 5]], [[2, -3]]) == dbsa.EINVAL
    assert _span_call(lib, fn, [[0, 5], [3, 4]], [[2, 3], [0, 0]]) == dbsa.EINVAL
    assert "selects no tokens" in _err(lib)
    assert _span_call(lib, fn, [[0, 5]], [[2, 3]], pool=0) == dbsa.EINVAL
    a = _attn()
    p = np.zeros((1, 2), np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    if fn == "gather":
        assert lib.dbsa_gather_rope_spans(ctypes.byref(a), None, p, 2, 1, 100, FAKE, FAKE, FAKE,
                                          FAKE, 100, None, FAKE, 1 << 40, None) == dbsa.EINVAL
        assert _span_call(lib, fn, [[0, 50]], [[20, 20]], cap=39) == dbsa.ENOSPC
    else:
        assert lib.dbsa_query_attn_spans(ctypes.byref(a), p, None, 2, 1, 100, FAKE, FAKE, 4,
                                         FAKE, FAKE, FAKE, FAKE, FAKE, None, 8, FAKE, FAKE,
                                         1 << 40, None) == dbsa.EINVAL
        assert _span_call(lib, fn, [[0, 5]], [[2, 3]], n_new=-1) == dbsa.EINVAL
        assert _span_call(lib, fn, [[0, 5]], [[2, 3]], n_new=0) == dbsa.OK  # nothing enqueued
        assert _span_call(lib, fn, [[0, 5]], [[2, 3]], tail_cap=3) == dbsa.ENOSPC
        # Back-to-back spans merge into one segment; 1100 separated spans
        # exceed the per-row segment table, 1100 adjacent ones do not.
        n = 1100
        gaps = np.arange(n, dtype=np.int32) * 2
        assert _span_call(lib, fn, [gaps], [np.ones(n, np.int32)], pool=4 * n) == \
            dbsa.EUNSUPPORTED
        assert "exceed" in _err(lib)
        # (A workspace too small to hold the call stops it after the span
        # checks, before anything is enqueued on the fake pointers.)
        adj = np.arange(n, dtype=np.int32)
        assert _span_call(lib, fn, [adj], [np.ones(n, np.int32)], pool=4 * n,
                          ws_bytes=16) == dbsa.ENOSPC
        assert "workspace" in _err(lib)


def test_noalloc_entry_checks_before_any_hip_call(lib):
    """The no-allocation Stage-2 entry validates like dbsa_query_attn_gathered
    and rejects, on the host, a call whose scratch would exceed its fixed
    array (255 batch rows x 2 key splits x 128 rows of fp32 partials > 32 MiB)."""
    a = dbsa.attn_t(4, 1, 128, dbsa.BF16, 1e4)
    blocks = dbsa.Blocks([200, 200, 200], 1, 2)
    p32 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    p64 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    def call(ids, n_new=32, tail=None, tail_cap=1 << 20):
        ids = np.ascontiguousarray(np.atleast_2d(np.asarray(ids, np.int32)))
        tl = np.zeros(ids.shape[0], np.int64) if tail is None else np.asarray(tail, np.int64)
        return lib.dbsa_query_attn_gathered_noalloc(
            ctypes.byref(a), ctypes.byref(blocks.t), p32(ids), ids.shape[1], ids.shape[0], FAKE,
            FAKE, n_new, FAKE, FAKE, FAKE, FAKE, FAKE, p64(tl), tail_cap, FAKE, None)
    assert call([[1, 0]]) == dbsa.EINVAL and "anchor" in _err(lib)
    assert call([[0, 1, 1]]) == dbsa.EINVAL
    assert call([[0, 1]], n_new=-1) == dbsa.EINVAL
    assert call([[0, 1]], n_new=0) == dbsa.OK  # nothing to do, nothing enqueued
    assert call([[0, 1]], tail_cap=16) == dbsa.ENOSPC and "tail_capacity" in _err(lib)
    big = np.tile(np.array([[0, 1, 2]], np.int32), (255, 1))
    assert call(big) == dbsa.ENOSPC
    assert "scratch" in _err(lib) and str(dbsa.NOALLOC_SCRATCH_BYTES) in _err(lib)


def test_batched_validation_and_workspace(lib):
    """The shared-block Stage-2 entry validates like dbsa_query_attn_gathered;
    its workspace bound covers every id choice of the shape and grows with
    the batch (partials) but not with the context."""
    a = _attn()
    blocks = dbsa.Blocks([100, 37, 250, 3, 64], 1, 2)
    p32 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    p64 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    def call(ids, n_new=4, tail=None, tail_cap=64, ws_bytes=1 << 40):
        ids = np.ascontiguousarray(np.atleast_2d(np.asarray(ids, np.int32)))
        tl = np.zeros(ids.shape[0], np.int64) if tail is None else np.asarray(tail, np.int64)
        return lib.dbsa_query_attn_batched(ctypes.byref(a), ctypes.byref(blocks.t), p32(ids),
                                           ids.shape[1], ids.shape[0], FAKE, FAKE, n_new, FAKE,
                                           FAKE, FAKE, FAKE, FAKE, p64(tl), tail_cap, FAKE, FAKE,
                                           ws_bytes, None)
    assert call([[2, 0]]) == dbsa.EINVAL and "anchor" in _err(lib)
    assert call([[0, 5]]) == dbsa.EINVAL and "out of range" in _err(lib)
    assert call([[0, 1, 1]]) == dbsa.EINVAL
    assert call([[0, 1]], n_new=-1) == dbsa.EINVAL
    assert call([[0, 1]], n_new=0) == dbsa.OK
    assert call([[0, 1]], tail=[-1]) == dbsa.EINVAL
    assert call([[0, 1]], tail=[62]) == dbsa.ENOSPC and "tail_capacity" in _err(lib)
    assert call([[0, 1]], ws_bytes=1024) == dbsa.ENOSPC and "workspace" in _err(lib)
    lens = [1024] * 90
    ws = lambda batch, n_new=48, tail=0: dbsa.dbsa_workspace_bytes(
        dbsa.OP_QUERY_BATCHED, 32, 8, 128, dbsa.BF16, 5e5, lens, 1, 2, rows=n_new, batch=batch,
        n_ids=28, max_ctx=tail + n_new)
    # K of every block (8 heads x 1440 tiles x 16 KiB) + bf16 partials and their weights
    k_img = 8 * 90 * 16 * 16384
    part = 64 * 8 * 28 * 192 * (256 + 4)
    assert k_img + part <= ws(64) < k_img + part + (64 << 20)
    assert ws(32) < ws(64)
    # a bound: the size does not depend on which blocks the rows select
    assert ws(64) == ws(64)
    with pytest.raises(dbsa.DbsaError):
        dbsa.dbsa_workspace_bytes(dbsa.OP_QUERY_BATCHED, 32, 8, 128, dbsa.BF16, 5e5, lens, 1, 2,
                                  rows=48, batch=64, n_ids=0, max_ctx=48)

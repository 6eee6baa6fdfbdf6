"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects malformed arguments on the host before any HIP
call (with the documented status codes)."""
import ctypes
import os
import re

import numpy as np
import pytest

from block_sparse_attention_sink_amd import dbsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # aligned, never dereferenced: every case below fails validation first


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

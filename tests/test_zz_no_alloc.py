"""The no-allocation Stage-2 entry point against the one with a workspace.

dbsa_query_attn_gathered_noalloc runs the same kernels and plan as
dbsa_query_attn_gathered with the library's static scratch array instead of a
workspace, so outputs and the tail buffers it appends to must agree bitwise.
Two calls in a row, the second smaller (it reuses the scratch the first left
behind), then a check against the oracle on one batch row.
"""
import numpy as np
import pytest
import torch

from oracle import dbsa_oracle as orc
from block_sparse_attention_sink_amd import dbsa
from block_sparse_attention_sink_amd.inputs import randn, select_ids
from tests.helpers import assert_close, host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(lens, ids, n_new, tail_len, hq, hkv, d, seed):
    batch = ids.shape[0]
    n = int(lens.sum())
    k = randn((n, hkv, d), seed, "bf16", DEV)
    v = randn((n, hkv, d), seed + 1, "bf16", DEV)
    q = randn((batch, n_new, hq, d), seed + 2, "bf16", DEV)
    kn = randn((batch, n_new, hkv, d), seed + 3, "bf16", DEV)
    vn = randn((batch, n_new, hkv, d), seed + 4, "bf16", DEV)
    cap = max(tail_len) + n_new
    tk = randn((batch, cap, hkv, d), seed + 5, "bf16", DEV)  # rows < tail_len: earlier tokens
    tv = randn((batch, cap, hkv, d), seed + 6, "bf16", DEV)
    return k, v, q, kn, vn, tk, tv


def _compare(lens, ids, n_new, tail_len, hq, hkv, d, seed, theta):
    k, v, q, kn, vn, tk, tv = _case(lens, ids, n_new, tail_len, hq, hkv, d, seed)
    tk2, tv2 = tk.clone(), tv.clone()
    want = dbsa.dbsa_query_attn_gathered(q, kn, vn, k, v, lens, ids, tk, tv, tail_len, theta)
    got = dbsa.dbsa_query_attn_gathered_noalloc(q, kn, vn, k, v, lens, ids, tk2, tv2, tail_len,
                                                theta)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert torch.equal(tk2, tk) and torch.equal(tv2, tv)
    return k, v, q, kn, vn, tk, tv, got


def test_noalloc_equals_workspace_entry_two_calls():
    rng = np.random.default_rng(2024)
    theta = 5e5
    # call 1: GQA 32/8, 2 batch rows with their own anchor + 12 blocks, 64 new
    # tokens each (256 packed rows per KV head, split-K partials in scratch)
    lens = rng.integers(50, 300, size=40).astype(np.int32)
    ids = np.stack([select_ids(rng, 40, 12) for _ in range(2)])
    k, v, q, kn, vn, tk, tv, got = _compare(lens, ids, 64, [0, 0], 32, 8, 128, 700, theta)
    # the first batch row against the oracle too
    kg, vg = orc.gather_rope(host64(k), host64(v), lens, ids[0], theta)
    want, _, _ = orc.query_attn(host64(q[0]), host64(kn[0]), host64(vn[0]), kg, vg, theta)
    assert_close(host64(got[0]), want, "bf16", "noalloc call 1, row 0")
    # call 2, smaller: one batch row, anchor + 3 blocks, 5 new tokens after 7
    # tokens already in the tail (a decode-like continuation)
    ids2 = np.array([[0, 4, 9, 31]], np.int32)
    k, v, q, kn, vn, tk, tv, got = _compare(lens, ids2, 5, [7], 32, 8, 128, 800, theta)
    kg, vg = orc.gather_rope(host64(k), host64(v), lens, ids2[0], theta)
    # the 7 tail tokens sit after the gathered ones, already rotated
    t_prev = host64(tk[0, :7])
    want, _, _ = orc.query_attn(host64(q[0]), host64(kn[0]), host64(vn[0]),
                                np.concatenate([kg, t_prev]),
                                np.concatenate([vg, host64(tv[0, :7])]), theta)
    assert_close(host64(got[0]), want, "bf16", "noalloc call 2")

"""GPU parity of the shared-block Stage-2 schedule (dbsa_query_attn_batched).

Every batch row's output is compared with the oracle's gather + re-RoPE +
query attention [Notes, Method > Stage 2, items 1-4]; the rows' own tail
tokens and the new tokens' K/V written back are checked too.  Cases cover
GQA group sizes 1-8, head_dim 64 and 128, packed row counts that are and are
not multiples of 32 (and above one 256-row workgroup), blocks of one token,
ids out of encoded order, rows sharing every block, and the full 32-layer
pool workload (all 64 queries on two layers).
"""
import numpy as np
import pytest
import torch

from oracle import dbsa_oracle as orc
from block_sparse_attention_sink_amd import dbsa
from block_sparse_attention_sink_amd.inputs import randn, workload
from tests.helpers import assert_bf16_rounding, assert_close, host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ids(rng, n_blocks, batch, n_pick, shuffle=True):
    rows = []
    for _ in range(batch):
        pick = rng.choice(np.arange(1, n_blocks), size=n_pick, replace=False)
        if not shuffle:
            pick = np.sort(pick)
        rows.append(np.concatenate([[0], pick]))
    return np.asarray(rows, np.int32)


def _inputs(lens, batch, n_new, tail_len, hq, hkv, d, seed):
    n = int(np.sum(lens))
    k = randn((n, hkv, d), seed, "bf16", DEV)
    v = randn((n, hkv, d), seed + 1, "bf16", DEV)
    q = randn((batch, n_new, hq, d), seed + 2, "bf16", DEV)
    kn = randn((batch, n_new, hkv, d), seed + 3, "bf16", DEV)
    vn = randn((batch, n_new, hkv, d), seed + 4, "bf16", DEV)
    cap = max(tail_len) + n_new
    # rows [0, tail_len) of the tail buffers: earlier tokens, K already rotated
    tk = randn((batch, cap, hkv, d), seed + 5, "bf16", DEV)
    tv = randn((batch, cap, hkv, d), seed + 6, "bf16", DEV)
    return k, v, q, kn, vn, tk, tv


def _check_rows(lens, ids, tail_len, k, v, q, kn, vn, tk0, tv0, tk, tv, out, theta, what,
                rows=None):
    kh, vh = host64(k), host64(v)
    n_new = q.shape[1]
    for b in (range(ids.shape[0]) if rows is None else rows):
        kg, vg = orc.gather_rope(kh, vh, lens, ids[b], theta)
        t = int(tail_len[b])
        kc = np.concatenate([kg, host64(tk0[b, :t])])
        vc = np.concatenate([vg, host64(tv0[b, :t])])
        want, k_all, _ = orc.query_attn(host64(q[b]), host64(kn[b]), host64(vn[b]), kc, vc, theta)
        assert_close(host64(out[b]), want, "bf16", f"{what} row {b}")
        # the new tokens' K (rotated at T' + tail + r) and V went to the tail buffer
        assert_bf16_rounding(host64(tk[b, t:t + n_new]), k_all[kc.shape[0]:],
                             f"{what} row {b} new K")
        assert torch.equal(tv[b, t:t + n_new], vn[b])
        assert torch.equal(tk[b, :t], tk0[b, :t]) and torch.equal(tv[b, :t], tv0[b, :t])


@pytest.mark.parametrize("hq,hkv,d,n_new", [(8, 2, 128, 7), (4, 4, 64, 33), (32, 8, 128, 1),
                                            (16, 2, 128, 40)])
def test_batched_matches_oracle(hq, hkv, d, n_new):
    rng = np.random.default_rng(1000 + hq + n_new)
    lens = rng.integers(1, 300, size=12).astype(np.int32)
    lens[[3, 7]] = 1  # one-token blocks
    batch = 5
    ids = _ids(rng, lens.size, batch, 4)
    tail_len = np.array([0, 3, 0, 17, 1], np.int64)
    k, v, q, kn, vn, tk, tv = _inputs(lens, batch, n_new, tail_len, hq, hkv, d, 41 + n_new)
    tk0, tv0 = tk.clone(), tv.clone()
    out = dbsa.dbsa_query_attn_batched(q, kn, vn, k, v, lens, ids, tk, tv, tail_len, 5e5)
    torch.cuda.synchronize()
    _check_rows(lens, ids, tail_len, k, v, q, kn, vn, tk0, tv0, tk, tv, out, 5e5,
                f"batched hq={hq} hkv={hkv} d={d} n_new={n_new}")


def test_batched_agrees_with_per_query_schedule():
    """Both schedules on the same inputs: each within the oracle tolerance,
    and within a few bf16 roundings of each other."""
    rng = np.random.default_rng(77)
    lens = rng.integers(40, 500, size=20).astype(np.int32)
    batch, n_new = 9, 16
    ids = _ids(rng, lens.size, batch, 6, shuffle=False)
    tail_len = np.zeros(batch, np.int64)
    k, v, q, kn, vn, tk, tv = _inputs(lens, batch, n_new, tail_len, 32, 8, 128, 91)
    tk2, tv2 = tk.clone(), tv.clone()
    a = dbsa.dbsa_query_attn_batched(q, kn, vn, k, v, lens, ids, tk, tv, tail_len, 1e4)
    b = dbsa.dbsa_query_attn_gathered(q, kn, vn, k, v, lens, ids, tk2, tv2, tail_len, 1e4)
    torch.cuda.synchronize()
    diff = (a.float() - b.float()).abs()
    assert diff.max().item() <= 4e-3, diff.max().item()
    assert torch.equal(tv, tv2)
    _check_rows(lens, ids, tail_len, k, v, q, kn, vn, tk2.clone().zero_(), tv2, tk, tv, a, 1e4,
                "batched vs oracle", rows=[0, 4, 8])


def test_batched_shared_and_anchor_only_rows():
    """Every row selecting the same blocks (each tile shared by the whole batch),
    then one-id rows (the anchor alone), with decode-length tails."""
    rng = np.random.default_rng(5)
    lens = rng.integers(20, 200, size=6).astype(np.int32)
    batch, n_new = 12, 3
    ids = np.tile(np.array([[0, 5, 2, 3]], np.int32), (batch, 1))
    tail_len = rng.integers(0, 30, size=batch).astype(np.int64)
    k, v, q, kn, vn, tk, tv = _inputs(lens, batch, n_new, tail_len, 8, 2, 128, 301)
    tk0, tv0 = tk.clone(), tv.clone()
    out = dbsa.dbsa_query_attn_batched(q, kn, vn, k, v, lens, ids, tk, tv, tail_len, 1e4)
    torch.cuda.synchronize()
    _check_rows(lens, ids, tail_len, k, v, q, kn, vn, tk0, tv0, tk, tv, out, 1e4, "all shared")
    ids1 = np.zeros((batch, 1), np.int32)
    k, v, q, kn, vn, tk, tv = _inputs(lens, batch, n_new, tail_len, 8, 2, 128, 401)
    tk0, tv0 = tk.clone(), tv.clone()
    out = dbsa.dbsa_query_attn_batched(q, kn, vn, k, v, lens, ids1, tk, tv, tail_len, 1e4)
    torch.cuda.synchronize()
    _check_rows(lens, ids1, tail_len, k, v, q, kn, vn, tk0, tv0, tk, tv, out, 1e4, "anchor only")


def test_batched_repeatable_bitwise():
    rng = np.random.default_rng(8)
    lens = rng.integers(50, 400, size=15).astype(np.int32)
    ids = _ids(rng, lens.size, 6, 5)
    tail_len = np.zeros(6, np.int64)
    k, v, q, kn, vn, tk, tv = _inputs(lens, 6, 24, tail_len, 32, 8, 128, 501)
    o1 = dbsa.dbsa_query_attn_batched(q, kn, vn, k, v, lens, ids, tk, tv, tail_len, 5e5).clone()
    o2 = dbsa.dbsa_query_attn_batched(q, kn, vn, k, v, lens, ids, tk, tv, tail_len, 5e5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("layer", [0, 1])
def test_pool_batch_all_queries_full_size(layer):
    """The 32-layer Llama-3.1 pool (89,568 tokens, 8 KV heads): all 64 queries,
    each with the anchor + its own 27 blocks and 48 query tokens, on one layer
    of a two-layer slice of the pool, every output row against the oracle."""
    w = workload(4)
    n = w.n_tokens
    pool_k = randn((2, n, w.n_kv_heads, w.head_dim), 700, "bf16", DEV)
    pool_v = randn((2, n, w.n_kv_heads, w.head_dim), 701, "bf16", DEV)
    k, v = pool_k[layer], pool_v[layer]
    b = w.batch
    q = randn((b, w.n_new, w.n_q_heads, w.head_dim), 702 + layer, "bf16", DEV)
    kn = randn((b, w.n_new, w.n_kv_heads, w.head_dim), 704 + layer, "bf16", DEV)
    vn = randn((b, w.n_new, w.n_kv_heads, w.head_dim), 706 + layer, "bf16", DEV)
    tk = torch.zeros((b, w.n_new, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    tv = torch.zeros_like(tk)
    out = dbsa.dbsa_query_attn_batched(q, kn, vn, k, v, w.block_lens, w.ids, tk, tv, [0] * b,
                                       w.theta)
    torch.cuda.synchronize()
    kh, vh = host64(k), host64(v)
    oh = host64(out)
    for r in range(b):
        kg, vg = orc.gather_rope(kh, vh, w.block_lens, w.ids[r], w.theta)
        want, _, _ = orc.query_attn(host64(q[r]), host64(kn[r]), host64(vn[r]), kg, vg, w.theta)
        assert_close(oh[r], want, "bf16", f"pool layer {layer} query {r}")

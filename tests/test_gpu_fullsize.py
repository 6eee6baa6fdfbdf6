"""GPU parity at the five workloads' full sizes.

The GPU runs each operation at full size, in the same launch configuration
the benchmark times; the CPU oracle evaluates sampled rows (prefill) or
sampled batch rows (Stage 2) one by one.  Row samples cover the first and
last rows of the anchor, the first j+1 blocks, a middle block and the last
block, plus seeded random rows.
"""
import numpy as np
import pytest
import torch

from oracle import dbsa_oracle as orc
from block_sparse_attention_sink_amd import dbsa
from block_sparse_attention_sink_amd.inputs import PATTERNS, randn, workload
from tests.helpers import assert_close, host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _sample_rows(lens, j, per_edge=12, n_random=24, seed=0):
    off = np.concatenate([[0], np.cumsum(lens)])
    nb = len(lens)
    blocks = sorted({0, 1 % nb, min(j, nb - 1), min(j + 1, nb - 1), nb // 2, nb - 1})
    rows = []
    for b in blocks:
        rows += list(range(off[b], min(off[b] + per_edge, off[b + 1])))
        rows += list(range(max(off[b + 1] - per_edge, off[b]), off[b + 1]))
    rng = np.random.default_rng(seed)
    rows += list(rng.integers(0, off[-1], size=n_random))
    return np.unique(np.asarray(rows, dtype=np.int64))


def _qkv(w, seed):
    n = w.n_tokens
    return (randn((n, w.n_q_heads, w.head_dim), seed, w.dtype, DEV),
            randn((n, w.n_kv_heads, w.head_dim), seed + 1, w.dtype, DEV),
            randn((n, w.n_kv_heads, w.head_dim), seed + 2, w.dtype, DEV))


def _check_prefill_rows(w, q, k, v, o, sink, j, rows, what):
    # The oracle takes the full Q; only the sampled rows are evaluated.
    qh = np.zeros((w.n_tokens,) + tuple(q.shape[1:]))
    qh[rows] = host64(q[torch.as_tensor(rows, device=q.device)])
    want = orc.prefill(qh, host64(k), host64(v), w.block_lens, sink, j, w.theta, rows=rows)
    got = host64(o[torch.as_tensor(rows, device=o.device)])
    assert_close(got, want, w.dtype, what)


def test_tiny_f32_workload_all_stages():
    """8 x 128 tokens, 1 head, d = 64, float32: every row and every stage."""
    w = workload(1)
    q, k, v = _qkv(w, 10)
    o = dbsa.dbsa_prefill(q, k, v, w.block_lens, w.sink, w.j, w.theta)
    kg, vg, ctx = dbsa.dbsa_gather_rope(k, v, w.block_lens, w.ids, w.theta,
                                        capacity=int(w.block_lens[w.ids[0]].sum()) + w.n_new)
    qn = randn((1, w.n_new, 1, w.head_dim), 20, "f32", DEV)
    kn = randn((1, w.n_new, 1, w.head_dim), 21, "f32", DEV)
    vn = randn((1, w.n_new, 1, w.head_dim), 22, "f32", DEV)
    on = dbsa.dbsa_query_attn(qn, kn, vn, kg, vg, ctx, w.theta)
    tail = torch.zeros((1, w.n_new, 1, w.head_dim), dtype=torch.float32, device=DEV)
    of = dbsa.dbsa_query_attn_gathered(qn, kn, vn, k, v, w.block_lens, w.ids, tail,
                                       torch.zeros_like(tail), [0], w.theta)
    torch.cuda.synchronize()
    assert_close(host64(o), orc.prefill(host64(q), host64(k), host64(v), w.block_lens, w.sink,
                                        w.j, w.theta), "f32", "tiny prefill")
    kgo, vgo = orc.gather_rope(host64(k), host64(v), w.block_lens, w.ids[0], w.theta)
    assert ctx[0] == 384
    assert_close(host64(kg[0, :384]), kgo, "f32", "tiny gather K")
    np.testing.assert_array_equal(host64(vg[0, :384]), vgo)
    want, _, _ = orc.query_attn(host64(qn[0]), host64(kn[0]), host64(vn[0]), kgo, vgo, w.theta)
    assert_close(host64(on[0]), want, "f32", "tiny query")
    assert_close(host64(of[0]), want, "f32", "tiny fused query")


@pytest.mark.parametrize("k_cfg", [2, 3])
def test_prefill_full_size_sampled_rows(k_cfg):
    w = workload(k_cfg)
    q, k, v = _qkv(w, 100 + k_cfg)
    o = torch.full_like(q, float("nan"))
    dbsa.dbsa_prefill(q, k, v, w.block_lens, w.sink, w.j, w.theta, out=o)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any(), "some output rows were never written"
    rows = _sample_rows(w.block_lens, w.j, seed=k_cfg)
    _check_prefill_rows(w, q, k, v, o, w.sink, w.j, rows, f"workload {k_cfg} prefill")


@pytest.mark.parametrize("pattern", list(PATTERNS))
def test_stress_patterns_full_size(pattern):
    """128 blocks of 512-2048 tokens (131072 tokens), GQA 32/8: each mask pattern."""
    w = workload(5)
    sink, j = PATTERNS[pattern]
    if j < 0:
        j = w.n_blocks - 1
    q, k, v = _qkv(w, 500)
    o = dbsa.dbsa_prefill(q, k, v, w.block_lens, sink, j, w.theta)
    torch.cuda.synchronize()
    rows = _sample_rows(w.block_lens, j, per_edge=8, n_random=40, seed=5)
    _check_prefill_rows(w, q, k, v, o, sink, j, rows, f"stress {pattern}")


def test_stress_append_one_block():
    """Append a 1024-token block onto the 131072-token pool (sink + previous 2)."""
    w = workload(5)
    new_len = w.append_len
    n_old = w.n_tokens
    k_cache = torch.empty((n_old + new_len, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16,
                          device=DEV)
    v_cache = torch.empty_like(k_cache)
    k_cache[:n_old] = randn((n_old, w.n_kv_heads, w.head_dim), 601, "bf16", DEV)
    v_cache[:n_old] = randn((n_old, w.n_kv_heads, w.head_dim), 602, "bf16", DEV)
    qn = randn((new_len, w.n_q_heads, w.head_dim), 603, "bf16", DEV)
    kn = randn((new_len, w.n_kv_heads, w.head_dim), 604, "bf16", DEV)
    vn = randn((new_len, w.n_kv_heads, w.head_dim), 605, "bf16", DEV)
    on = dbsa.dbsa_append_block(qn, kn, vn, k_cache, v_cache, w.block_lens, w.sink, w.j,
                                w.theta)
    torch.cuda.synchronize()
    assert torch.equal(k_cache[n_old:], kn) and torch.equal(v_cache[n_old:], vn)
    lens2 = np.append(w.block_lens, new_len)
    sample = np.unique(np.concatenate([np.arange(0, 16), np.arange(new_len - 16, new_len),
                                       np.random.default_rng(6).integers(0, new_len, 16)]))
    rows = n_old + sample
    qh = np.zeros((n_old + new_len, w.n_q_heads, w.head_dim))
    qh[rows] = host64(qn[torch.as_tensor(sample, device=DEV)])
    want = orc.prefill(qh, host64(k_cache), host64(v_cache), lens2, w.sink, w.j, w.theta,
                       rows=rows)
    assert_close(host64(on[torch.as_tensor(sample, device=DEV)]), want, "bf16", "stress append")


@pytest.mark.parametrize("k_cfg", [2, 3])
@pytest.mark.parametrize("fused", [False, True])
def test_stage2_full_size(k_cfg, fused):
    """Anchor + 30% of the blocks, 64 query tokens (+ 16 decode steps for workload 3)."""
    w = workload(k_cfg)
    _, k, v = _qkv(w, 200 + k_cfg)
    ids = w.ids
    tp = int(w.block_lens[ids[0]].sum())
    steps = w.decode_steps
    n_all = w.n_new + steps
    qn = randn((1, n_all, w.n_q_heads, w.head_dim), 210, "bf16", DEV)
    kn = randn((1, n_all, w.n_kv_heads, w.head_dim), 211, "bf16", DEV)
    vn = randn((1, n_all, w.n_kv_heads, w.head_dim), 212, "bf16", DEV)
    sl = lambda t, a, b: t[:, a:b].contiguous()
    outs = []
    if fused:
        tk = torch.zeros((1, n_all, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
        tv = torch.zeros_like(tk)
        outs.append(dbsa.dbsa_query_attn_gathered(sl(qn, 0, w.n_new), sl(kn, 0, w.n_new),
                                                  sl(vn, 0, w.n_new), k, v, w.block_lens, ids,
                                                  tk, tv, [0], w.theta))
        for s in range(steps):
            a = w.n_new + s
            outs.append(dbsa.dbsa_query_attn_gathered(sl(qn, a, a + 1), sl(kn, a, a + 1),
                                                      sl(vn, a, a + 1), k, v, w.block_lens, ids,
                                                      tk, tv, [a], w.theta))
    else:
        kg, vg, ctx = dbsa.dbsa_gather_rope(k, v, w.block_lens, ids, w.theta, capacity=tp + n_all)
        outs.append(dbsa.dbsa_query_attn(sl(qn, 0, w.n_new), sl(kn, 0, w.n_new),
                                         sl(vn, 0, w.n_new), kg, vg, ctx, w.theta))
        for s in range(steps):
            a = w.n_new + s
            outs.append(dbsa.dbsa_query_attn(sl(qn, a, a + 1), sl(kn, a, a + 1), sl(vn, a, a + 1),
                                             kg, vg, [tp + a], w.theta))
    torch.cuda.synchronize()
    kgo, vgo = orc.gather_rope(host64(k), host64(v), w.block_lens, ids[0], w.theta)
    want, kc, vc = orc.query_attn(host64(qn[0, :w.n_new]), host64(kn[0, :w.n_new]),
                                  host64(vn[0, :w.n_new]), kgo, vgo, w.theta)
    assert_close(host64(outs[0][0]), want, "bf16", f"workload {k_cfg} query fused={fused}")
    if steps:
        dec, _, _ = orc.decode([host64(qn[0, w.n_new + s:w.n_new + s + 1]) for s in range(steps)],
                               [host64(kn[0, w.n_new + s:w.n_new + s + 1]) for s in range(steps)],
                               [host64(vn[0, w.n_new + s:w.n_new + s + 1]) for s in range(steps)],
                               kc, vc, w.theta)
        for s in range(steps):
            assert_close(host64(outs[1 + s][0]), dec[s], "bf16", f"decode step {s}")


@pytest.mark.parametrize("fused", [False, True])
def test_pool_batch_one_layer(fused):
    """32-layer pool layout, 64 queries each with its own anchor + 27 blocks, 48 tokens.

    Layer 1 of a 2-layer slice of the pool is used (pointer offset into the
    [layer][token][head][d] pool); four batch rows are checked.
    """
    w = workload(4)
    n = w.n_tokens
    pool_k = randn((2, n, w.n_kv_heads, w.head_dim), 300, "bf16", DEV)
    pool_v = randn((2, n, w.n_kv_heads, w.head_dim), 301, "bf16", DEV)
    k, v = pool_k[1], pool_v[1]
    b = w.batch
    qn = randn((b, w.n_new, w.n_q_heads, w.head_dim), 302, "bf16", DEV)
    kn = randn((b, w.n_new, w.n_kv_heads, w.head_dim), 303, "bf16", DEV)
    vn = randn((b, w.n_new, w.n_kv_heads, w.head_dim), 304, "bf16", DEV)
    if fused:
        tk = torch.zeros((b, w.n_new, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
        o = dbsa.dbsa_query_attn_gathered(qn, kn, vn, k, v, w.block_lens, w.ids, tk,
                                          torch.zeros_like(tk), [0] * b, w.theta)
    else:
        cap = int(max(w.block_lens[r].sum() for r in w.ids)) + w.n_new
        kg, vg, ctx = dbsa.dbsa_gather_rope(k, v, w.block_lens, w.ids, w.theta, capacity=cap)
        o = dbsa.dbsa_query_attn(qn, kn, vn, kg, vg, ctx, w.theta)
    torch.cuda.synchronize()
    kh, vh = host64(k), host64(v)
    for r in (0, 17, 40, 63):
        kgo, vgo = orc.gather_rope(kh, vh, w.block_lens, w.ids[r], w.theta)
        want, _, _ = orc.query_attn(host64(qn[r]), host64(kn[r]), host64(vn[r]), kgo, vgo, w.theta)
        assert_close(host64(o[r]), want, "bf16", f"pool batch row {r} fused={fused}")

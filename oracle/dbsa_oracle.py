"""Reference oracle for Dynamic Block-Sparse Attention (DBSA).

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` call it.  It shares no code, constants or helpers with the HIP
path: it is plain NumPy in float64 with no blocking, fusion or reordering
beyond what the definitions below state.

Source of every definition: the paper-notes page "Efficient Many-Shot
In-Context Learning with Dynamic Block-Sparse Attention" (zhaoyang97
Paper-Notes, ACL 2025, arXiv 2503.08640), cited below as [Notes, <section>].

Readings taken where the page is silent (each one is listed in the design
document):
  * positions are token positions; block lengths are given in tokens;
  * RoPE is the rotate-half form: pair (i, i + d/2) is rotated by p * w_i with
    w_i = theta ** (-2 i / d), no frequency scaling (a caller may pass its own
    w_i table instead of theta);
  * the sink is the whole first block; previous blocks and the sink are seen in
    full, the own block causally (diagonal included);
  * softmax scale is 1/sqrt(d) unless given; GQA maps q head h to kv head
    h // (Hq / Hkv);
  * the query tokens of Stage 2 see the whole gathered cache and each other
    causally, at positions continuing after the gathered tokens.

Parity status: every function here is pinned by a CPU test against a closed
form, a library routine or a brute-force computation (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "offsets",
    "token_block",
    "rope",
    "visible",
    "masked_attention",
    "prefill",
    "append_block",
    "gather_rope",
    "gather_rope_spans",
    "query_attn",
    "decode",
]


def offsets(block_lens) -> np.ndarray:
    """Start token of every block plus the total, [Notes, Method > Stage 1, item 1].

    The demonstration set is cut into consecutive blocks b_1 .. b_{n/k}; with
    block lengths L_i (tokens) block i covers tokens [off[i], off[i+1]).
    """
    lens = np.asarray(block_lens, dtype=np.int64)
    out = np.zeros(lens.size + 1, dtype=np.int64)
    out[1:] = np.cumsum(lens)
    return out


def token_block(block_lens) -> np.ndarray:
    """Block index of every token of the concatenated pool."""
    lens = np.asarray(block_lens, dtype=np.int64)
    return np.repeat(np.arange(lens.size, dtype=np.int64), lens)


def rope(x: np.ndarray, pos, theta) -> np.ndarray:
    """Rotary position transform of x [T, H, d] at integer positions pos [T].

    [Notes, Method > Stage 1, item 3] (sequential positions, K/V kept before the
    rotary transform) and [Notes, Method > Stage 2, item 3] (re-applied at new
    positions).  The page gives no formula; the rotate-half form is used: for
    i < d/2, w_i = theta^(-2i/d), phi = p * w_i (float64) and
        (x_i, x_{i+d/2}) -> (x_i cos phi - x_{i+d/2} sin phi,
                             x_{i+d/2} cos phi + x_i sin phi).
    `theta` may instead be the d/2 angular frequencies w_i themselves (radians
    per position), for frequency-scaled variants the page leaves open.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    if np.ndim(theta) == 0:
        w = float(theta) ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    else:
        w = np.asarray(theta, dtype=np.float64).reshape(half)
    phi = np.asarray(pos, dtype=np.float64)[:, None] * w[None, :]  # [T, d/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    a = x[..., :half]
    b = x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def visible(block_lens, sink: int, j: int, rows=None) -> np.ndarray:
    """Boolean visibility matrix [len(rows), N], [Notes, Method > Stage 1, item 2].

    Block b_i attends to the anchor block b_1 (the attention sink), to the
    previous j blocks b_{i-j} .. b_{i-1} and causally to itself.  With 0-based
    blocks, key s is visible to query t iff
        s <= t  and  (blk(s) >= blk(t) - j  or  (sink and blk(s) == 0)).
    The ablation patterns of [Notes, Ablations > sparse attention pattern] are
    parameter choices: self-only (sink 0, j 0), sink+self (1, 0), DBSA (1, j),
    full causal attention (any j >= n_blocks - 1).
    """
    blk = token_block(block_lens)
    n = blk.size
    t = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    s = np.arange(n, dtype=np.int64)
    bt = blk[t][:, None]
    bs = blk[s][None, :]
    near = bs >= bt - int(j)
    anchor = (bs == 0) if sink else np.zeros_like(near)
    return (s[None, :] <= t[:, None]) & (near | anchor)


def masked_attention(q_rot, k_rot, v, mask, scale: float) -> np.ndarray:
    """Softmax attention of rotated queries over rotated keys under a mask.

    q_rot [R, Hq, d], k_rot [S, Hkv, d], v [S, Hkv, d], mask [R, S] boolean.
    Query head h reads kv head h // (Hq / Hkv).  For each row the weights are
    exp(score - max) over the visible keys, normalised to sum 1.
    """
    q_rot = np.asarray(q_rot, dtype=np.float64)
    k_rot = np.asarray(k_rot, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    r, hq, d = q_rot.shape
    hkv = k_rot.shape[1]
    group = hq // hkv
    out = np.empty((r, hq, v.shape[-1]), dtype=np.float64)
    for h in range(hq):
        g = h // group
        scores = scale * (q_rot[:, h, :] @ k_rot[:, g, :].T)  # [R, S]
        scores = np.where(mask, scores, -np.inf)
        top = scores.max(axis=1, keepdims=True)
        w = np.exp(scores - top)  # exp(-inf) == 0 for hidden keys
        out[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def _scale(d: int, scale):
    return 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)


def prefill(q, k, v, block_lens, sink: int, j: int, theta: float, scale=None,
            rows=None, row_chunk: int = 512) -> np.ndarray:
    """Stage-1 block-sparse streaming encoding of one attention layer.

    [Notes, Method > Stage 1, items 2-3]: tokens sit at sequential positions
    0..N-1; Q and K are rotated there; each row attends to the keys
    ``visible`` allows.  Returns O [len(rows), Hq, d] (all rows by default).
    The K/V cache this stage leaves behind is the caller's K and V, unrotated.
    Rows are processed in chunks of ``row_chunk`` only to bound memory; each
    row's arithmetic does not depend on the chunking.
    """
    q = np.asarray(q, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    sc = _scale(q.shape[-1], scale)
    k_rot = rope(k, np.arange(n), theta)
    out = np.empty((rows.size, q.shape[1], np.asarray(v).shape[-1]), dtype=np.float64)
    for a in range(0, rows.size, row_chunk):
        rr = rows[a:a + row_chunk]
        q_rot = rope(q[rr], rr, theta)
        out[a:a + row_chunk] = masked_attention(q_rot, k_rot, v,
                                                visible(block_lens, sink, j, rr), sc)
    return out


def append_block(q_new, k_new, v_new, k_cache, v_cache, block_lens, sink: int,
                 j: int, theta: float, scale=None):
    """Encode one more block onto an existing pool, [Notes, Method > Stage 1, item 4].

    The new block becomes block n_b at positions N .. N+L_new-1 and is encoded
    under the same mask as every other block.  Returns (O_new, K', V', lens')
    with the caches extended by the new, unrotated K/V.
    """
    lens = list(np.asarray(block_lens, dtype=np.int64)) + [np.asarray(q_new).shape[0]]
    k_all = np.concatenate([np.asarray(k_cache, np.float64), np.asarray(k_new, np.float64)])
    v_all = np.concatenate([np.asarray(v_cache, np.float64), np.asarray(v_new, np.float64)])
    n_old = np.asarray(k_cache).shape[0]
    n_all = k_all.shape[0]
    # Only the new rows are computed; their Q rows are the new block's Q.
    q_all = np.zeros((n_all,) + np.asarray(q_new).shape[1:], dtype=np.float64)
    q_all[n_old:] = np.asarray(q_new, np.float64)
    o_new = prefill(q_all, k_all, v_all, lens, sink, j, theta, scale,
                    rows=np.arange(n_old, n_all))
    return o_new, k_all, v_all, np.asarray(lens, dtype=np.int64)


def gather_rope(k_pool, v_pool, block_lens, ids, theta: float):
    """Stage-2 KV assembly, [Notes, Method > Stage 2, items 1-3].

    ids lists the selected blocks, anchor (block 0) first, in the order the
    caller wants them placed.  The cached (unrotated) K/V of those blocks are
    concatenated and K is rotated at the new sequential positions 0..T'-1;
    V is not rotated.  Returns (K_g, V_g) of T' tokens.
    """
    off = offsets(block_lens)
    ids = [int(b) for b in ids]
    k_sel = np.concatenate([np.asarray(k_pool, np.float64)[off[b]:off[b + 1]] for b in ids])
    v_sel = np.concatenate([np.asarray(v_pool, np.float64)[off[b]:off[b + 1]] for b in ids])
    return rope(k_sel, np.arange(k_sel.shape[0]), theta), v_sel


def gather_rope_spans(k_pool, v_pool, span_src, span_len, theta):
    """Stage-2 KV assembly at example granularity, [Notes, Ablations >
    block-level vs example-level retrieval]: the cached K/V of the pool token
    spans [src, src + len), in the given order, concatenated; K rotated at the
    new sequential positions 0..T'-1, V not rotated."""
    k_pool = np.asarray(k_pool, np.float64)
    v_pool = np.asarray(v_pool, np.float64)
    idx = np.concatenate([np.arange(int(s), int(s) + int(n), dtype=np.int64)
                          for s, n in zip(span_src, span_len)])
    k_sel, v_sel = k_pool[idx], v_pool[idx]
    return rope(k_sel, np.arange(k_sel.shape[0]), theta), v_sel


def query_attn(q, k_new, v_new, k_ctx_rot, v_ctx, theta: float, scale=None):
    """Query tokens over the gathered cache, [Notes, Method > Stage 2, item 4].

    The ctx_len = len(k_ctx_rot) cached tokens are seen in full; the n_new
    query tokens sit at positions ctx_len + r, are rotated there, and see each
    other causally.  Returns (O [n_new, Hq, d], K_c, V_c) where the caches are
    extended by the new tokens (K rotated, V as given).
    """
    q = np.asarray(q, np.float64)
    ctx = np.asarray(k_ctx_rot).shape[0]
    n_new = q.shape[0]
    pos = ctx + np.arange(n_new)
    k_c = np.concatenate([np.asarray(k_ctx_rot, np.float64), rope(k_new, pos, theta)])
    v_c = np.concatenate([np.asarray(v_ctx, np.float64), np.asarray(v_new, np.float64)])
    s = np.arange(ctx + n_new)
    mask = s[None, :] <= pos[:, None]
    o = masked_attention(rope(q, pos, theta), k_c, v_c, mask, _scale(q.shape[-1], scale))
    return o, k_c, v_c


def decode(qs, ks, vs, k_ctx_rot, v_ctx, theta: float, scale=None):
    """Autoregressive steps after the query, [Notes, Method > Stage 2, item 4].

    Step s appends one token (qs[s], ks[s], vs[s], each [1, H, d]) at the next
    position and attends to everything before it and itself.  Returns the list
    of per-step outputs and the final caches.
    """
    outs = []
    k_c, v_c = k_ctx_rot, v_ctx
    for q1, k1, v1 in zip(qs, ks, vs):
        o, k_c, v_c = query_attn(q1, k1, v1, k_c, v_c, theta, scale)
        outs.append(o)
    return outs, k_c, v_c

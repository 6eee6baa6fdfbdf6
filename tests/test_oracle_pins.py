"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, a library routine
(scipy's matrix exponential, torch's scaled-dot-product attention) or a
brute-force scalar computation written independently here.  Citations are to
the paper-notes page "Efficient Many-Shot In-Context Learning with Dynamic
Block-Sparse Attention" [Notes].
"""
import itertools
import math

import numpy as np
import pytest
import scipy.linalg
import torch
import torch.nn.functional as F

from oracle import dbsa_oracle as orc


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# RoPE: rotation structure and frequencies
# ----------------------------------------------------------------------------

def test_rope_equals_matrix_exponential_of_generator():
    """RoPE(x, p) = expm(p A) x with A the skew generator of the pair rotations.

    Frequencies for d = 8, theta = 1e4 are written out by hand:
    theta^(-2i/8) = 10^(-i) -> 1, 0.1, 0.01, 0.001.
    """
    d = 8
    w = [1.0, 0.1, 0.01, 0.001]
    gen = np.zeros((d, d))
    for i, wi in enumerate(w):
        gen[i, i + 4] = -wi      # d x_i / dp       = -w x_{i+4}
        gen[i + 4, i] = wi       # d x_{i+4} / dp   = +w x_i
    rng = _rng(1)
    x = rng.standard_normal((5, 3, d))
    for p in [0, 1, 7, 1000, 123457]:
        want = np.einsum("ab,thb->tha", scipy.linalg.expm(p * gen), x)
        got = orc.rope(x, np.full(5, p), 1e4)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-9 * max(1, p / 1000))


def test_rope_identity_norm_and_relativity():
    rng = _rng(2)
    d, theta = 128, 5e5
    x = rng.standard_normal((6, 2, d))
    np.testing.assert_array_equal(orc.rope(x, np.zeros(6), theta), x)
    y = orc.rope(x, np.arange(6) * 9973, theta)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # <R(q,a), R(k,b)> = <R(q,a-b), k>
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for a, b in [(5, 3), (90000, 12), (131071, 131000), (40, 41)]:
        lhs = np.sum(orc.rope(q, [a], theta) * orc.rope(k, [b], theta))
        rhs = np.sum(orc.rope(q, [a - b], theta) * k)
        assert abs(lhs - rhs) < 1e-9
    # Group property: re-rotating a rotated vector by a delta = rotating once.
    r1 = orc.rope(orc.rope(x, np.arange(6) * 11, theta), np.arange(6) * 7 + 3, theta)
    r2 = orc.rope(x, np.arange(6) * 18 + 3, theta)
    np.testing.assert_allclose(r1, r2, atol=1e-12)


def test_rope_frequency_table_is_pairwise_rotation():
    """A caller's frequency table: each pair (i, i + d/2) turns by p * w_i.

    Checked against 2x2 rotation matrices applied pair by pair in a loop, and
    the table theta^(-2i/d) reproduces the theta form exactly.
    """
    rng = _rng(21)
    d = 16
    w = np.abs(rng.standard_normal(d // 2)) * 0.3
    x = rng.standard_normal((4, 2, d))
    pos = np.array([0, 3, 250, 77777])
    want = np.empty_like(x)
    for t, p in enumerate(pos):
        for i in range(d // 2):
            c, s = np.cos(p * w[i]), np.sin(p * w[i])
            rot = np.array([[c, -s], [s, c]])
            pair = np.stack([x[t, :, i], x[t, :, i + d // 2]])  # [2, H]
            out = rot @ pair
            want[t, :, i], want[t, :, i + d // 2] = out[0], out[1]
    np.testing.assert_allclose(orc.rope(x, pos, w), want, atol=1e-12)
    plain = 5e5 ** (-(2.0 * np.arange(d // 2)) / d)
    np.testing.assert_array_equal(orc.rope(x, pos, plain), orc.rope(x, pos, 5e5))
    # relativity holds for any table
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    lhs = np.sum(orc.rope(q, [9000], w) * orc.rope(k, [1234], w))
    rhs = np.sum(orc.rope(q, [9000 - 1234], w) * k)
    assert abs(lhs - rhs) < 1e-9


# ----------------------------------------------------------------------------
# Mask: two formulations and the closed form of the row counts
# ----------------------------------------------------------------------------

def _set_based_visible(lens, sink, j):
    """Reading of [Notes, Method > Stage 1, item 2] as sets of blocks.

    Block i may see the anchor (if sink), the blocks i-j..i-1 and itself; then
    the decoder's causal rule keeps keys at or before the query.
    """
    starts = [0]
    for L in lens:
        starts.append(starts[-1] + L)
    n = starts[-1]
    m = np.zeros((n, n), dtype=bool)
    for i in range(len(lens)):
        allowed = set(range(max(i - j, 0), i + 1))
        if sink:
            allowed.add(0)
        for t in range(starts[i], starts[i + 1]):
            for b in allowed:
                for s in range(starts[b], starts[b + 1]):
                    if s <= t:
                        m[t, s] = True
    return m


def test_mask_matches_set_based_reading_bruteforce():
    rng = _rng(3)
    for nb in range(1, 8):
        for trial in range(3):
            lens = list(rng.integers(1, 6, size=nb))
            for j in range(0, nb + 1):
                for sink in (0, 1):
                    np.testing.assert_array_equal(orc.visible(lens, sink, j),
                                                  _set_based_visible(lens, sink, j))


def _closed_form_pairs(lens, sink, j):
    """Visible pairs from interval arithmetic.

    Row t of block i sees [off[lo], t] (lo = max(i-j, 0)) plus the anchor's L_0
    keys when the anchor is not already inside that window.
    """
    off = [0]
    for L in lens:
        off.append(off[-1] + L)
    total = 0
    for i, L in enumerate(lens):
        lo = max(i - j, 0)
        extra = lens[0] if (sink and lo > 0) else 0
        # sum over t in block i of (t - off[lo] + 1 + extra)
        total += L * (off[i] - off[lo] + extra) + L * (L + 1) // 2
    return total


def test_mask_row_counts_closed_form():
    rng = _rng(4)
    for nb in (1, 2, 5, 9):
        lens = list(rng.integers(1, 40, size=nb))
        for j in (0, 1, 2, 8):
            for sink in (0, 1):
                assert orc.visible(lens, sink, j).sum() == _closed_form_pairs(lens, sink, j)


def test_mask_pair_count_llama2_shape():
    """30 blocks x 1024 tokens, sink + previous 2: 103,824,384 pairs per head."""
    lens = [1024] * 30
    assert _closed_form_pairs(lens, 1, 2) == 103_824_384
    n = 30 * 1024
    count = 0
    for a in range(0, n, 4096):
        count += int(orc.visible(lens, 1, 2, rows=np.arange(a, min(a + 4096, n))).sum())
    assert count == 103_824_384


# ----------------------------------------------------------------------------
# Prefill: special cases that reduce to library attention / closed forms
# ----------------------------------------------------------------------------

def _qkv(rng, n, hq, hkv, d):
    return (rng.standard_normal((n, hq, d)), rng.standard_normal((n, hkv, d)),
            rng.standard_normal((n, hkv, d)))


def _sdpa_causal(q_rot, k_rot, v, scale):
    """torch scaled-dot-product attention (float64, CPU), causal, GQA by repeat."""
    hq, hkv = q_rot.shape[1], k_rot.shape[1]
    g = hq // hkv
    qt = torch.from_numpy(q_rot).permute(1, 0, 2)
    kt = torch.from_numpy(k_rot).repeat_interleave(g, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)
    o = F.scaled_dot_product_attention(qt.contiguous(), kt.contiguous(), vt.contiguous(),
                                       is_causal=True, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_full_pattern_is_causal_sdpa():
    """j >= n_blocks - 1 is plain causal attention (ablation 'full attention')."""
    rng = _rng(5)
    lens = [7, 3, 12, 5, 9]
    n = sum(lens)
    q, k, v = _qkv(rng, n, 4, 2, 16)
    theta = 1e4
    scale = 1 / 4.0
    want = _sdpa_causal(orc.rope(q, np.arange(n), theta), orc.rope(k, np.arange(n), theta), v, scale)
    for j in (4, 5, 50):
        got = orc.prefill(q, k, v, lens, 1, j, theta)
        np.testing.assert_allclose(got, want, atol=1e-12)
        got0 = orc.prefill(q, k, v, lens, 0, j, theta)
        np.testing.assert_allclose(got0, want, atol=1e-12)


def test_self_only_is_per_block_causal_at_local_positions():
    """Self-only attention = each block encoded alone at positions 0..L-1 (RoPE is relative)."""
    rng = _rng(6)
    lens = [6, 11, 4, 9]
    n = sum(lens)
    q, k, v = _qkv(rng, n, 2, 1, 8)
    theta = 1e4
    got = orc.prefill(q, k, v, lens, 0, 0, theta)
    a = 0
    for L in lens:
        sl = slice(a, a + L)
        loc = np.arange(L)
        want = _sdpa_causal(orc.rope(q[sl], loc, theta), orc.rope(k[sl], loc, theta), v[sl],
                            1 / math.sqrt(8))
        np.testing.assert_allclose(got[sl], want, atol=1e-12)
        a += L


def test_zero_queries_give_visible_block_fractions():
    """Q = 0 makes all visible scores equal: O[t] is the mean of the visible V rows.

    With V[s] = one-hot(blk(s)), O[t][b] = (#visible keys of block b) / |vis(t)|,
    counted here by interval arithmetic.
    """
    lens = [5, 3, 8, 2, 6, 4]
    nb = len(lens)
    off = np.concatenate([[0], np.cumsum(lens)])
    n = off[-1]
    for sink, j in [(1, 2), (0, 0), (1, 0), (0, 1), (1, 5)]:
        q = np.zeros((n, 1, nb))
        k = _rng(7).standard_normal((n, 1, nb))
        v = np.zeros((n, 1, nb))
        for b in range(nb):
            v[off[b]:off[b + 1], 0, b] = 1.0
        got = orc.prefill(q, k, v, lens, sink, j, 1e4)[:, 0, :]
        for t in range(n):
            i = int(np.searchsorted(off, t, side="right") - 1)
            lo = max(i - j, 0)
            cnt = np.zeros(nb)
            for b in range(lo, i):
                cnt[b] = lens[b]
            cnt[i] = t - off[i] + 1
            if sink and lo > 0:
                cnt[0] = lens[0]
            np.testing.assert_allclose(got[t], cnt / cnt.sum(), atol=1e-14)


def test_softmax_rows_sum_to_one():
    rng = _rng(8)
    lens = [9, 4, 13]
    n = sum(lens)
    q, k, _ = _qkv(rng, n, 4, 2, 8)
    got = orc.prefill(q * 3, k, np.ones((n, 2, 8)), lens, 1, 1, 5e5)
    np.testing.assert_allclose(got, 1.0, atol=1e-14)


def _bruteforce_prefill(q, k, v, lens, sink, j, theta):
    """Scalar-loop attention: explicit angles, explicit mask, explicit softmax."""
    n, hq, d = q.shape
    hkv = k.shape[1]
    half = d // 2
    blk = []
    for b, L in enumerate(lens):
        blk += [b] * L

    def rot(x, p):
        out = [0.0] * d
        for i in range(half):
            ang = p * (theta ** (-(2.0 * i) / d))
            c, s = math.cos(ang), math.sin(ang)
            out[i] = x[i] * c - x[i + half] * s
            out[i + half] = x[i + half] * c + x[i] * s
        return out

    o = np.zeros_like(q)
    for t in range(n):
        for h in range(hq):
            g = h // (hq // hkv)
            qr = rot(list(q[t, h]), t)
            sc = []
            for s in range(t + 1):
                if blk[s] >= blk[t] - j or (sink and blk[s] == 0):
                    kr = rot(list(k[s, g]), s)
                    sc.append((s, sum(a * b for a, b in zip(qr, kr)) / math.sqrt(d)))
            m = max(x for _, x in sc)
            wts = [(s, math.exp(x - m)) for s, x in sc]
            tot = sum(w for _, w in wts)
            for s, w in wts:
                o[t, h] += w / tot * v[s, g]
    return o


def test_prefill_bruteforce_small():
    rng = _rng(9)
    lens = [3, 4, 2, 5, 3]
    n = sum(lens)
    q, k, v = _qkv(rng, n, 4, 2, 6)
    for sink, j in [(1, 2), (0, 1), (1, 0)]:
        np.testing.assert_allclose(orc.prefill(q, k, v, lens, sink, j, 1e4),
                                   _bruteforce_prefill(q, k, v, lens, sink, j, 1e4), atol=1e-12)


def test_append_equals_prefill_of_extended_pool():
    """[Notes, Method > Stage 1, item 4]: encoding one more block = its rows of the full encode."""
    rng = _rng(10)
    lens = [6, 5, 7, 4]
    new_len = 6
    n = sum(lens) + new_len
    q, k, v = _qkv(rng, n, 4, 2, 8)
    n_old = sum(lens)
    for sink, j in [(1, 2), (0, 0), (1, 0), (1, 8)]:
        o_new, k2, v2, lens2 = orc.append_block(q[n_old:], k[n_old:], v[n_old:], k[:n_old],
                                                v[:n_old], lens, sink, j, 5e5)
        full = orc.prefill(q, k, v, lens + [new_len], sink, j, 5e5)
        np.testing.assert_array_equal(k2, k)
        np.testing.assert_array_equal(v2, v)
        np.testing.assert_allclose(o_new, full[n_old:], atol=1e-13)


# ----------------------------------------------------------------------------
# Stage 2: gather + re-RoPE + query attention
# ----------------------------------------------------------------------------

def test_gather_places_blocks_in_given_order():
    rng = _rng(11)
    lens = [3, 5, 2, 4]
    n = sum(lens)
    k = rng.standard_normal((n, 2, 8))
    v = rng.standard_normal((n, 2, 8))
    ids = [0, 3, 1]
    kg, vg = orc.gather_rope(k, v, lens, ids, 1e4)
    raw_k = np.concatenate([k[0:3], k[10:14], k[3:8]])
    raw_v = np.concatenate([v[0:3], v[10:14], v[3:8]])
    np.testing.assert_array_equal(vg, raw_v)
    # Undo the rotation with the inverse (negative) positions: recovers the cache.
    np.testing.assert_allclose(orc.rope(kg, -np.arange(kg.shape[0]), 1e4), raw_k, atol=1e-13)


def test_gather_spans_places_tokens_in_given_order():
    """Example-level spans: token t of the result is the pool token at the
    t-th place of the spans' concatenation, K turned back by -t recovers it,
    and spans that cover whole blocks give the block gather exactly."""
    rng = _rng(12)
    lens = [3, 5, 2, 4]
    n = sum(lens)
    k = rng.standard_normal((n, 2, 8))
    v = rng.standard_normal((n, 2, 8))
    src, ln = [0, 11, 4, 1, 9], [2, 3, 0, 3, 1]
    kg, vg = orc.gather_rope_spans(k, v, src, ln, 1e4)
    order = []
    for s_, l_ in zip(src, ln):
        t = s_
        while t < s_ + l_:
            order.append(t)
            t += 1
    assert order == [0, 1, 11, 12, 13, 1, 2, 3, 9]
    assert kg.shape[0] == len(order)
    for t, p in enumerate(order):
        np.testing.assert_array_equal(vg[t], v[p])
        np.testing.assert_allclose(orc.rope(kg[t:t + 1], [-t], 1e4)[0], k[p], atol=1e-13)
    kb, vb = orc.gather_rope(k, v, lens, [0, 3, 1], 1e4)
    ks, vs = orc.gather_rope_spans(k, v, [0, 10, 3], [3, 4, 5], 1e4)
    np.testing.assert_array_equal(ks, kb)
    np.testing.assert_array_equal(vs, vb)
    # splitting a span in two changes nothing
    k2, v2 = orc.gather_rope_spans(k, v, [0, 10, 12, 3], [3, 2, 2, 5], 1e4)
    np.testing.assert_array_equal(k2, kb)
    np.testing.assert_array_equal(v2, vb)


def test_anchor_only_stage2_is_causal_sdpa_over_anchor_and_query():
    rng = _rng(12)
    lens = [6, 4, 5]
    n = sum(lens)
    _, k, v = _qkv(rng, n, 4, 2, 8)
    nq = 5
    q_new, k_new, v_new = _qkv(rng, nq, 4, 2, 8)
    theta = 1e4
    kg, vg = orc.gather_rope(k, v, lens, [0], theta)
    got, _, _ = orc.query_attn(q_new, k_new, v_new, kg, vg, theta)
    # The same thing as a plain causal decoder pass over [anchor; query].
    seq_q = np.concatenate([np.zeros((6, 4, 8)), q_new])
    seq_k = np.concatenate([k[:6], k_new])
    seq_v = np.concatenate([v[:6], v_new])
    pos = np.arange(6 + nq)
    want = _sdpa_causal(orc.rope(seq_q, pos, theta), orc.rope(seq_k, pos, theta), seq_v,
                        1 / math.sqrt(8))[6:]
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_all_blocks_in_order_equals_fixed_icl_attention():
    """Pre-RoPE caching + re-rotation at the original positions = the directly rotated pool."""
    rng = _rng(13)
    lens = [4, 6, 3, 5]
    n = sum(lens)
    _, k, v = _qkv(rng, n, 4, 1, 8)
    q_new, k_new, v_new = _qkv(rng, 3, 4, 1, 8)
    theta = 5e5
    kg, vg = orc.gather_rope(k, v, lens, [0, 1, 2, 3], theta)
    got, _, _ = orc.query_attn(q_new, k_new, v_new, kg, vg, theta)
    seq_q = np.concatenate([np.zeros((n, 4, 8)), q_new])
    seq_k = np.concatenate([k, k_new])
    seq_v = np.concatenate([v, v_new])
    pos = np.arange(n + 3)
    want = _sdpa_causal(orc.rope(seq_q, pos, theta), orc.rope(seq_k, pos, theta), seq_v,
                        1 / math.sqrt(8))[n:]
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_stage2_shift_invariance():
    """Adding a constant to every Stage-2 position leaves the output unchanged."""
    rng = _rng(14)
    lens = [5, 7, 4, 6]
    n = sum(lens)
    _, k, v = _qkv(rng, n, 2, 2, 16)
    q_new, k_new, v_new = _qkv(rng, 4, 2, 2, 16)
    theta = 1e4
    ids = [0, 2, 3]
    kg, vg = orc.gather_rope(k, v, lens, ids, theta)
    base, _, _ = orc.query_attn(q_new, k_new, v_new, kg, vg, theta)
    c = 777
    tp = kg.shape[0]
    kg_shift = orc.rope(kg, np.full(tp, c), theta)  # every cached key moved by +c
    pos_new = tp + c + np.arange(4)
    k_all = np.concatenate([kg_shift, orc.rope(k_new, pos_new, theta)])
    v_all = np.concatenate([vg, v_new])
    mask = np.arange(tp + 4)[None, :] <= (tp + np.arange(4))[:, None]
    shifted = orc.masked_attention(orc.rope(q_new, pos_new, theta), k_all, v_all, mask,
                                   1 / 4.0)
    np.testing.assert_allclose(shifted, base, atol=1e-12)


def test_decode_steps_equal_one_causal_pass():
    """Feeding tokens one at a time (decode) = feeding them together with a causal mask."""
    rng = _rng(15)
    lens = [5, 4, 6]
    n = sum(lens)
    _, k, v = _qkv(rng, n, 4, 2, 8)
    kg, vg = orc.gather_rope(k, v, lens, [0, 2], 1e4)
    q_new, k_new, v_new = _qkv(rng, 6, 4, 2, 8)
    together, kc, vc = orc.query_attn(q_new, k_new, v_new, kg, vg, 1e4)
    outs, kc2, vc2 = orc.decode([q_new[i:i + 1] for i in range(6)],
                                [k_new[i:i + 1] for i in range(6)],
                                [v_new[i:i + 1] for i in range(6)], kg, vg, 1e4)
    np.testing.assert_allclose(np.concatenate(outs), together, atol=1e-13)
    np.testing.assert_allclose(kc2, kc, atol=1e-13)
    np.testing.assert_array_equal(vc2, vc)


def test_query_attention_bruteforce_small():
    rng = _rng(16)
    lens = [3, 2, 4]
    n = sum(lens)
    _, k, v = _qkv(rng, n, 2, 1, 4)
    q_new, k_new, v_new = _qkv(rng, 3, 2, 1, 4)
    theta = 1e4
    ids = [0, 2]
    got, _, _ = orc.query_attn(q_new, k_new, v_new, *orc.gather_rope(k, v, lens, ids, theta),
                               theta)
    raw_k = np.concatenate([k[0:3], k[5:9], k_new])
    raw_v = np.concatenate([v[0:3], v[5:9], v_new])
    tp = 7

    def rot(x, p):
        out = list(x)
        for i in range(2):
            ang = p * theta ** (-i / 2)
            out[i] = x[i] * math.cos(ang) - x[i + 2] * math.sin(ang)
            out[i + 2] = x[i + 2] * math.cos(ang) + x[i] * math.sin(ang)
        return out

    for r in range(3):
        for h in range(2):
            qr = rot(q_new[r, h], tp + r)
            sc = [sum(a * b for a, b in zip(qr, rot(raw_k[s, 0], s))) / 2.0
                  for s in range(tp + r + 1)]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            want = sum(wi * raw_v[s, 0] for s, wi in enumerate(w)) / sum(w)
            np.testing.assert_allclose(got[r, h], want, atol=1e-12)

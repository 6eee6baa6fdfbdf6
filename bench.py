#!/usr/bin/env python3
"""Benchmark of the DBSA hot path on one MI355X.

One step = one pass of the whole hot path over the two largest benchmark
workloads, inputs resident in HBM:
  * Stage 1 on the 131,072-token stress pool (128 blocks of 512-2048 tokens,
    GQA 32/8, head_dim 128, bf16, sink + previous 2 blocks):
      dbsa_prefill        block-sparse streaming prefill (mask -> key-tile
                          walk, RoPE, flash attention; K/V stay unrotated),
      dbsa_append_block   one new 1024-token block encoded onto that pool;
  * Stage 2 on the Llama-3.1-8B-shaped 32-layer pool (90 blocks of 50 demos,
    89,568 tokens, 0.125 MiB of K/V per token): for each of the 32 layers, a
    batch of 64 queries, each with the anchor + its own 27 blocks and 48 query
    tokens -- gather, re-RoPE and query attention in the shared-block schedule
    (dbsa_query_attn_batched: each selected block's K/V loaded once for all
    the queries that chose it).
Prints one JSON line.  `value` = the stress prefill's FLOP on executed
(unmasked) key tiles / the prefill's own time (HIP events on the stream it
runs on).  `roofline` is the prefill call (MFMA-bound; exact visible-pair
FLOP), `roofline_stage2` the Stage-2 call of one layer (bound by HBM or MFMA
according to the schedule; algorithmic bytes / FLOP of that schedule).  The
Llama-2-7B layer (30 x 1024 tokens) is reported as a sub-object.  The CPU
baseline is the fp64 oracle on bounded samples of the same two workloads, on
this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KEY_TILE, WG_ROWS = 64, 256
CSRC = os.path.join(ROOT, "block_sparse_attention_sink_amd", "csrc")
PREFILL_SOURCES = [os.path.join(CSRC, f) for f in ("k_stage1.hip", "dbsa_device.hpp",
                                                   "dbsa_internal.hpp")]
STAGE2_SOURCES = [os.path.join(CSRC, f) for f in ("k_shared.hip", "k_stage2.hip", "k_tables.hip",
                                                  "dbsa_device.hpp", "dbsa_internal.hpp")]
PREFILL_PROFILE = os.path.join(ROOT, "profiles", "k_prefill_bf16_stress_131072_sink_prev2.md")
STAGE2_PROFILE = os.path.join(ROOT, "profiles", "stage2_llama31_pool_batch64x48.md")


# ---------------------------------------------------------------------------
# Algorithmic work (closed forms of the block mask; no GPU code)
# ---------------------------------------------------------------------------
def visible_pairs(lens, sink, j):
    """Sum over rows of the visible-key count (interval form of the block mask)."""
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total = 0
    for i, L in enumerate(lens):
        lo = max(i - j, 0)
        extra = lens[0] if (sink and lo > 0) else 0
        total += int(L) * int(off[i] - off[lo] + extra) + int(L) * (int(L) + 1) // 2
    return total


PREFILL_MAX_PACKED_HEADS = 4  # query heads of one KV head sharing a prefill workgroup


def prefill_row_tile(hq, hkv):
    """Tokens per prefill workgroup: 256 MFMA rows = tokens x the query heads
    of one KV head packed together (at most PREFILL_MAX_PACKED_HEADS)."""
    g = hq // hkv
    gw = 1
    while gw * 2 <= min(g, PREFILL_MAX_PACKED_HEADS) and g % (gw * 2) == 0:
        gw *= 2
    return WG_ROWS // gw, gw


def executed_tiles(lens, sink, j, row_tile=WG_ROWS):
    """64-key tiles the prefill walks per query head, summed over its
    row_tile-token query tiles."""
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = int(off[-1])
    nb = len(lens)
    blk_of = lambda t: int(np.searchsorted(off, t, side="right") - 1)
    lo_of = lambda t: int(off[max(min(blk_of(t), nb - 1) - j, 0)])
    tiles = 0
    for r0 in range(0, n, row_tile):
        r1 = min(r0 + row_tile, n)
        w0 = lo_of(r0) // KEY_TILE
        w1 = -(-r1 // KEY_TILE)
        ns = min(-(-int(off[1]) // KEY_TILE), w0) if (sink and lo_of(r1 - 1) > 0) else 0
        tiles += ns + (w1 - w0)
    return tiles


def prefill_work(lens, sink, j, hq, hkv, d):
    pairs = visible_pairs(lens, sink, j)
    rt, _ = prefill_row_tile(hq, hkv)
    tiles = executed_tiles(lens, sink, j, rt)
    return {"exact_pairs_per_head": pairs, "exact_flop": 4.0 * d * hq * pairs,
            "executed_tiles_per_head": tiles, "tile_tokens_x_keys": [rt, KEY_TILE],
            "executed_tile_flop": 4.0 * d * hq * tiles * rt * KEY_TILE}


def stage2_work(lens, ids, n_new, hq, hkv, d, esz=2):
    """Per-query schedule: every batch row reads the unrotated K/V of its own
    gathered tokens once, plus its Q, new K/V and O.  FLOP: each query token
    sees the whole gathered context and the new tokens up to itself."""
    tp = np.array([int(lens[r].sum()) for r in ids], dtype=np.int64)
    batch = len(ids)
    kv = int(tp.sum()) * hkv * d * esz * 2
    io = batch * n_new * (2 * hq + 2 * hkv) * d * esz
    pairs = int((tp * n_new).sum()) + batch * n_new * (n_new + 1) // 2
    uniq = np.unique(np.concatenate(list(ids)))
    union = int(lens[uniq].sum()) * hkv * d * esz * 2
    return {"bytes_per_query_schedule": kv + io, "kv_bytes_per_query_schedule": kv,
            "bytes_pool_union": union + io, "flop": 4.0 * d * hq * pairs,
            "context_tokens_mean": float(tp.mean())}


# ---------------------------------------------------------------------------
# Profile summaries (HBM traffic per launch, if taken on the current sources)
# ---------------------------------------------------------------------------
def _code_only(text):
    """C++ source with comments and blank lines removed, lines right-stripped:
    an edit to a comment leaves the kernel, and so its counters, unchanged.
    (The kernel sources hold no string literal that contains a comment
    marker.)"""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def source_digest(paths):
    """sha256 over the code of the kernel's source files (comments left out),
    concatenated in order."""
    h = hashlib.sha256()
    for p in paths:
        h.update(_code_only(open(p).read()).encode())
        h.update(b"\n")
    return h.hexdigest()


def profile_traffic(path, sources):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not t:
        return None
    return float(t.group(1)) if m.group(1) == source_digest(sources) else None


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


# ---------------------------------------------------------------------------
# Workload set-up (seeded synthetic tensors, resident in HBM)
# ---------------------------------------------------------------------------
class PrefillCase:
    """Stage 1 of workload k: Q/K/V of the pool, a cache with room for the
    appended block, the block's Q/K/V."""

    def __init__(self, k, dev, sink=None, j=None, with_append=True):
        import torch
        from block_sparse_attention_sink_amd.inputs import randn, workload
        w = self.w = workload(k)
        self.sink = w.sink if sink is None else sink
        self.j = w.j if j is None else j
        n, hq, hkv, d = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim
        self.q = randn((n, hq, d), 1001 + k, w.dtype, dev)
        la = w.append_len if with_append else 0
        self.k_cache = torch.empty((n + la, hkv, d), dtype=self.q.dtype, device=dev)
        self.v_cache = torch.empty_like(self.k_cache)
        self.k_cache[:n].copy_(randn((n, hkv, d), 1101 + k, w.dtype, dev))
        self.v_cache[:n].copy_(randn((n, hkv, d), 1201 + k, w.dtype, dev))
        self.k, self.v = self.k_cache[:n], self.v_cache[:n]
        self.o = torch.empty_like(self.q)
        self.work = prefill_work(w.block_lens, self.sink, self.j, hq, hkv, d)
        self.la = la
        if la:
            self.qa = randn((la, hq, d), 1301 + k, w.dtype, dev)
            self.ka = randn((la, hkv, d), 1302 + k, w.dtype, dev)
            self.va = randn((la, hkv, d), 1303 + k, w.dtype, dev)
            self.oa = torch.empty_like(self.qa)
            lens_a = np.append(w.block_lens, la).astype(np.int32)
            self.append_pairs = visible_pairs(lens_a, self.sink, self.j) - \
                visible_pairs(w.block_lens, self.sink, self.j)

    def prefill(self):
        from block_sparse_attention_sink_amd import dbsa
        w = self.w
        dbsa.dbsa_prefill(self.q, self.k, self.v, w.block_lens, self.sink, self.j, w.theta,
                          out=self.o)

    def append(self):
        from block_sparse_attention_sink_amd import dbsa
        w = self.w
        dbsa.dbsa_append_block(self.qa, self.ka, self.va, self.k_cache, self.v_cache,
                               w.block_lens, self.sink, self.j, w.theta, out=self.oa)


class Stage2Case:
    """Stage 2 of workload k: the pool (all its layers), the batch's query
    tokens and their tail buffers."""

    def __init__(self, k, dev, layers=None):
        import torch
        from block_sparse_attention_sink_amd.inputs import randn, workload
        w = self.w = workload(k)
        n, hq, hkv, d = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim
        self.layers = w.layers if layers is None else layers
        self.pool_k = torch.empty((self.layers, n, hkv, d), dtype=torch.bfloat16, device=dev)
        self.pool_v = torch.empty_like(self.pool_k)
        for l in range(self.layers):
            self.pool_k[l].copy_(randn((n, hkv, d), 2000 + 2 * l, w.dtype, dev))
            self.pool_v[l].copy_(randn((n, hkv, d), 2001 + 2 * l, w.dtype, dev))
        b, nn = w.batch, w.n_new
        self.qn = randn((b, nn, hq, d), 2101, w.dtype, dev)
        self.kn = randn((b, nn, hkv, d), 2102, w.dtype, dev)
        self.vn = randn((b, nn, hkv, d), 2103, w.dtype, dev)
        self.on = torch.empty_like(self.qn)
        self.kt = torch.empty((b, nn, hkv, d), dtype=self.qn.dtype, device=dev)
        self.vt = torch.empty_like(self.kt)
        self.work = stage2_work(w.block_lens, w.ids, nn, hq, hkv, d)

    def layer(self, l, schedule="per_query"):
        from block_sparse_attention_sink_amd import dbsa
        w = self.w
        fn = dbsa.dbsa_query_attn_batched if schedule == "shared" else \
            dbsa.dbsa_query_attn_gathered
        fn(self.qn, self.kn, self.vn, self.pool_k[l], self.pool_v[l], w.block_lens, w.ids,
           self.kt, self.vt, [0] * w.batch, w.theta, out=self.on)


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def run_main(args, dev):
    import torch

    pre = PrefillCase(5, dev)
    st2 = Stage2Case(4, dev)
    L = st2.layers
    marks = []

    def step(record):
        e = _events(4) if record else None
        if record:
            e[0].record()
        pre.prefill()
        if record:
            e[1].record()
        pre.append()
        if record:
            e[2].record()
        for l in range(L):
            st2.layer(l, "shared")
        if record:
            e[3].record()
            marks.append(e)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0, t1 = _events(2)
    t0.record()
    for _ in range(args.steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    ms_prefill = float(np.mean([m[0].elapsed_time(m[1]) for m in marks]))
    ms_append = float(np.mean([m[1].elapsed_time(m[2]) for m in marks]))
    ms_stage2 = float(np.mean([m[2].elapsed_time(m[3]) for m in marks]))
    ms_layer = ms_stage2 / L

    pw, sw = pre.work, st2.work
    value = pw["executed_tile_flop"] / (ms_prefill * 1e-3) / 1e12
    achieved = pw["exact_flop"] / (ms_prefill * 1e-3) / 1e12
    s2_tflops = sw["flop"] / (ms_layer * 1e-3) / 1e12
    s2_unique_gbs = sw["bytes_pool_union"] / (ms_layer * 1e-3) / 1e9
    s2_perq_gbs = sw["bytes_per_query_schedule"] / (ms_layer * 1e-3) / 1e9
    w5, w4 = pre.w, st2.w
    # The per-query schedule on the same layer, for comparison.
    ms_perq = time_calls(lambda: [st2.layer(l, "per_query") for l in range(4)], 3) / 4

    llama2 = run_llama2(dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(pre, st2, args.cpu_seconds)
    out = {
        "metric": "DBSA prefill TFLOP/s (unmasked tiles) + gather/query-attn GB/s, % roofline",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) Q/K/V (seeded), no model weights",
        "config": {
            "workload": f"{w5.name} prefill (sink + previous {pre.j}) + append of "
                        f"{pre.la} tokens; {w4.name} Stage 2 (gather + re-RoPE + query "
                        f"attention, shared-block schedule, {L} layers)",
            "prefill": {"n_tokens": w5.n_tokens, "n_blocks": w5.n_blocks, "q_heads": w5.n_q_heads,
                        "kv_heads": w5.n_kv_heads, "head_dim": w5.head_dim, "sink": pre.sink,
                        "j": pre.j, "rope_theta": w5.theta},
            "stage2": {"layers": L, "pool_tokens": w4.n_tokens, "batch": w4.batch,
                       "blocks_per_query": int(w4.ids.shape[1]), "query_tokens": w4.n_new,
                       "q_heads": w4.n_q_heads, "kv_heads": w4.n_kv_heads,
                       "head_dim": w4.head_dim, "rope_theta": w4.theta,
                       "context_tokens_mean": sw["context_tokens_mean"]},
            "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": profile_traffic(PREFILL_PROFILE, PREFILL_SOURCES),
                     "kernel": "dbsa_prefill call (k_pack_bf16 + k_prefill_bf16), stress pool",
                     "ms_per_launch": ms_prefill,
                     "algorithmic_flop_per_launch": pw["exact_flop"]},
        "roofline_stage2": {"bound": "mfma", "achieved": s2_tflops, "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": s2_tflops / PEAK_BF16_TFLOPS,
                            "traffic": profile_traffic(STAGE2_PROFILE, STAGE2_SOURCES),
                            "kernel": "dbsa_query_attn_batched call (k_pack_shared_bf16 + "
                                      "k_shared_bf16 + k_query_bf16 + k_merge), one layer of "
                                      "the pool, 64 queries x 48 tokens",
                            "schedule": "shared blocks: each selected block's K/V read once for "
                                        "all queries that chose it; bound by the attention FLOP",
                            "ms_per_launch": ms_layer,
                            "algorithmic_flop_per_launch": sw["flop"],
                            "unique_bytes_per_launch": sw["bytes_pool_union"],
                            "unique_GB/s": s2_unique_gbs},
        "prefill": {"exact_TFLOP": pw["exact_flop"] / 1e12,
                    "executed_tile_TFLOP": pw["executed_tile_flop"] / 1e12,
                    "tile_tokens_x_keys": pw["tile_tokens_x_keys"],
                    "exact_TFLOP/s": achieved, "executed_tile_TFLOP/s": value},
        "append": {"tokens": pre.la, "ms": ms_append,
                   "TFLOP/s": 4.0 * w5.head_dim * w5.n_q_heads * pre.append_pairs
                   / (ms_append * 1e-3) / 1e12},
        "stage2": {"ms_all_layers": ms_stage2, "attention_TFLOP/s": s2_tflops,
                   "per_query_schedule_bytes_GB/s": s2_perq_gbs,
                   "per_query_schedule": {"ms_per_layer": ms_perq,
                                          "GB/s": sw["bytes_per_query_schedule"]
                                          / (ms_perq * 1e-3) / 1e9,
                                          "note": "dbsa_query_attn_gathered on the same layer: "
                                                  "each batch row reads its own blocks"}},
        "step_breakdown_ms": {"prefill": ms_prefill, "append": ms_append,
                              "stage2_all_layers": ms_stage2},
        "llama2_layer": llama2,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def time_calls(fn, reps):
    """Median of `reps` timed calls of fn (HIP events on the current stream)."""
    import torch
    ts = []
    for _ in range(reps + 1):
        a, b = _events(2)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts[1:]))


def run_llama2(dev, reps=10):
    """The Llama-2-7B layer (30 x 1024 tokens, MHA 32, j = 2): prefill, and the
    fused Stage 2 of anchor + 9 blocks with 64 query tokens (caches flushed
    before each Stage-2 repetition)."""
    import torch
    from block_sparse_attention_sink_amd import dbsa
    from block_sparse_attention_sink_amd.inputs import randn
    pre = PrefillCase(2, dev, with_append=False)
    w = pre.w
    hkv, d = w.n_kv_heads, w.head_dim
    nn = w.n_new
    qn = randn((1, nn, w.n_q_heads, d), 3001, "bf16", dev)
    kn = randn((1, nn, hkv, d), 3002, "bf16", dev)
    vn = randn((1, nn, hkv, d), 3003, "bf16", dev)
    on = torch.empty_like(qn)
    kt = torch.empty((1, nn, hkv, d), dtype=torch.bfloat16, device=dev)
    vt = torch.empty_like(kt)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    acc = torch.zeros((), dtype=torch.float32, device=dev)

    def timed(fn, flush_first):
        ts = []
        for _ in range(reps + 2):
            if flush_first:
                acc.add_(flush.sum())
            a, b = _events(2)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts[2:]))
    ms_p = timed(pre.prefill, False)
    ms_s = timed(lambda: dbsa.dbsa_query_attn_gathered(qn, kn, vn, pre.k, pre.v, w.block_lens,
                                                       w.ids, kt, vt, [0], w.theta, out=on), True)
    sw = stage2_work(w.block_lens, w.ids, nn, w.n_q_heads, hkv, d)
    return {"workload": w.name,
            "prefill_ms": ms_p,
            "prefill_exact_TFLOP/s": pre.work["exact_flop"] / (ms_p * 1e-3) / 1e12,
            "prefill_frac_bf16": pre.work["exact_flop"] / (ms_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "stage2_fused_us": ms_s * 1e3,
            "stage2_GB/s": sw["bytes_per_query_schedule"] / (ms_s * 1e-3) / 1e9,
            "stage2_frac_hbm": sw["bytes_per_query_schedule"] / (ms_s * 1e-3) / 1e9
            / PEAK_HBM_GBS,
            "note": "median of 10; Stage 2 with a 1 GiB cache flush before each repetition"}


def cpu_baseline(pre, st2, seconds):
    """The fp64 oracle on bounded samples of the two workloads: random rows of
    the stress prefill (about `seconds`), and whole (query, layer) units of
    the Stage-2 batch (about seconds / 2)."""
    from oracle import dbsa_oracle as orc
    h = lambda t: t.float().cpu().numpy().astype(np.float64)
    w = pre.w
    lens, n = w.block_lens, w.n_tokens
    qh, kh, vh = h(pre.q), h(pre.k), h(pre.v)
    rng = np.random.default_rng(7)
    order = rng.permutation(n)
    done, secs = 0, 0.0
    while secs < seconds and done < min(n, 8192):
        batch = np.sort(order[done:done + 64])
        t = time.perf_counter()
        orc.prefill(qh, kh, vh, lens, pre.sink, pre.j, w.theta, rows=batch)
        secs += time.perf_counter() - t
        done += batch.size
    rows = order[:done]
    off = np.concatenate([[0], np.cumsum(lens)])
    blk = np.searchsorted(off, rows, side="right") - 1
    lo = off[np.maximum(blk - pre.j, 0)]
    vis = (rows - lo + 1) + np.where((lo > 0) & bool(pre.sink), lens[0], 0)
    value = 4.0 * w.head_dim * w.n_q_heads * float(vis.sum()) / secs / 1e12

    w4 = st2.w
    units, s2_secs, s2_bytes = 0, 0.0, 0
    qn, kn, vn = h(st2.qn), h(st2.kn), h(st2.vn)
    while s2_secs < seconds / 2 and units < 8:
        b, l = int(rng.integers(w4.batch)), int(rng.integers(st2.layers))
        t = time.perf_counter()
        kg, vg = orc.gather_rope(h(st2.pool_k[l]), h(st2.pool_v[l]), w4.block_lens, w4.ids[b],
                                 w4.theta)
        orc.query_attn(qn[b], kn[b], vn[b], kg, vg, w4.theta)
        s2_secs += time.perf_counter() - t
        units += 1
        s2_bytes += kg.shape[0] * w4.n_kv_heads * w4.head_dim * 2 * 2 + \
            w4.n_new * (2 * w4.n_q_heads + 2 * w4.n_kv_heads) * w4.head_dim * 2
    return {"value": value, "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"stress prefill oracle (fp64 masked-dense NumPy) on {done} random rows x "
                      f"all {w.n_q_heads} heads, {secs:.1f} s; value counts the exact visible "
                      "pairs of the sampled rows",
            "stage2": {"GB/s": s2_bytes / s2_secs / 1e9, "units": units,
                       "seconds": s2_secs,
                       "sample": f"{units} (query, layer) units of the pool batch: gather + "
                                 "re-RoPE + query attention in fp64, bytes as the per-query "
                                 "schedule counts them"}}


# ---------------------------------------------------------------------------
# Single-operation runs (for rocprofv3) and the per-workload table
# ---------------------------------------------------------------------------
def profile_op(dev, op, k, steps, warmup):
    """Run one hot-path operation of workload k `steps` times: the prefill of
    its pool, its append, the fused Stage 2 of its batch (one layer), or a
    1 GiB device copy (counter calibration)."""
    import torch
    if op in ("prefill", "append"):
        case = PrefillCase(k, dev, with_append=(op == "append"))
        fn = case.prefill if op == "prefill" else case.append
    elif op in ("fused", "batched"):
        case = Stage2Case(k, dev, layers=1)
        if case.w.n_new == 0:
            raise SystemExit(f"workload {k} has no Stage-2 queries")
        sched = "shared" if op == "batched" else "per_query"
        fn = lambda: case.layer(0, sched)
    else:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a0, a1 = _events(2)
    a0.record()
    for _ in range(steps):
        fn()
    a1.record()
    torch.cuda.synchronize()
    print(json.dumps({"profile_op": op, "workload": k, "steps": steps,
                      "ms_per_call": a0.elapsed_time(a1) / steps}), flush=True)


def run_all_workloads(dev):
    """Median time of every hot-path operation on the five workloads (caches
    flushed before each Stage-2 repetition), with its algorithmic rate."""
    import torch
    from block_sparse_attention_sink_amd import dbsa
    from block_sparse_attention_sink_amd.inputs import PATTERNS, randn, workload

    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink_acc = torch.zeros((), dtype=torch.float32, device=dev)

    def timed(fn, reps, flush_first=False):
        ts = []
        for r in range(reps + 2):
            if flush_first:
                sink_acc.add_(flush.sum())
            a, b = _events(2)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts[2:]))

    def emit(wl, op, ms, work, unit, **extra):
        rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        peak = PEAK_BF16_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBS
        print(json.dumps({"workload": wl, "op": op, "ms": ms, "rate": rate, "unit": unit,
                          "frac_of_peak": rate / peak, **extra}), flush=True)

    for k in (1, 2, 3, 4, 5):
        w = workload(k)
        lens, d, hq, hkv = w.block_lens, w.head_dim, w.n_q_heads, w.n_kv_heads
        dt = w.dtype
        esz = 4 if dt == "f32" else 2
        n = w.n_tokens
        patterns = [(nm, PATTERNS[nm]) for nm in w.patterns] or [("dbsa", (w.sink, w.j))]
        if k != 4:
            q = randn((n, hq, d), 11, dt, dev)
            kk = randn((n, hkv, d), 12, dt, dev)
            vv = randn((n, hkv, d), 13, dt, dev)
            o = torch.empty_like(q)
            for nm, (sk, jj) in patterns:
                jj = len(lens) if jj < 0 else jj
                pw = prefill_work(lens, sk, jj, hq, hkv, d)
                ms = timed(lambda: dbsa.dbsa_prefill(q, kk, vv, lens, sk, jj, w.theta, out=o),
                           5 if k != 5 else 3)
                # Skipping masked blocks: time should follow the executed tiles.
                emit(w.name, f"prefill[{nm}]", ms, pw["exact_flop"], "TFLOP/s",
                     executed_tiles_per_head=pw["executed_tiles_per_head"],
                     ms_per_1000_tiles=ms / (pw["executed_tiles_per_head"] / 1000.0),
                     note="exact visible-pair flop")
        if w.append_len:
            la = w.append_len
            qa = randn((la, hq, d), 14, dt, dev)
            ka = randn((la, hkv, d), 15, dt, dev)
            va = randn((la, hkv, d), 16, dt, dev)
            # Constant cost per new block [Notes, Highlights]: the same block
            # appended onto pools of 32, 64 and 128 blocks of the stress
            # lengths, with the anchor and the last j blocks (the ones the new
            # block sees) held at 1024 tokens so that only the pool grows.
            for nb in (32, 64, 128):
                lens_p = lens[:nb].copy()
                lens_p[0] = 1024
                lens_p[nb - w.j:] = 1024
                npool = int(lens_p.sum())
                if npool > n:
                    continue
                kc = torch.empty((npool + la, hkv, d), dtype=kk.dtype, device=dev)
                vc = torch.empty_like(kc)
                kc[:npool].copy_(kk[:npool])
                vc[:npool].copy_(vv[:npool])
                lens_a = np.append(lens_p, la).astype(np.int32)
                new_pairs = visible_pairs(lens_a, w.sink, w.j) - visible_pairs(lens_p, w.sink, w.j)
                ms = timed(lambda: dbsa.dbsa_append_block(qa, ka, va, kc, vc, lens_p, w.sink,
                                                          w.j, w.theta), 7)
                emit(w.name, f"append_block[pool of {nb} blocks]", ms,
                     4.0 * d * hq * new_pairs, "TFLOP/s",
                     note=f"{la} new tokens, {new_pairs / la:.0f} visible keys per row on "
                          f"average, pool {npool} tokens")
                del kc, vc
        if w.n_new == 0:
            continue
        layers = w.layers
        batch = w.batch
        nn = w.n_new
        if k == 4:
            st2 = Stage2Case(4, dev)
            pool_k, pool_v = st2.pool_k, st2.pool_v
            # The one-time setup of the pool: Stage 1 of every layer in one
            # dbsa_prefill_layers call (one query tensor stands in for every
            # layer's; the cost does not depend on it).
            qs = randn((n, hq, d), 11, dt, dev)
            os_ = torch.empty((layers, n, hq, d), dtype=qs.dtype, device=dev)
            ms = timed(lambda: dbsa.dbsa_prefill_layers(qs, pool_k, pool_v, lens, w.sink, w.j,
                                                        w.theta, out=os_), 2)
            emit(w.name, f"prefill[{layers} layers]", ms,
                 layers * 4.0 * d * hq * visible_pairs(lens, w.sink, w.j), "TFLOP/s",
                 note="exact visible-pair flop, every layer of the pool (dbsa_prefill_layers)")
            del qs, os_
        else:
            pool_k, pool_v = [kk], [vv]
        tp = [int(lens[r].sum()) for r in w.ids]
        qn = randn((batch, nn, hq, d), 21, dt, dev)
        kn = randn((batch, nn, hkv, d), 22, dt, dev)
        vn = randn((batch, nn, hkv, d), 23, dt, dev)
        on = torch.empty_like(qn)
        steps = max(w.decode_steps, 0)
        tail_cap = nn + steps
        kt = torch.empty((batch, tail_cap, hkv, d), dtype=qn.dtype, device=dev)
        vt = torch.empty_like(kt)
        kv_bytes = sum(tp) * hkv * d * esz * 2
        io = (qn.numel() + kn.numel() + vn.numel() + on.numel()) * esz

        def fused_all():
            for l in range(len(pool_k)):
                dbsa.dbsa_query_attn_gathered(qn, kn, vn, pool_k[l], pool_v[l], lens, w.ids, kt,
                                              vt, [0] * batch, w.theta, out=on)
        ms = timed(fused_all, 5, flush_first=True)
        emit(w.name, f"fused_gather_query[{len(pool_k)} layers x {batch} x {nn} tokens]", ms,
             len(pool_k) * (kv_bytes + io), "GB/s",
             note="unrotated K/V of the gathered blocks read once + Q, new K/V, O")
        if len(pool_k) == 1:
            cap = max(tp) + nn + steps
            kg = torch.empty((batch, cap, hkv, d), dtype=qn.dtype, device=dev)
            vg = torch.empty_like(kg)
            ms_g = timed(lambda: dbsa.dbsa_gather_rope(kk, vv, lens, w.ids, w.theta, k_out=kg,
                                                       v_out=vg), 5, flush_first=True)
            emit(w.name, "gather_rope", ms_g, 2 * kv_bytes, "GB/s",
                 note="read + write of the gathered K/V")
            ms_q = timed(lambda: dbsa.dbsa_query_attn(qn, kn, vn, kg, vg, tp, w.theta, out=on),
                         5, flush_first=True)
            emit(w.name, "query_attn", ms_q, kv_bytes + io, "GB/s",
                 note="rotated K/V of the context read once + Q, new K/V, O")
        if steps:
            q1 = randn((batch, 1, hq, d), 31, dt, dev)
            k1 = randn((batch, 1, hkv, d), 32, dt, dev)
            v1 = randn((batch, 1, hkv, d), 33, dt, dev)
            o1 = torch.empty_like(q1)

            def decode():
                for s in range(steps):
                    dbsa.dbsa_query_attn_gathered(q1, k1, v1, kk, vv, lens, w.ids, kt, vt,
                                                  [nn + s] * batch, w.theta, out=o1)
            ms = timed(decode, 3, flush_first=True)
            byt = steps * kv_bytes
            emit(w.name, f"decode[{steps} steps]", ms, byt, "GB/s",
                 note="per step: the gathered K/V read once (tail tokens not counted)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate oracle time budget for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-op", choices=["prefill", "append", "fused", "batched", "copy"],
                    help="run only this operation --steps times (for rocprofv3); prints timing")
    ap.add_argument("--profile-workload", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="workload of --profile-op (4: one layer of the pool)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="time every operation of the five workloads (one JSON line each)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DBSA hot path here runs on a single "
              "MI355X (no multi-GPU path is built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_attention_sink_amd import dbsa

    dbsa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.all_workloads:
        run_all_workloads(dev)
    elif args.profile_op:
        profile_op(dev, args.profile_op, args.profile_workload, args.steps, args.warmup)
    else:
        run_main(args, dev)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the DBSA hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic batch of the
Llama-2-7B-shaped layer (30 blocks x 1024 tokens, 32 MHA heads, d = 128,
bf16, sink + previous 2 blocks):
  * dbsa_prefill            block-sparse streaming prefill of the pool
                            (mask -> key-tile walk, RoPE, flash attention;
                            the unrotated K/V stay as the cache),
  * dbsa_gather_rope        gather of anchor + 9 selected blocks, re-RoPE,
  * dbsa_query_attn         64 query tokens over the gathered cache.
Prints one JSON line.  `value` = prefill FLOP on executed (unmasked) 64-key
tiles per step / step time.  The roofline object is for the dominant call,
dbsa_prefill (K-tile pack + flash kernel), timed with HIP events on the
stream it runs on.  The CPU baseline is the fp64 oracle on a bounded row
sample of the same workload, on this host's cores.
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
KEY_TILE, ROW_TILE = 64, 256
PREFILL_PROFILE = os.path.join(ROOT, "profiles", "k_prefill_bf16_llama2_30x1024.md")
PREFILL_SOURCES = [os.path.join(ROOT, "block_sparse_attention_sink_amd", "csrc", f)
                   for f in ("k_stage1.hip", "dbsa_device.hpp", "dbsa_internal.hpp")]


def visible_pairs(lens, sink, j):
    """Sum over rows of the visible-key count (interval form of the block mask)."""
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total = 0
    for i, L in enumerate(lens):
        lo = max(i - j, 0)
        extra = lens[0] if (sink and lo > 0) else 0
        total += int(L) * int(off[i] - off[lo] + extra) + int(L) * (int(L) + 1) // 2
    return total


def executed_tiles(lens, sink, j):
    """64-key tiles the prefill walks, summed over 256-row query tiles."""
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = int(off[-1])
    nb = len(lens)
    blk_of = lambda t: int(np.searchsorted(off, t, side="right") - 1)
    lo_of = lambda t: int(off[max(min(blk_of(t), nb - 1) - j, 0)])
    tiles = 0
    for r0 in range(0, n, ROW_TILE):
        r1 = min(r0 + ROW_TILE, n)
        w0 = lo_of(r0) // KEY_TILE
        w1 = -(-r1 // KEY_TILE)
        ns = min(-(-int(off[1]) // KEY_TILE), w0) if (sink and lo_of(r1 - 1) > 0) else 0
        tiles += ns + (w1 - w0)
    return tiles


def source_digest(paths):
    """sha256 over the concatenated bytes of the kernel's source files."""
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate oracle time budget for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-op", choices=["prefill", "gather", "query", "fused", "copy"],
                    help="run only this operation --steps times (for rocprofv3); prints timing")
    ap.add_argument("--profile-workload", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="workload of --profile-op prefill / fused (4: one layer of the pool)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="time every operation of the five workloads (one JSON line each)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DBSA hot path here runs on a single "
              "MI355X (no multi-GPU path is built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_attention_sink_amd import dbsa
    from block_sparse_attention_sink_amd.inputs import randn, workload

    dbsa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.all_workloads:
        run_all_workloads(dev)
        return
    if args.profile_op in ("prefill", "fused") and args.profile_workload != 2:
        profile_workload_op(dev, args.profile_op, args.profile_workload, args.steps, args.warmup)
        return
    w = workload(2)
    lens, sink, j, theta = w.block_lens, w.sink, w.j, w.theta
    n, hq, hkv, d = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim
    ids = w.ids
    n_new = w.n_new
    tp = int(lens[ids[0]].sum())

    q = randn((n, hq, d), 1001, "bf16", dev)
    k = randn((n, hkv, d), 1002, "bf16", dev)
    v = randn((n, hkv, d), 1003, "bf16", dev)
    o = torch.empty_like(q)
    qn = randn((1, n_new, hq, d), 1004, "bf16", dev)
    kn = randn((1, n_new, hkv, d), 1005, "bf16", dev)
    vn = randn((1, n_new, hkv, d), 1006, "bf16", dev)
    on = torch.empty_like(qn)
    kg = torch.empty((1, tp + n_new, hkv, d), dtype=torch.bfloat16, device=dev)
    vg = torch.empty_like(kg)
    ctx = np.array([tp], np.int64)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = []

    def step(record=False):
        e = [ev() for _ in range(4)] if record else None
        if record:
            e[0].record()
        dbsa.dbsa_prefill(q, k, v, lens, sink, j, theta, out=o)
        if record:
            e[1].record()
        dbsa.dbsa_gather_rope(k, v, lens, ids, theta, k_out=kg, v_out=vg)
        if record:
            e[2].record()
        dbsa.dbsa_query_attn(qn, kn, vn, kg, vg, ctx, theta, out=on)
        if record:
            e[3].record()
            marks.append(e)

    if args.profile_op:
        tail_k = torch.empty((1, n_new, hkv, d), dtype=torch.bfloat16, device=dev)
        tail_v = torch.empty_like(tail_k)
        copy_src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        copy_dst = torch.empty_like(copy_src)
        ops = {
            "prefill": lambda: dbsa.dbsa_prefill(q, k, v, lens, sink, j, theta, out=o),
            "gather": lambda: dbsa.dbsa_gather_rope(k, v, lens, ids, theta, k_out=kg, v_out=vg),
            "query": lambda: dbsa.dbsa_query_attn(qn, kn, vn, kg, vg, ctx, theta, out=on),
            "fused": lambda: dbsa.dbsa_query_attn_gathered(qn, kn, vn, k, v, lens, ids, tail_k,
                                                           tail_v, [0], theta, out=on),
            "copy": lambda: copy_dst.copy_(copy_src),
        }
        fn = ops[args.profile_op]
        dbsa.dbsa_gather_rope(k, v, lens, ids, theta, k_out=kg, v_out=vg)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a0, a1 = ev(), ev()
        a0.record()
        for _ in range(args.steps):
            fn()
        a1.record()
        torch.cuda.synchronize()
        print(json.dumps({"profile_op": args.profile_op, "steps": args.steps,
                          "ms_per_call": a0.elapsed_time(a1) / args.steps,
                          "copy_bytes_read": copy_src.numel() * 4}))
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = ev(), ev()
    t0.record()
    for _ in range(args.steps):
        step(record=True)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    ms_prefill = float(np.mean([m[0].elapsed_time(m[1]) for m in marks]))
    ms_gather = float(np.mean([m[1].elapsed_time(m[2]) for m in marks]))
    ms_query = float(np.mean([m[2].elapsed_time(m[3]) for m in marks]))

    pairs = visible_pairs(lens, sink, j)
    exact_flop = 4.0 * d * hq * pairs
    tiles = executed_tiles(lens, sink, j)
    tile_flop = 4.0 * d * hq * tiles * ROW_TILE * KEY_TILE
    value = tile_flop / (ms_step * 1e-3) / 1e12
    achieved = exact_flop / (ms_prefill * 1e-3) / 1e12

    # Stage 2 alone, caches flushed between repetitions by reading 1 GiB (a
    # read leaves clean lines; a write-based flush would leave up to the
    # last-level cache's size of dirty lines to be written back inside the
    # timed call).
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    kv_bytes = tp * hkv * d * 2 * 2
    io_bytes = (qn.numel() + kn.numel() + vn.numel() + on.numel()) * 2
    tail_k = torch.empty((1, n_new, hkv, d), dtype=torch.bfloat16, device=dev)
    tail_v = torch.empty_like(tail_k)

    def timed(fn, reps=10):
        ts = []
        for _ in range(reps + 2):
            flush_sink.add_(flush.sum())
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts[2:]))

    g_ms = timed(lambda: dbsa.dbsa_gather_rope(k, v, lens, ids, theta, k_out=kg, v_out=vg))
    q_ms = timed(lambda: dbsa.dbsa_query_attn(qn, kn, vn, kg, vg, ctx, theta, out=on))
    f_ms = timed(lambda: dbsa.dbsa_query_attn_gathered(qn, kn, vn, k, v, lens, ids, tail_k, tail_v,
                                                       [0], theta, out=on))
    stage2 = {
        "context_tokens": tp, "query_tokens": n_new,
        "gather_rope": {"us": g_ms * 1e3, "GB/s": 2 * kv_bytes / (g_ms * 1e-3) / 1e9,
                        "bytes": 2 * kv_bytes},
        "query_attn": {"us": q_ms * 1e3, "GB/s": (kv_bytes + io_bytes) / (q_ms * 1e-3) / 1e9,
                       "bytes": kv_bytes + io_bytes},
        "gather_plus_query": {"us": (g_ms + q_ms) * 1e3,
                              "GB/s": (kv_bytes + io_bytes) / ((g_ms + q_ms) * 1e-3) / 1e9},
        "fused_gather_query": {"us": f_ms * 1e3,
                               "GB/s": (kv_bytes + io_bytes) / (f_ms * 1e-3) / 1e9,
                               "frac_hbm": (kv_bytes + io_bytes) / (f_ms * 1e-3) / 1e9
                               / PEAK_HBM_GBS},
        "note": "algorithmic bytes = unrotated K+V of the gathered tokens read once + Q, new K/V, "
                "O; gather counts its read and write; caches flushed (1 GiB read) between "
                "repetitions",
    }

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import dbsa_oracle as orc
        h = lambda t: t.float().cpu().numpy().astype(np.float64)
        qh, kh, vh = h(q), h(k), h(v)
        rng = np.random.default_rng(7)
        # Random rows of the whole pool, in batches, until about --cpu-seconds
        # of oracle time have been spent.
        order = rng.permutation(n)
        done, secs = 0, 0.0
        while secs < args.cpu_seconds and done < min(n, 8192):
            batch = np.sort(order[done:done + 64])
            t = time.perf_counter()
            orc.prefill(qh, kh, vh, lens, sink, j, theta, rows=batch)
            secs += time.perf_counter() - t
            done += batch.size
        rows = order[:done]
        n_rows = done
        off = np.concatenate([[0], np.cumsum(lens)])
        blk = np.searchsorted(off, rows, side="right") - 1
        lo = off[np.maximum(blk - j, 0)]
        vis = (rows - lo + 1) + np.where((lo > 0) & bool(sink), lens[0], 0)
        cpu = {"value": 4.0 * d * hq * float(vis.sum()) / secs / 1e12, "unit": "TFLOP/s",
               "cores": cpu_threads(), "kind": "oracle",
               "sample": f"dbsa_prefill oracle (fp64 masked-dense NumPy) on {n_rows} random rows "
                         f"x all {hq} heads of the same workload, {secs:.1f} s; value counts the "
                         "exact visible pairs of the sampled rows"}

    traffic = profile_traffic(PREFILL_PROFILE, PREFILL_SOURCES)
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
        "config": {"workload": w.name, "n_tokens": n, "n_blocks": int(lens.size),
                   "block_len": int(lens[0]), "q_heads": hq, "kv_heads": hkv, "head_dim": d,
                   "sink": sink, "j": j, "rope_theta": theta, "stage2_blocks": int(ids.shape[1]),
                   "stage2_context": tp, "query_tokens": n_new, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "dbsa_prefill call = k_pack_bf16 + k_prefill_bf16",
                     "ms_per_launch": ms_prefill,
                     "algorithmic_flop_per_launch": exact_flop},
        "prefill": {"exact_pairs_per_head": pairs, "exact_TFLOP": exact_flop / 1e12,
                    "executed_tiles_per_head": tiles,
                    "tile_rows_x_keys": [ROW_TILE, KEY_TILE],
                    "executed_tile_TFLOP": tile_flop / 1e12,
                    "exact_TFLOP/s": exact_flop / (ms_prefill * 1e-3) / 1e12,
                    "executed_tile_TFLOP/s": tile_flop / (ms_prefill * 1e-3) / 1e12},
        "step_breakdown_ms": {"prefill": ms_prefill, "gather_rope": ms_gather,
                              "query_attn": ms_query},
        "stage2": stage2,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def profile_workload_op(dev, op, k, steps, warmup):
    """Run one hot-path operation of workload k `steps` times (for rocprofv3):
    the prefill of its pool, or the fused gather + query of its batch (one
    layer)."""
    import torch
    from block_sparse_attention_sink_amd import dbsa
    from block_sparse_attention_sink_amd.inputs import randn, workload

    w = workload(k)
    n, hq, hkv, d, dt = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype
    kk = randn((n, hkv, d), 12, dt, dev)
    vv = randn((n, hkv, d), 13, dt, dev)
    if op == "prefill":
        q = randn((n, hq, d), 11, dt, dev)
        o = torch.empty_like(q)
        fn = lambda: dbsa.dbsa_prefill(q, kk, vv, w.block_lens, w.sink, w.j, w.theta, out=o)
    else:
        if w.n_new == 0:
            raise SystemExit(f"workload {k} has no Stage-2 queries")
        b, nn = w.batch, w.n_new
        qn = randn((b, nn, hq, d), 21, dt, dev)
        kn = randn((b, nn, hkv, d), 22, dt, dev)
        vn = randn((b, nn, hkv, d), 23, dt, dev)
        on = torch.empty_like(qn)
        kt = torch.empty((b, nn, hkv, d), dtype=qn.dtype, device=dev)
        vt = torch.empty_like(kt)
        fn = lambda: dbsa.dbsa_query_attn_gathered(qn, kn, vn, kk, vv, w.block_lens, w.ids, kt,
                                                   vt, [0] * b, w.theta, out=on)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(steps):
        fn()
    a1.record()
    torch.cuda.synchronize()
    print(json.dumps({"profile_op": op, "workload": w.name, "steps": steps,
                      "ms_per_call": a0.elapsed_time(a1) / steps}))


def run_all_workloads(dev):
    """Median time of every hot-path operation on the five workloads (caches
    flushed before each Stage-2 repetition), with its algorithmic rate."""
    import torch
    from block_sparse_attention_sink_amd import dbsa
    from block_sparse_attention_sink_amd.inputs import PATTERNS, randn, workload

    ev = lambda: torch.cuda.Event(enable_timing=True)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink_acc = torch.zeros((), dtype=torch.float32, device=dev)

    def timed(fn, reps, flush_first=False):
        ts = []
        for r in range(reps + 2):
            if flush_first:
                sink_acc.add_(flush.sum())
            a, b = ev(), ev()
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
                flop = 4.0 * d * hq * visible_pairs(lens, sk, jj)
                ms = timed(lambda: dbsa.dbsa_prefill(q, kk, vv, lens, sk, jj, w.theta, out=o),
                           5 if k != 5 else 3)
                emit(w.name, f"prefill[{nm}]", ms, flop, "TFLOP/s",
                     note="exact visible-pair flop")
        if w.append_len:
            la = w.append_len
            cap = n + la
            kc = torch.empty((cap, hkv, d), dtype=kk.dtype, device=dev)
            vc = torch.empty_like(kc)
            kc[:n].copy_(kk)
            vc[:n].copy_(vv)
            qa = randn((la, hq, d), 14, dt, dev)
            ka = randn((la, hkv, d), 15, dt, dev)
            va = randn((la, hkv, d), 16, dt, dev)
            lens_a = np.append(lens, la).astype(np.int32)
            new_pairs = visible_pairs(lens_a, w.sink, w.j) - visible_pairs(lens, w.sink, w.j)
            ctx = new_pairs / la
            flop = 4.0 * d * hq * new_pairs
            ms = timed(lambda: dbsa.dbsa_append_block(qa, ka, va, kc, vc, lens, w.sink, w.j,
                                                      w.theta), 5)
            emit(w.name, "append_block", ms, flop, "TFLOP/s",
                 note=f"{la} new tokens, {ctx:.0f} visible keys per row on average")
        if w.n_new == 0:
            continue
        layers = w.layers
        batch = w.batch
        nn = w.n_new
        if k == 4:
            pool_k = torch.empty((layers, n, hkv, d), dtype=torch.bfloat16, device=dev)
            pool_v = torch.empty_like(pool_k)
            for l in range(layers):
                pool_k[l].copy_(randn((n, hkv, d), 100 + l, dt, dev))
                pool_v[l].copy_(randn((n, hkv, d), 200 + l, dt, dev))
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


if __name__ == "__main__":
    main()

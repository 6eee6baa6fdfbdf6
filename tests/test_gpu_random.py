"""Randomised GPU parity against the oracle: prefill and append [Notes, Method > Stage 1,
items 2-4], the shared-block and the per-query Stage 2 [Notes, Method > Stage 2, items 1-4].

Each case draws its own shapes from a fixed seed: GQA groups 1-8 (1 to 8 KV heads), head
dim 64 or 128, 2-13 blocks of 1-699 tokens (now and then a one-token block), sink on or
off, j = 0-4, theta 1e4 or 5e5; appends of 1-1099 tokens; Stage-2 batches of 1-6 rows with
1-49 new tokens, 1-12 selected blocks in given or encoded order and tail buffers of 0-19
tokens.  The draws are deterministic, so the cases are the same on every run.
"""
import numpy as np
import pytest
import torch

from oracle import dbsa_oracle as orc
from block_sparse_attention_sink_amd import dbsa
from block_sparse_attention_sink_amd.inputs import randn
from tests.helpers import assert_close, host64
from tests.test_gpu_batched import _check_rows, _ids, _inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for case in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        hq = hkv * int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        nb = int(rng.integers(2, 14))
        lens = rng.integers(1, 700, size=nb).astype(np.int32)
        if rng.random() < 0.3:
            lens[rng.integers(0, nb)] = 1
        c = dict(case=case, hq=hq, hkv=hkv, d=d, lens=lens, sink=int(rng.integers(0, 2)),
                 j=int(rng.integers(0, 5)), theta=float(rng.choice([1e4, 5e5])),
                 seed=int(rng.integers(0, 10000)), kind=case % 3)
        if c["kind"] == 0:
            c["la"] = int(rng.integers(1, 1100))
        else:
            batch = int(rng.integers(1, 7))
            c["n_new"] = int(rng.integers(1, 50))
            n_pick = int(rng.integers(1, nb))
            c["ids"] = _ids(rng, nb, batch, n_pick, shuffle=bool(rng.integers(0, 2)))
            tail = rng.integers(0, 20, size=batch).astype(np.int64)
            if rng.random() < 0.5:
                tail[:] = 0
            c["tail"] = tail
        out.append(c)
    return out


CASES = _cases(12, 45)


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"case{c['case']}")
def test_random_case(c):
    hq, hkv, d, lens, theta, seed = c["hq"], c["hkv"], c["d"], c["lens"], c["theta"], c["seed"]
    n = int(lens.sum())
    what = (f"case {c['case']} hq={hq} hkv={hkv} d={d} lens={lens.tolist()} sink={c['sink']} "
            f"j={c['j']}")
    if c["kind"] == 0:
        q = randn((n, hq, d), seed, "bf16", DEV)
        k = randn((n, hkv, d), seed + 1, "bf16", DEV)
        v = randn((n, hkv, d), seed + 2, "bf16", DEV)
        o = dbsa.dbsa_prefill(q, k, v, lens, c["sink"], c["j"], theta)
        torch.cuda.synchronize()
        want = orc.prefill(host64(q), host64(k), host64(v), lens, c["sink"], c["j"], theta)
        assert_close(host64(o), want, "bf16", what + " prefill")
        la = c["la"]
        qa = randn((la, hq, d), seed + 3, "bf16", DEV)
        ka = randn((la, hkv, d), seed + 4, "bf16", DEV)
        va = randn((la, hkv, d), seed + 5, "bf16", DEV)
        kc = torch.zeros((n + la, hkv, d), dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros_like(kc)
        kc[:n].copy_(k)
        vc[:n].copy_(v)
        oa = dbsa.dbsa_append_block(qa, ka, va, kc, vc, lens, c["sink"], c["j"], theta)
        torch.cuda.synchronize()
        full = orc.prefill(np.concatenate([host64(q), host64(qa)]), host64(kc), host64(vc),
                           np.append(lens, la).astype(np.int32), c["sink"], c["j"], theta)
        assert_close(host64(oa), full[n:], "bf16", what + f" append of {la}")
        assert torch.equal(kc[n:], ka) and torch.equal(vc[n:], va)
    else:
        ids, tail, n_new = c["ids"], c["tail"], c["n_new"]
        batch = ids.shape[0]
        k, v, q, kn, vn, tk, tv = _inputs(lens, batch, n_new, tail, hq, hkv, d, seed)
        tk0, tv0 = tk.clone(), tv.clone()
        fn = dbsa.dbsa_query_attn_batched if c["kind"] == 1 else dbsa.dbsa_query_attn_gathered
        out = fn(q, kn, vn, k, v, lens, ids, tk, tv, tail, theta)
        torch.cuda.synchronize()
        _check_rows(lens, ids, tail, k, v, q, kn, vn, tk0, tv0, tk, tv, out, theta,
                    what + f" {fn.__name__} ids={ids.tolist()} tail={tail.tolist()}")

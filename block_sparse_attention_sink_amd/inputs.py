"""Seeded synthetic workloads for DBSA.

This module only draws inputs: block lengths, selected block ids and N(0,1)
tensors.  It contains none of the method's arithmetic, so both the HIP path's
tests and the oracle's tests may use it.

The shapes follow the paper-notes page "Efficient Many-Shot In-Context
Learning with Dynamic Block-Sparse Attention" [Notes]: 50 demonstrations per
block, previous j = 2 blocks, 30% retrieval ratio (Method > configuration),
30k / 90k-token contexts on Llama-2-7B / Llama-3.1-8B shapes (Experiments >
setup) and a KV cache of 0.125 MiB per token (Ablations > storage cost).
No dataset or model is used: token content is random.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = ["Workload", "workload", "WORKLOADS", "block_lengths_stress", "select_ids",
           "randn", "PATTERNS", "llama31_inv_freq"]

# (sink, j) of the ablation patterns [Notes, Ablations > sparse attention pattern]
# j = -1 stands for "full causal" and is replaced by n_blocks - 1 at use.
PATTERNS = {
    "self_only": (0, 0),
    "sink_self": (1, 0),
    "sink_prev2_self": (1, 2),
    "sink_prev8_self": (1, 8),
    "full_causal": (1, -1),
}


@dataclass
class Workload:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                      # "bf16" | "f32"
    block_lens: np.ndarray          # int32 [n_blocks], tokens
    sink: int
    j: int
    theta: float
    ids: np.ndarray                 # int32 [batch, n_ids], anchor first
    n_new: int                      # query tokens per batch row
    decode_steps: int = 0
    layers: int = 1
    append_len: int = 0
    patterns: List[str] = field(default_factory=list)
    seed: int = 0

    @property
    def n_tokens(self) -> int:
        return int(np.sum(self.block_lens))

    @property
    def n_blocks(self) -> int:
        return int(self.block_lens.size)

    @property
    def batch(self) -> int:
        return int(self.ids.shape[0])


def select_ids(rng: np.random.Generator, n_blocks: int, n_pick: int) -> np.ndarray:
    """Anchor block 0 followed by n_pick distinct other blocks in encoded order."""
    pick = np.sort(rng.choice(np.arange(1, n_blocks), size=n_pick, replace=False))
    return np.concatenate([[0], pick]).astype(np.int32)


def _demo_block_lengths(rng: np.random.Generator, n_blocks: int) -> np.ndarray:
    # 50 demonstrations per block, each 12..28 tokens long (uniform).
    return rng.integers(12, 29, size=(n_blocks, 50)).sum(axis=1).astype(np.int32)


def block_lengths_stress(rng: np.random.Generator, n_blocks: int = 128, total: int = 131072,
                         lo: int = 512, hi: int = 2048) -> np.ndarray:
    """Variable block lengths in [lo, hi] that sum to `total`.

    Draw uniformly, pin one block at lo and one at hi (edge coverage), then
    move the other blocks by +-1 token at random, within [lo, hi], until the
    sum is `total`.
    """
    lens = rng.integers(lo, hi + 1, size=n_blocks).astype(np.int64)
    pinned = rng.choice(np.arange(1, n_blocks), size=2, replace=False)
    lens[pinned[0]] = lo
    lens[pinned[1]] = hi
    free = np.setdiff1d(np.arange(n_blocks), pinned)
    diff = int(lens.sum()) - total
    while diff != 0:
        step = -1 if diff > 0 else 1
        cand = rng.choice(free, size=min(abs(diff), free.size), replace=False)
        ok = cand[(lens[cand] + step >= lo) & (lens[cand] + step <= hi)]
        lens[ok] += step
        diff += step * ok.size
    return lens.astype(np.int32)


def workload(k: int, seed: Optional[int] = None) -> Workload:
    """The five measured/tested workloads (k = 1..5)."""
    seed = k if seed is None else seed
    rng = np.random.default_rng(seed)
    if k == 1:
        lens = np.full(8, 128, np.int32)
        return Workload("tiny_mha1_d64_f32_8x128", 1, 1, 64, "f32", lens, 1, 2, 1e4,
                        np.array([[0, 3, 6]], np.int32), 16, seed=seed)
    if k == 2:
        lens = np.full(30, 1024, np.int32)
        return Workload("llama2_7b_mha32_d128_bf16_30x1024", 32, 32, 128, "bf16", lens, 1, 2,
                        1e4, select_ids(rng, 30, 9)[None, :], 64, seed=seed)
    if k == 3:
        lens = _demo_block_lengths(rng, 90)
        return Workload("llama31_8b_gqa32x8_d128_bf16_90blk_demo12to28", 32, 8, 128, "bf16",
                        lens, 1, 2, 5e5, select_ids(rng, 90, 27)[None, :], 64,
                        decode_steps=16, seed=seed)
    if k == 4:
        lens = _demo_block_lengths(rng, 90)
        ids = np.stack([select_ids(rng, 90, 27) for _ in range(64)])
        return Workload("llama31_8b_pool32layers_90k_batch64x48", 32, 8, 128, "bf16", lens, 1,
                        2, 5e5, ids, 48, layers=32, seed=seed)
    if k == 5:
        lens = block_lengths_stress(rng)
        return Workload("stress_gqa32x8_d128_bf16_128blk_512to2048_131072", 32, 8, 128, "bf16",
                        lens, 1, 2, 5e5, np.zeros((1, 1), np.int32), 0, append_len=1024,
                        patterns=list(PATTERNS), seed=seed)
    raise ValueError(f"no workload {k}")


WORKLOADS = (1, 2, 3, 4, 5)


def randn(shape, seed: int, dtype: str = "bf16", device: str = "cpu"):
    """N(0,1) tensor from a seeded torch generator, stored in `dtype`.

    bf16 values are the round-to-nearest-even image of float32 draws; the
    oracle reads exactly those stored values.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def llama31_inv_freq(theta: float, head_dim: int, factor: float = 8.0,
                     low_freq_factor: float = 1.0, high_freq_factor: float = 4.0,
                     original_context: int = 8192) -> np.ndarray:
    """A frequency-scaled RoPE table (radians per position) in the form the
    Llama-3.1 models use, as an input for the RoPE-table option of both the
    library and the oracle (the method's pages give only theta).

    With w_i = theta^(-2i/d) and wavelength 2 pi / w_i: frequencies whose
    wavelength is below original_context / high_freq_factor are kept, those
    above original_context / low_freq_factor are divided by `factor`, and the
    band between is blended linearly in original_context / wavelength.
    """
    w = theta ** (-(2.0 * np.arange(head_dim // 2, dtype=np.float64)) / head_dim)
    wavelen = 2.0 * np.pi / w
    lo_wl = original_context / low_freq_factor
    hi_wl = original_context / high_freq_factor
    smooth = (original_context / wavelen - low_freq_factor) / (high_freq_factor - low_freq_factor)
    blended = (1.0 - smooth) * w / factor + smooth * w
    return np.where(wavelen < hi_wl, w, np.where(wavelen > lo_wl, w / factor, blended))

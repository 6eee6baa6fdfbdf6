"""CPU checks of the input generators and of the binding's argument checks.

The Llama-3.1 frequency table is an input (both the library and the oracle
take it); it is pinned against the Llama-3 RoPE initialisation that the
`transformers` package ships, an implementation independent of this one.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_sink_amd import dbsa
from block_sparse_attention_sink_amd.inputs import (block_lengths_stress, llama31_inv_freq,
                                                    select_ids, workload)


@pytest.mark.parametrize("theta,head_dim", [(5e5, 128), (5e5, 64), (1e4, 128)])
def test_llama31_table_matches_transformers(theta, head_dim):
    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    cfg = LlamaConfig(hidden_size=32 * head_dim, num_attention_heads=32, num_key_value_heads=8,
                      head_dim=head_dim, max_position_embeddings=131072,
                      rope_scaling={"rope_type": "llama3", "factor": 8.0, "low_freq_factor": 1.0,
                                    "high_freq_factor": 4.0,
                                    "original_max_position_embeddings": 8192,
                                    "rope_theta": theta})
    ref, _ = ROPE_INIT_FUNCTIONS["llama3"](cfg, torch.device("cpu"))
    ours = llama31_inv_freq(theta, head_dim)
    # transformers computes in float32: a few float32 ulps apart
    np.testing.assert_allclose(ours, ref.double().numpy(), rtol=4e-7, atol=0)
    # the plain frequencies come out when nothing is scaled
    plain = theta ** (-(2.0 * np.arange(head_dim // 2)) / head_dim)
    np.testing.assert_allclose(llama31_inv_freq(theta, head_dim, factor=1.0), plain, rtol=1e-15)


def test_llama31_table_bands():
    table = llama31_inv_freq(5e5, 128)
    plain = 5e5 ** (-(2.0 * np.arange(64)) / 128)
    wl = 2 * np.pi / plain
    hi, lo = wl < 2048, wl > 8192
    np.testing.assert_array_equal(table[hi], plain[hi])
    np.testing.assert_allclose(table[lo], plain[lo] / 8, rtol=1e-15)
    assert np.all(np.diff(table) < 0)
    mid = ~hi & ~lo
    assert np.all(table[mid] <= plain[mid]) and np.all(table[mid] >= plain[mid] / 8)


def test_stress_lengths_and_selection():
    lens = block_lengths_stress(np.random.default_rng(5))
    assert lens.size == 128 and lens.sum() == 131072
    assert lens.min() == 512 and lens.max() == 2048
    ids = select_ids(np.random.default_rng(0), 90, 27)
    assert ids[0] == 0 and ids.size == 28 and np.all(np.diff(ids) > 0)
    w = workload(4)
    assert w.ids.shape == (64, 28) and np.all(w.ids[:, 0] == 0)


# ---------------------------------------------------------------------------
# Binding: mismatched shapes are rejected before anything reaches the library
# (CPU tensors: a call that passed the shape checks would stop at "must be a
# GPU tensor" instead).
# ---------------------------------------------------------------------------
def _t(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _raises_shape(fn, *args, **kw):
    with pytest.raises(dbsa.DbsaError) as e:
        fn(*args, **kw)
    assert e.value.code == dbsa.EINVAL
    assert "shape" in str(e.value) or "holds" in str(e.value) or "rows" in str(e.value), str(e.value)


def test_binding_rejects_shapes_prefill():
    lens = [5, 7]
    _raises_shape(dbsa.dbsa_prefill, _t(11, 4, 64), _t(12, 2, 64), _t(12, 2, 64), lens, 1, 2, 1e4)
    _raises_shape(dbsa.dbsa_prefill, _t(12, 4, 64), _t(12, 2, 64), _t(12, 2, 128), lens, 1, 2, 1e4)
    _raises_shape(dbsa.dbsa_prefill, _t(12, 4, 64), _t(12, 2, 128), _t(12, 2, 128), lens, 1, 2,
                  1e4)
    _raises_shape(dbsa.dbsa_prefill, _t(12, 4, 64), _t(12, 2, 64), _t(12, 2, 64), lens, 1, 2, 1e4,
                  out=_t(12, 2, 64))
    with pytest.raises(dbsa.DbsaError, match="GPU tensor"):
        dbsa.dbsa_prefill(_t(12, 4, 64), _t(12, 2, 64), _t(12, 2, 64), lens, 1, 2, 1e4)
    _raises_shape(dbsa.dbsa_prefill_layers, _t(3, 12, 4, 64), _t(3, 12, 2, 64), _t(2, 12, 2, 64),
                  lens, 1, 2, 1e4)
    _raises_shape(dbsa.dbsa_prefill_layers, _t(3, 12, 4, 64), _t(3, 13, 2, 64), _t(3, 13, 2, 64),
                  lens, 1, 2, 1e4)


def test_binding_rejects_shapes_append():
    lens = [5, 7]
    q, k = _t(4, 4, 64), _t(4, 2, 64)
    _raises_shape(dbsa.dbsa_append_block, q, _t(5, 2, 64), k, _t(20, 2, 64), _t(20, 2, 64), lens,
                  1, 2, 1e4)
    _raises_shape(dbsa.dbsa_append_block, q, k, k, _t(20, 2, 64), _t(21, 2, 64), lens, 1, 2, 1e4)
    _raises_shape(dbsa.dbsa_append_block, q, k, k, _t(20, 4, 64), _t(20, 4, 64), lens, 1, 2, 1e4)


def test_binding_rejects_shapes_stage2():
    lens, ids = [5, 7, 9], [[0, 2]]
    pool = _t(21, 2, 64)
    # pool shorter than the blocks
    _raises_shape(dbsa.dbsa_gather_rope, _t(20, 2, 64), _t(20, 2, 64), lens, ids, 1e4)
    _raises_shape(dbsa.dbsa_gather_rope, pool, _t(21, 2, 128), lens, ids, 1e4)
    _raises_shape(dbsa.dbsa_gather_rope, pool, pool, lens, ids, 1e4, k_out=_t(2, 30, 2, 64),
                  v_out=_t(2, 30, 2, 64))
    q, kn = _t(1, 3, 4, 64), _t(1, 3, 2, 64)
    ctx = _t(1, 40, 2, 64)
    _raises_shape(dbsa.dbsa_query_attn, q, _t(1, 4, 2, 64), kn, ctx, ctx, [10], 1e4)
    _raises_shape(dbsa.dbsa_query_attn, q, kn, kn, ctx, _t(1, 41, 2, 64), [10], 1e4)
    _raises_shape(dbsa.dbsa_query_attn, q, kn, kn, _t(2, 40, 2, 64), _t(2, 40, 2, 64), [10], 1e4)
    _raises_shape(dbsa.dbsa_query_attn, q, kn, kn, ctx, ctx, [10], 1e4, out=_t(1, 3, 2, 64))
    tail = _t(1, 8, 2, 64)
    _raises_shape(dbsa.dbsa_query_attn_gathered, q, kn, kn, _t(20, 2, 64), _t(20, 2, 64), lens,
                  ids, tail, tail, [0], 1e4)
    _raises_shape(dbsa.dbsa_query_attn_gathered, q, kn, kn, pool, pool, lens, [[0, 1], [0, 2]],
                  tail, tail, [0], 1e4)
    _raises_shape(dbsa.dbsa_query_attn_gathered, q, kn, kn, _t(21, 1, 64), _t(21, 1, 64), lens,
                  ids, tail, tail, [0], 1e4)
    _raises_shape(dbsa.dbsa_query_attn_spans, q, kn, kn, pool, pool, [[0, 3]], [[2, 2]],
                  _t(1, 8, 2, 128), _t(1, 8, 2, 128), [0], 1e4)
    _raises_shape(dbsa.dbsa_gather_rope_spans, pool, _t(22, 2, 64), [[0]], [[3]], 1e4)

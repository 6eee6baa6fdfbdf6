"""GPU parity of the HIP path against the CPU oracle (small and medium sizes).

Sizes span several 128-row query tiles and 64-key tiles with ragged tails.
Every call goes through the C ABI (libdbsa.so) via the ctypes binding.
"""
import numpy as np
import pytest
import torch

from oracle import dbsa_oracle as orc
from block_sparse_attention_sink_amd import dbsa
from block_sparse_attention_sink_amd.inputs import llama31_inv_freq, randn
from tests.helpers import assert_close, assert_bf16_rounding, host64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _qkv(n, hq, hkv, d, dtype, seed):
    return (randn((n, hq, d), seed, dtype, DEV), randn((n, hkv, d), seed + 1, dtype, DEV),
            randn((n, hkv, d), seed + 2, dtype, DEV))


def _run_prefill(lens, hq, hkv, d, dtype, sink, j, theta, seed, qmul=1.0):
    n = int(np.sum(lens))
    q, k, v = _qkv(n, hq, hkv, d, dtype, seed)
    if qmul != 1.0:
        q = (q.float() * qmul).to(q.dtype)
    o = dbsa.dbsa_prefill(q, k, v, lens, sink, j, theta)
    torch.cuda.synchronize()
    want = orc.prefill(host64(q), host64(k), host64(v), lens, sink, j, theta)
    return host64(o), want


PATTERNS = [(1, 2), (0, 0), (1, 0), (0, 1), (1, 100)]


@pytest.mark.parametrize("sink,j", PATTERNS)
def test_prefill_bf16_gqa_ragged(sink, j):
    rng = np.random.default_rng(100 + 7 * sink + j)
    lens = rng.integers(1, 300, size=9).astype(np.int32)
    got, want = _run_prefill(lens, 8, 2, 128, "bf16", sink, j, 1e4, seed=11)
    assert_close(got, want, "bf16", f"prefill sink={sink} j={j}")


def test_prefill_bf16_head_dim_64_mha():
    lens = np.array([200, 64, 130, 1, 77, 190], np.int32)
    got, want = _run_prefill(lens, 4, 4, 64, "bf16", 1, 2, 1e4, seed=21)
    assert_close(got, want, "bf16", "prefill d=64")


def test_prefill_bf16_sharp_softmax():
    """Q x 8: peaked softmax rows, so a wrong mask or position shows up sharply.

    Tolerance (derived, not the workload one): rounding the rotated Q and K to
    bf16 perturbs each score by about 8 * 2^-9 * sqrt(2/3) = 0.013 (std), which
    moves the weights of near-tied top keys by a few percent; the normalised
    output error stays near 1e-2.  A wrong mask, position or head mapping moves
    the peak to another key and gives a normalised error of order 1.
    """
    rng = np.random.default_rng(5)
    lens = rng.integers(20, 200, size=8).astype(np.int32)
    got, want = _run_prefill(lens, 4, 1, 128, "bf16", 1, 2, 5e5, seed=31, qmul=8.0)
    nrm = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert nrm <= 3e-2, nrm
    assert np.max(np.abs(got - want)) <= 0.3


def test_prefill_f32_tiny_workload():
    """8 blocks x 128 tokens, one head, d = 64, float32, sink + previous 2."""
    lens = np.full(8, 128, np.int32)
    got, want = _run_prefill(lens, 1, 1, 64, "f32", 1, 2, 1e4, seed=1)
    assert_close(got, want, "f32", "prefill f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_layers_equals_per_layer(dtype):
    """Three layers through one dbsa_prefill_layers call give, bitwise, what
    three dbsa_prefill calls give; a shared Q (stride 0) as well."""
    rng = np.random.default_rng(53)
    lens = rng.integers(30, 400, size=6).astype(np.int32)
    n = int(lens.sum())
    hq, hkv, d = (8, 2, 128) if dtype == "bf16" else (2, 1, 64)
    q = randn((3, n, hq, d), 211, dtype, DEV)
    k = randn((3, n, hkv, d), 212, dtype, DEV)
    v = randn((3, n, hkv, d), 213, dtype, DEV)
    o = dbsa.dbsa_prefill_layers(q, k, v, lens, 1, 2, 5e5)
    o_shared = dbsa.dbsa_prefill_layers(q[1].contiguous(), k, v, lens, 1, 2, 5e5)
    for l in range(3):
        ol = dbsa.dbsa_prefill(q[l].contiguous(), k[l].contiguous(), v[l].contiguous(), lens, 1,
                               2, 5e5)
        os_ = dbsa.dbsa_prefill(q[1].contiguous(), k[l].contiguous(), v[l].contiguous(), lens, 1,
                                2, 5e5)
        torch.cuda.synchronize()
        assert torch.equal(o[l], ol), l
        assert torch.equal(o_shared[l], os_), l
    want = orc.prefill(host64(q[2]), host64(k[2]), host64(v[2]), lens, 1, 2, 5e5)
    assert_close(host64(o[2]), want, dtype, "layer 2")


def test_prefill_mask_probe_exact_fractions():
    """Q = 0, V = one-hot(block): every output is (#visible keys of block b) / |vis(t)|.

    Small blocks keep |vis| under ~170, so one missing or extra key moves an
    output by more than bf16 rounding.
    """
    rng = np.random.default_rng(9)
    lens = rng.integers(1, 40, size=60).astype(np.int32)
    n = int(lens.sum())
    d = 128
    blk = np.repeat(np.arange(lens.size), lens)
    q = torch.zeros((n, 2, d), dtype=torch.bfloat16, device=DEV)
    k = randn((n, 1, d), 3, "bf16", DEV)
    v = torch.zeros((n, 1, d), dtype=torch.float32)
    v[np.arange(n), 0, blk % d] = 1.0  # blocks 0..59 each own a column
    v = v.to(torch.bfloat16).to(DEV)
    for sink, j in [(1, 2), (0, 0), (1, 0), (1, 5), (0, 3)]:
        o = host64(dbsa.dbsa_prefill(q, k, v, lens, sink, j, 1e4))
        want = orc.prefill(np.zeros((n, 2, d)), host64(k), host64(v), lens, sink, j, 1e4)
        assert_bf16_rounding(o, want, f"mask probe sink={sink} j={j}")


def test_prefill_single_block_and_tiny_pool():
    for lens in ([1], [5], [63], [64], [65], [129, 1]):
        lens = np.array(lens, np.int32)
        got, want = _run_prefill(lens, 2, 1, 128, "bf16", 1, 2, 1e4, seed=41)
        assert_close(got, want, "bf16", f"prefill lens={lens.tolist()}")


def test_prefill_one_token_blocks_every_pattern():
    """Blocks of one to three tokens (many blocks per key tile, so every tile
    is partial) under each sink / window pattern."""
    rng = np.random.default_rng(61)
    lens = rng.integers(1, 4, size=150).astype(np.int32)
    for sink, j in PATTERNS:
        got, want = _run_prefill(lens, 4, 2, 64, "bf16", sink, j, 1e4, seed=63)
        assert_close(got, want, "bf16", f"prefill tiny blocks sink={sink} j={j}")


@pytest.mark.parametrize("sink,j", [(1, 2), (0, 5)])
def test_prefill_many_blocks_table_uploaded(sink, j):
    """700 blocks: the block-offset table (701 ints) is too big for the kernel
    arguments and is written into the workspace by copy kernels instead."""
    rng = np.random.default_rng(91 + j)
    lens = rng.integers(1, 5, size=700).astype(np.int32)
    got, want = _run_prefill(lens, 4, 2, 128, "bf16", sink, j, 1e4, seed=93)
    assert_close(got, want, "bf16", f"prefill 700 blocks sink={sink} j={j}")


def test_prefill_repeatable_bitwise():
    rng = np.random.default_rng(77)
    lens = rng.integers(50, 400, size=10).astype(np.int32)
    n = int(lens.sum())
    q, k, v = _qkv(n, 8, 2, 128, "bf16", 51)
    o1 = dbsa.dbsa_prefill(q, k, v, lens, 1, 2, 1e4).clone()
    o2 = dbsa.dbsa_prefill(q, k, v, lens, 1, 2, 1e4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_prefill_leaves_no_stale_output():
    """Every output element is written (NaN-filled output buffer first)."""
    lens = np.array([100, 37, 250, 3], np.int32)
    n = int(lens.sum())
    q, k, v = _qkv(n, 4, 2, 128, "bf16", 61)
    out = torch.full_like(q, float("nan"))
    dbsa.dbsa_prefill(q, k, v, lens, 1, 1, 1e4, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()


# ----------------------------------------------------------------------------
# Append
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("sink,j", [(1, 2), (0, 0), (1, 0), (1, 8)])
def test_append_matches_oracle(dtype, sink, j):
    rng = np.random.default_rng(3 + j)
    lens = rng.integers(30, 260, size=7).astype(np.int32)
    new_len = 173
    n_old = int(lens.sum())
    hq, hkv, d = (4, 2, 128) if dtype == "bf16" else (2, 1, 64)
    q, k, v = _qkv(n_old + new_len, hq, hkv, d, dtype, 71)
    cap = n_old + new_len + 5
    k_cache = torch.zeros((cap, hkv, d), dtype=TORCH_DT[dtype], device=DEV)
    v_cache = torch.zeros_like(k_cache)
    k_cache[:n_old] = k[:n_old]
    v_cache[:n_old] = v[:n_old]
    o_new = dbsa.dbsa_append_block(q[n_old:].contiguous(), k[n_old:].contiguous(),
                                   v[n_old:].contiguous(), k_cache, v_cache, lens, sink, j, 5e5)
    torch.cuda.synchronize()
    want, _, _, _ = orc.append_block(host64(q[n_old:]), host64(k[n_old:]), host64(v[n_old:]),
                                     host64(k[:n_old]), host64(v[:n_old]), lens, sink, j, 5e5)
    assert_close(host64(o_new), want, dtype, f"append sink={sink} j={j}")
    assert torch.equal(k_cache[:n_old + new_len], k)
    assert torch.equal(v_cache[:n_old + new_len], v)


@pytest.mark.parametrize("j", [2, 8])
def test_append_split_keys(j):
    """An append with few query tiles and a long window: its key tiles are cut
    into parts (one workgroup each) whose partials are merged."""
    rng = np.random.default_rng(40 + j)
    lens = rng.integers(500, 700, size=10).astype(np.int32)
    new_len = 300
    n_old = int(lens.sum())
    q, k, v = _qkv(n_old + new_len, 4, 2, 128, "bf16", 131 + j)
    k_cache = torch.zeros((n_old + new_len, 2, 128), dtype=torch.bfloat16, device=DEV)
    v_cache = torch.zeros_like(k_cache)
    k_cache[:n_old] = k[:n_old]
    v_cache[:n_old] = v[:n_old]
    o_new = dbsa.dbsa_append_block(q[n_old:].contiguous(), k[n_old:].contiguous(),
                                   v[n_old:].contiguous(), k_cache, v_cache, lens, 1, j, 5e5)
    torch.cuda.synchronize()
    want, _, _, _ = orc.append_block(host64(q[n_old:]), host64(k[n_old:]), host64(v[n_old:]),
                                     host64(k[:n_old]), host64(v[:n_old]), lens, 1, j, 5e5)
    assert_close(host64(o_new), want, "bf16", f"append split keys j={j}")


def test_append_onto_many_blocks():
    """Append onto a 600-block pool (uploaded offset table), sink + previous 2."""
    rng = np.random.default_rng(95)
    lens = rng.integers(1, 6, size=600).astype(np.int32)
    new_len = 150
    n_old = int(lens.sum())
    q, k, v = _qkv(n_old + new_len, 4, 2, 128, "bf16", 97)
    k_cache = torch.zeros((n_old + new_len, 2, 128), dtype=torch.bfloat16, device=DEV)
    v_cache = torch.zeros_like(k_cache)
    k_cache[:n_old] = k[:n_old]
    v_cache[:n_old] = v[:n_old]
    o_new = dbsa.dbsa_append_block(q[n_old:].contiguous(), k[n_old:].contiguous(),
                                   v[n_old:].contiguous(), k_cache, v_cache, lens, 1, 2, 5e5)
    torch.cuda.synchronize()
    want, _, _, _ = orc.append_block(host64(q[n_old:]), host64(k[n_old:]), host64(v[n_old:]),
                                     host64(k[:n_old]), host64(v[:n_old]), lens, 1, 2, 5e5)
    assert_close(host64(o_new), want, "bf16", "append onto 600 blocks")


def test_workspace_per_stream():
    """Calls on two streams get two workspaces (calls that may overlap must
    not share one), and both results are right while they run side by side."""
    rng = np.random.default_rng(99)
    lens = rng.integers(100, 400, size=8).astype(np.int32)
    n = int(lens.sum())
    q, k, v = _qkv(n, 8, 2, 128, "bf16", 101)
    want = dbsa.dbsa_prefill(q, k, v, lens, 1, 2, 1e4).clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s in (s1, s2):
        with torch.cuda.stream(s):
            outs.append(dbsa.dbsa_prefill(q, k, v, lens, 1, 2, 1e4))
    torch.cuda.synchronize()
    keys = {key for key in dbsa._ws_cache if key[0] == str(q.device)}
    assert (str(q.device), s1.cuda_stream) in keys and (str(q.device), s2.cuda_stream) in keys
    ws1 = dbsa._ws_cache[(str(q.device), s1.cuda_stream)]
    ws2 = dbsa._ws_cache[(str(q.device), s2.cuda_stream)]
    assert ws1.data_ptr() != ws2.data_ptr()
    for o in outs:
        assert torch.equal(o, want)


def test_append_bitwise_equals_prefill_rows_on_tile_boundary():
    """With the pool a multiple of 128 tokens, append visits exactly the key tiles
    the full prefill visits for those rows, in the same order."""
    lens = np.array([256, 128, 384, 128], np.int32)
    new_len = 200
    n_old = int(lens.sum())
    q, k, v = _qkv(n_old + new_len, 8, 2, 128, "bf16", 81)
    full = dbsa.dbsa_prefill(q, k, v, np.append(lens, new_len), 1, 2, 1e4)
    k_cache = torch.zeros_like(k)
    v_cache = torch.zeros_like(v)
    k_cache[:n_old] = k[:n_old]
    v_cache[:n_old] = v[:n_old]
    o_new = dbsa.dbsa_append_block(q[n_old:].contiguous(), k[n_old:].contiguous(),
                                   v[n_old:].contiguous(), k_cache, v_cache, lens, 1, 2, 1e4)
    torch.cuda.synchronize()
    assert torch.equal(o_new, full[n_old:])


# ----------------------------------------------------------------------------
# Stage 2
# ----------------------------------------------------------------------------

def _pool(lens, hkv, d, dtype, seed):
    n = int(np.sum(lens))
    return randn((n, hkv, d), seed, dtype, DEV), randn((n, hkv, d), seed + 1, dtype, DEV)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_rope(dtype):
    rng = np.random.default_rng(13)
    lens = rng.integers(1, 300, size=20).astype(np.int32)
    hkv, d = (4, 128) if dtype == "bf16" else (1, 64)
    kp, vp = _pool(lens, hkv, d, dtype, 91)
    ids = np.array([[0, 3, 17, 5, 9], [0, 19, 1, 2, 11]], np.int32)
    ko, vo, ctx = dbsa.dbsa_gather_rope(kp, vp, lens, ids, 1e4)
    torch.cuda.synchronize()
    for b in range(ids.shape[0]):
        kg, vg = orc.gather_rope(host64(kp), host64(vp), lens, ids[b], 1e4)
        assert ctx[b] == kg.shape[0]
        np.testing.assert_array_equal(host64(vo[b, :ctx[b]]), vg)
        if dtype == "bf16":
            assert_bf16_rounding(host64(ko[b, :ctx[b]]), kg, f"gather K row {b}")
        else:
            assert_close(host64(ko[b, :ctx[b]]), kg, "f32", f"gather K row {b}")


def _stage2_case(dtype, hq, hkv, d, lens, ids, n_new, theta, seed, fused):
    kp, vp = _pool(lens, hkv, d, dtype, seed)
    batch = ids.shape[0]
    q = randn((batch, n_new, hq, d), seed + 5, dtype, DEV)
    kn = randn((batch, n_new, hkv, d), seed + 6, dtype, DEV)
    vn = randn((batch, n_new, hkv, d), seed + 7, dtype, DEV)
    if fused:
        tail_k = torch.zeros((batch, n_new + 3, hkv, d), dtype=TORCH_DT[dtype], device=DEV)
        tail_v = torch.zeros_like(tail_k)
        o = dbsa.dbsa_query_attn_gathered(q, kn, vn, kp, vp, lens, ids, tail_k, tail_v,
                                          [0] * batch, theta)
    else:
        ko, vo, ctx = dbsa.dbsa_gather_rope(kp, vp, lens, ids, theta,
                                            capacity=int(max(lens[r].sum() for r in ids)) + n_new)
        o = dbsa.dbsa_query_attn(q, kn, vn, ko, vo, ctx, theta)
    torch.cuda.synchronize()
    for b in range(batch):
        kg, vg = orc.gather_rope(host64(kp), host64(vp), lens, ids[b], theta)
        want, _, _ = orc.query_attn(host64(q[b]), host64(kn[b]), host64(vn[b]), kg, vg, theta)
        assert_close(host64(o[b]), want, dtype, f"query b={b} fused={fused}")
    return o


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_query_attn(dtype, fused):
    rng = np.random.default_rng(17)
    lens = rng.integers(20, 400, size=16).astype(np.int32)
    ids = np.array([[0, 2, 5, 9, 14], [0, 15, 7, 1, 3]], np.int32)
    hq, hkv, d = (8, 2, 128) if dtype == "bf16" else (2, 1, 64)
    _stage2_case(dtype, hq, hkv, d, lens, ids, 19, 1e4, 101, fused)


def test_query_attn_gqa_many_rows_and_split():
    """64 tokens x 4 heads = 256 packed rows per KV head; long context forces split-K."""
    rng = np.random.default_rng(19)
    lens = rng.integers(300, 1200, size=24).astype(np.int32)
    ids = np.array([[0, 3, 4, 8, 12, 20, 23]], np.int32)
    for fused in (False, True):
        _stage2_case("bf16", 16, 4, 128, lens, ids, 64, 5e5, 111, fused)


def test_query_many_rows_head_dim_64_and_three_waves():
    """Many packed rows per KV head on the 32-row kernels: head_dim 64 with
    two row groups of 80 rows (3 wavefronts each), and head_dim 128 with 76
    rows in one group; both fused and materialised, split and unsplit."""
    rng = np.random.default_rng(43)
    lens = rng.integers(30, 300, size=10).astype(np.int32)
    ids = np.array([[0, 2, 3, 7, 9], [0, 1, 5, 6, 8]], np.int32)
    for fused in (False, True):
        _stage2_case("bf16", 16, 2, 64, lens, ids, 20, 1e4, 191, fused)
        _stage2_case("bf16", 8, 2, 128, lens, ids[:1], 19, 5e5, 193, fused)
    long_lens = rng.integers(900, 1500, size=12).astype(np.int32)
    _stage2_case("bf16", 32, 8, 128, long_lens, np.array([[0, 3, 5, 8, 11]], np.int32), 48, 5e5,
                 195, True)


def test_query_key_halves_row_counts():
    """At most 64 packed rows per KV head run two wavefronts per row set, one
    per half of every key tile, merged at the end: 1, 32, 33 and 40 rows (a
    second row wavefront partly live), both head dims, with split-K over a
    long context and without it over a short one."""
    rng = np.random.default_rng(53)
    short = rng.integers(30, 60, size=6).astype(np.int32)
    long_lens = rng.integers(400, 1200, size=10).astype(np.int32)
    ids_s = np.array([[0, 2, 5]], np.int32)
    ids_l = np.array([[0, 3, 4, 8], [0, 1, 6, 9]], np.int32)
    for fused in (False, True):
        for d in (64, 128):
            _stage2_case("bf16", 8, 2, d, short, ids_s, 10, 1e4, 211 + d, fused)      # 40 rows, one split
            _stage2_case("bf16", 8, 2, d, long_lens, ids_l, 10, 5e5, 213 + d, fused)  # 40 rows, split-K
        _stage2_case("bf16", 4, 4, 128, long_lens, ids_l, 1, 1e4, 217, fused)         # 1 row (MHA decode)
        _stage2_case("bf16", 8, 2, 128, long_lens, ids_l[:1], 8, 1e4, 219, fused)     # 32 rows
        _stage2_case("bf16", 2, 2, 64, short, ids_s, 33, 1e4, 221, fused)             # 33 rows


def test_query_ten_row_groups():
    """300 query tokens x 4-head groups = 1200 packed rows: ten row groups of
    120 rows (four wavefronts), placed eight workgroup ids apart, with and
    without split-K."""
    rng = np.random.default_rng(59)
    lens = rng.integers(100, 700, size=8).astype(np.int32)
    for fused in (False, True):
        _stage2_case("bf16", 8, 2, 128, lens, np.array([[0, 3, 6]], np.int32), 300, 1e4, 231, fused)
    _stage2_case("bf16", 4, 1, 64, lens, np.array([[0, 1, 2, 4, 5, 7]], np.int32), 300, 5e5, 233,
                 True)


def test_query_odd_head_count_pads_the_grid():
    """3 KV heads x 4-head groups x 48 tokens = 192 rows in two row groups: the
    (split, head) work items are not a multiple of 8, so the grid carries
    padding slots that must exit cleanly."""
    rng = np.random.default_rng(47)
    lens = rng.integers(200, 900, size=9).astype(np.int32)
    ids = np.array([[0, 2, 5, 8]], np.int32)
    for fused in (False, True):
        _stage2_case("bf16", 12, 3, 128, lens, ids, 48, 5e5, 201, fused)
        _stage2_case("bf16", 12, 3, 64, lens, ids, 7, 1e4, 203, fused)


def test_query_fused_equals_materialised_bitwise():
    rng = np.random.default_rng(23)
    lens = rng.integers(50, 700, size=12).astype(np.int32)
    ids = np.array([[0, 4, 6, 11], [0, 1, 2, 3]], np.int32)
    a = _stage2_case("bf16", 8, 2, 128, lens, ids, 24, 1e4, 121, False)
    b = _stage2_case("bf16", 8, 2, 128, lens, ids, 24, 1e4, 121, True)
    assert torch.equal(a, b)


def test_rope_frequency_table_prefill_and_stage2():
    """A frequency-scaled RoPE table (Llama-3.1 style) through prefill and both
    Stage-2 paths, against the oracle given the same table."""
    table = llama31_inv_freq(5e5, 128)
    rng = np.random.default_rng(29)
    lens = rng.integers(40, 500, size=7).astype(np.int32)
    got, want = _run_prefill(lens, 8, 2, 128, "bf16", 1, 2, table, seed=151)
    assert_close(got, want, "bf16", "prefill with table")
    ids = np.array([[0, 3, 6, 2]], np.int32)
    a = _stage2_case("bf16", 8, 2, 128, lens, ids, 17, table, 161, False)
    b = _stage2_case("bf16", 8, 2, 128, lens, ids, 17, table, 161, True)
    assert torch.equal(a, b)


def test_anchor_only_and_single_token():
    lens = np.array([70, 33, 90], np.int32)
    _stage2_case("bf16", 4, 4, 128, lens, np.array([[0]], np.int32), 1, 1e4, 131, False)
    _stage2_case("bf16", 4, 4, 128, lens, np.array([[0]], np.int32), 1, 1e4, 131, True)
    _stage2_case("bf16", 4, 1, 64, lens, np.array([[0, 2]], np.int32), 3, 1e4, 141, True)
    # Context of 21 keys: the wavefronts holding keys 32..63 of the only tile
    # see none, and their (empty) softmax state must carry zero weight.
    short = np.array([20, 9], np.int32)
    for fused in (False, True):
        _stage2_case("bf16", 4, 4, 128, short, np.array([[0]], np.int32), 1, 1e4, 143, fused)
        _stage2_case("bf16", 8, 2, 64, short, np.array([[0, 1]], np.int32), 2, 1e4, 145, fused)


@pytest.mark.parametrize("fused", [False, True])
def test_decode_steps(fused):
    """Query tokens then single-token decode steps; each step appends its K/V."""
    rng = np.random.default_rng(29)
    lens = rng.integers(100, 500, size=10).astype(np.int32)
    ids = np.array([[0, 2, 7, 9]], np.int32)
    hq, hkv, d, theta = 8, 2, 128, 5e5
    kp, vp = _pool(lens, hkv, d, "bf16", 151)
    n_q, steps = 12, 4
    q = randn((1, n_q + steps, hq, d), 155, "bf16", DEV)
    kn = randn((1, n_q + steps, hkv, d), 156, "bf16", DEV)
    vn = randn((1, n_q + steps, hkv, d), 157, "bf16", DEV)
    tp = int(lens[ids[0]].sum())
    outs = []
    if fused:
        tk = torch.zeros((1, n_q + steps, hkv, d), dtype=torch.bfloat16, device=DEV)
        tv = torch.zeros_like(tk)
        outs.append(dbsa.dbsa_query_attn_gathered(q[:, :n_q].contiguous(), kn[:, :n_q].contiguous(),
                                                  vn[:, :n_q].contiguous(), kp, vp, lens, ids, tk,
                                                  tv, [0], theta))
        for s in range(steps):
            sl = slice(n_q + s, n_q + s + 1)
            outs.append(dbsa.dbsa_query_attn_gathered(q[:, sl].contiguous(), kn[:, sl].contiguous(),
                                                      vn[:, sl].contiguous(), kp, vp, lens, ids,
                                                      tk, tv, [n_q + s], theta))
    else:
        ko, vo, ctx = dbsa.dbsa_gather_rope(kp, vp, lens, ids, theta, capacity=tp + n_q + steps)
        outs.append(dbsa.dbsa_query_attn(q[:, :n_q].contiguous(), kn[:, :n_q].contiguous(),
                                         vn[:, :n_q].contiguous(), ko, vo, ctx, theta))
        for s in range(steps):
            sl = slice(n_q + s, n_q + s + 1)
            outs.append(dbsa.dbsa_query_attn(q[:, sl].contiguous(), kn[:, sl].contiguous(),
                                             vn[:, sl].contiguous(), ko, vo, [tp + n_q + s], theta))
    torch.cuda.synchronize()
    kg, vg = orc.gather_rope(host64(kp), host64(vp), lens, ids[0], theta)
    want, kc, vc = orc.query_attn(host64(q[0, :n_q]), host64(kn[0, :n_q]), host64(vn[0, :n_q]), kg,
                                  vg, theta)
    assert_close(host64(outs[0][0]), want, "bf16", "query part")
    dec, _, _ = orc.decode([host64(q[0, n_q + s:n_q + s + 1]) for s in range(steps)],
                           [host64(kn[0, n_q + s:n_q + s + 1]) for s in range(steps)],
                           [host64(vn[0, n_q + s:n_q + s + 1]) for s in range(steps)], kc, vc,
                           theta)
    for s in range(steps):
        assert_close(host64(outs[1 + s][0]), dec[s], "bf16", f"decode step {s}")


def test_batched_queries_own_ids():
    """A batch of queries, each with its own selected blocks (anchor first)."""
    rng = np.random.default_rng(31)
    lens = rng.integers(12 * 5, 28 * 5, size=30).astype(np.int32)
    ids = np.stack([np.concatenate([[0], np.sort(rng.choice(np.arange(1, 30), 9, replace=False))])
                    for _ in range(6)]).astype(np.int32)
    for fused in (False, True):
        _stage2_case("bf16", 8, 2, 128, lens, ids, 5, 5e5, 161, fused)


def _span_case(dtype, hq, hkv, d, n_pool, src, ln, n_new, theta, seed):
    """Example-level retrieval: gather pool token spans (fused and via the
    materialised gather) and run the query over them; both against the oracle."""
    kp = randn((n_pool, hkv, d), seed, dtype, DEV)
    vp = randn((n_pool, hkv, d), seed + 1, dtype, DEV)
    batch = src.shape[0]
    q = randn((batch, n_new, hq, d), seed + 5, dtype, DEV)
    kn = randn((batch, n_new, hkv, d), seed + 6, dtype, DEV)
    vn = randn((batch, n_new, hkv, d), seed + 7, dtype, DEV)
    tp = int(ln.sum(axis=1).max())
    ko, vo, ctx = dbsa.dbsa_gather_rope_spans(kp, vp, src, ln, theta, n_q_heads=hq,
                                              capacity=tp + n_new)
    o_mat = dbsa.dbsa_query_attn(q, kn, vn, ko, vo, ctx, theta)
    tail_k = torch.zeros((batch, n_new, hkv, d), dtype=TORCH_DT[dtype], device=DEV)
    tail_v = torch.zeros_like(tail_k)
    o_fused = dbsa.dbsa_query_attn_spans(q, kn, vn, kp, vp, src, ln, tail_k, tail_v, [0] * batch,
                                         theta)
    torch.cuda.synchronize()
    for b in range(batch):
        kg, vg = orc.gather_rope_spans(host64(kp), host64(vp), src[b], ln[b], theta)
        assert ctx[b] == kg.shape[0]
        np.testing.assert_array_equal(host64(vo[b, :ctx[b]]), vg)
        if dtype == "bf16":
            assert_bf16_rounding(host64(ko[b, :ctx[b]]), kg, f"span gather K row {b}")
        else:
            assert_close(host64(ko[b, :ctx[b]]), kg, "f32", f"span gather K row {b}")
        want, _, _ = orc.query_attn(host64(q[b]), host64(kn[b]), host64(vn[b]), kg, vg, theta)
        assert_close(host64(o_mat[b]), want, dtype, f"span query b={b} materialised")
        assert_close(host64(o_fused[b]), want, dtype, f"span query b={b} fused")
    return o_mat, o_fused


def _demo_spans(rng, n_pool, anchor, rows, n_demos, lo, hi):
    """Anchor span first, then demonstrations at arbitrary pool offsets (not
    block-aligned); some rows get fewer demos (zero-length padding), one pair
    of demos is back to back."""
    src = np.zeros((rows, n_demos + 1), np.int32)
    ln = np.zeros((rows, n_demos + 1), np.int32)
    for r in range(rows):
        src[r, 0], ln[r, 0] = 0, anchor
        k = n_demos - (r % 3)
        for i in range(1, k + 1):
            ln[r, i] = rng.integers(lo, hi)
            src[r, i] = rng.integers(anchor, n_pool - ln[r, i])
        if k >= 3:
            src[r, 3] = src[r, 2] + ln[r, 2]
            ln[r, 3] = min(ln[r, 3], n_pool - src[r, 3])
    return src, ln


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_example_level_spans(dtype):
    rng = np.random.default_rng(37)
    n_pool = 4000
    src, ln = _demo_spans(rng, n_pool, 57, 3, 9, 5, 120)
    hq, hkv, d = (8, 2, 128) if dtype == "bf16" else (2, 1, 64)
    o_mat, o_fused = _span_case(dtype, hq, hkv, d, n_pool, src, ln, 13, 1e4, 171)
    if dtype == "bf16":
        assert torch.equal(o_mat, o_fused)


def test_example_level_many_short_spans():
    """Hundreds of one- to three-token spans per row: many segments per tile,
    a segment change inside almost every key tile."""
    rng = np.random.default_rng(41)
    n_pool = 3000
    n = 700
    src = np.stack([np.sort(rng.choice(n_pool - 3, n, replace=False)) for _ in range(2)])
    ln = rng.integers(1, 4, size=(2, n))
    src, ln = src.astype(np.int32), ln.astype(np.int32)
    o_mat, o_fused = _span_case("bf16", 8, 2, 128, n_pool, src, ln, 6, 5e5, 181)
    assert torch.equal(o_mat, o_fused)


def test_spans_with_table_head_dim_64_and_decode():
    """Example-level spans combined with a RoPE frequency table (head_dim 64,
    bf16), then decode steps over the same spans with a growing tail buffer."""
    rng = np.random.default_rng(59)
    n_pool = 2500
    src, ln = _demo_spans(rng, n_pool, 40, 2, 7, 5, 90)
    table = llama31_inv_freq(5e5, 64)
    _span_case("bf16", 8, 2, 64, n_pool, src, ln, 9, table, 221)
    # query tokens then single-token steps, each appending to the tail
    hq, hkv, d, theta = 8, 2, 128, 5e5
    kp = randn((n_pool, hkv, d), 231, "bf16", DEV)
    vp = randn((n_pool, hkv, d), 232, "bf16", DEV)
    n_q, steps = 6, 3
    q = randn((1, n_q + steps, hq, d), 233, "bf16", DEV)
    kn = randn((1, n_q + steps, hkv, d), 234, "bf16", DEV)
    vn = randn((1, n_q + steps, hkv, d), 235, "bf16", DEV)
    tk = torch.zeros((1, n_q + steps, hkv, d), dtype=torch.bfloat16, device=DEV)
    tv = torch.zeros_like(tk)
    outs = [dbsa.dbsa_query_attn_spans(q[:, :n_q].contiguous(), kn[:, :n_q].contiguous(),
                                       vn[:, :n_q].contiguous(), kp, vp, src[:1], ln[:1], tk, tv,
                                       [0], theta)]
    for s_ in range(steps):
        sl = slice(n_q + s_, n_q + s_ + 1)
        outs.append(dbsa.dbsa_query_attn_spans(q[:, sl].contiguous(), kn[:, sl].contiguous(),
                                               vn[:, sl].contiguous(), kp, vp, src[:1], ln[:1],
                                               tk, tv, [n_q + s_], theta))
    torch.cuda.synchronize()
    kg, vg = orc.gather_rope_spans(host64(kp), host64(vp), src[0], ln[0], theta)
    want, _, _ = orc.query_attn(host64(q[0]), host64(kn[0]), host64(vn[0]), kg, vg, theta)
    got = np.concatenate([host64(o[0]) for o in outs])
    assert_close(got, want, "bf16", "span query + decode steps")

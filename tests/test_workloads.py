"""The seeded generator produces the workloads' stated shapes and structure."""
import math

import numpy as np
import pytest

import workloads as W


def _check_common(w):
    both = np.concatenate([w.fill_slots, w.new_slots])
    assert np.unique(both).size == both.size                      # no duplicate slots
    assert both.min() >= 0 and both.max() < w.num_blocks * w.block_size
    used = np.unique(both // w.block_size)
    assert not np.isin(w.unused_blocks, used).any()
    assert w.poison_block in set(w.unused_blocks.tolist())
    # padding entries of every table point at the poison block
    for s in range(w.num_seqs):
        nb = math.ceil(int(w.context_lens[s]) / w.block_size)
        assert np.all(w.block_tables[s, nb:] == w.poison_block)
    # near-zero waste: each sequence wastes less than one block
    for s in range(w.num_seqs):
        n = int(w.context_lens[s])
        assert math.ceil(n / w.block_size) * w.block_size - n < w.block_size


def test_tiny_decode_structure():
    w = W.make(1)
    assert w.context_lens.tolist() == [1, 17, 64, 200]
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks) == (4, 2, 64, 16, 64)
    assert w.block_tables.shape == (4, 13) and w.scale == np.float32(0.125)
    assert w.unused_blocks.size == 64 - 20 and w.new_slots.size == 4
    _check_common(w)
    # the 20 used blocks are the first 20 entries of one seeded permutation of 64
    perm = np.random.default_rng(np.random.SeedSequence([1001, 1])).permutation(64)
    used = [int(b) for s in range(4) for b in w.block_tables[s, :math.ceil(w.context_lens[s] / 16)]]
    assert used == perm[:20].tolist()


def test_qwen3_06b_shapes():
    w = W.make(2)
    assert w.num_seqs == 256 and (w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size) == (16, 8, 128, 256)
    assert w.context_lens.min() >= 100 and w.context_lens.max() <= 1024
    assert w.new_slots.size == 256 and w.fill_slots.size == int(w.context_lens.sum()) - 256
    _check_common(w)


def test_qwen3_8b_shared_prefix():
    w = W.make(3)
    assert w.num_seqs == 1024 and w.num_q_heads == 32
    assert w.context_lens.min() >= 100 and w.context_lens.max() <= 2048
    sharers = np.flatnonzero((w.block_tables[:, :2] == w.shared_blocks).all(axis=1))
    assert sharers.size == 307 and np.all(w.context_lens[sharers] >= 513)
    _check_common(w)


def test_mixed_chunked_prefill():
    w = W.make(4)
    assert w.cu_seqlens_q.tolist() == list(range(0, 4097, 512))
    assert np.diff(w.cu_seqlens_k).tolist() == [256 * i + 512 for i in range(8)]
    assert w.num_seqs == 248 and w.new_slots.size == 8 * 512 + 248
    assert w.pq.shape == (4096, 32, 128)
    _check_common(w)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5e-39, 3.0e38], np.float32)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> 1 + 2^-6 (even)
    assert W.f32_to_bf16_bits(x)[:3].tolist() == [0x3F80, 0x3F80, 0x3F82]


def test_draws_do_not_depend_on_chunking():
    a = W.bf16_normal(5, 3, (3, 1000), chunk=1 << 22)
    b = W.bf16_normal(5, 3, (3, 1000), chunk=1 << 22)
    assert np.array_equal(a, b)


def test_norm_inputs_seeded_and_shaped():
    x, r, w = W.norm_inputs(5, 3, 128)
    x2, r2, w2 = W.norm_inputs(5, 3, 128)
    assert x.shape == r.shape == (3, 128) and w.shape == (128,)
    assert x.dtype == r.dtype == w.dtype == np.uint16
    assert np.array_equal(x, x2) and np.array_equal(r, r2) and np.array_equal(w, w2)
    assert not np.array_equal(x, W.norm_inputs(6, 3, 128)[0])


def _golden():
    import os
    vals = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "page_workload_values.txt")
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = (x.strip() for x in line.split("=", 1))
            vals[k] = [int(t) for t in v.split()]
    return vals


def test_workload_shapes_follow_the_pages():
    """Sequence counts, length ranges and block sizes printed on the pages
    (tests/golden/page_workload_values.txt, each value with its citation)."""
    g = _golden()
    w2 = W.make(2)
    assert w2.num_seqs == g["qwen3_06b_num_seqs"][0]
    assert g["qwen3_06b_len_lo"][0] <= w2.context_lens.min() and w2.context_lens.max() <= g["qwen3_06b_len_hi"][0]
    w3 = W.make(3)
    assert w3.num_seqs == g["qwen3_8b_num_seqs"][0]
    # a decode step's context is an input of 100-1024 tokens plus up to 1024 generated
    lo, hi = g["qwen3_8b_len_lo"][0], g["qwen3_8b_len_hi"][0]
    assert lo <= w3.context_lens.min() and w3.context_lens.max() <= 2 * hi
    for n in (2, 3, 4, 5, 6):
        assert W.make(n).block_size == g["block_size"][0]
    assert set(g["block_size_alternatives"]) <= {16, 32, 64, 128, 256}   # all supported

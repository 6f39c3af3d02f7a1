"""The algorithmic work that bench.py divides by time: prefill flops, decode
bytes and store bytes, checked against closed forms of their definitions
(4*D*Hq flops per unmasked (query, key) pair; K+V bytes of each valid token of
each unique (block, KV head), plus q, out, table entries and lengths)."""
import numpy as np

import bench
import workloads as W


def test_mixed_step_prefill_flops_closed_form():
    # 8 chunks of 512 new tokens on cached prefixes 256*i: query j of chunk i
    # (bottom-right causal) sees 256*i + j + 1 keys
    w = W.make(4)
    pairs = sum(512 * 256 * i + 512 * 513 // 2 for i in range(8))
    flops, nbytes = bench.prefill_work(w)
    assert pairs == 4_720_640
    assert flops == 4 * w.head_dim * w.num_q_heads * pairs == 77_342_965_760
    assert nbytes > 0


def test_decode_bytes_private_and_shared_blocks():
    w = W.custom(seed=5, Hq=4, Hkv=2, D=64, bs=16, context_lens=(1, 17, 40))
    row = w.num_kv_heads * w.head_dim * 2 * 2            # K+V of one token, all KV heads (bf16)
    tokens = 1 + 17 + 40
    entries = 1 + 2 + 3                                   # ceil(n / 16) table entries read
    extra = 2 * 3 * w.num_q_heads * w.head_dim * 2 + 4 * entries + 4 * 3
    total, logical, kv = bench.decode_bytes(w)
    assert kv == tokens * row
    assert total == logical == tokens * row + extra

    # two sequences sharing their first two blocks: the shared tokens count once
    # in the unique figure and once per reader in the logical one
    ws = W.custom(seed=6, Hq=4, Hkv=2, D=64, bs=16, context_lens=(40, 50), sharers=(0, 1),
                  shared_prefix_blocks=2)
    assert np.array_equal(ws.block_tables[0, :2], ws.block_tables[1, :2])
    total, logical, kv = bench.decode_bytes(ws)
    assert kv == (40 + 50 - 32) * row
    assert logical - total == 32 * row


def test_decode_bytes_fp8_and_store_bytes():
    w = W.custom(seed=7, Hq=8, Hkv=2, D=128, bs=32, context_lens=(33, 64), kv_dtype="fp8")
    row = w.num_kv_heads * w.head_dim * 1 * 2
    extra = 2 * 2 * w.num_q_heads * w.head_dim * 2 + 4 * (2 + 2) + 4 * 2 + 2 * 4 * w.num_kv_heads
    assert bench.decode_bytes(w)[0] == (33 + 64) * row + extra
    T = w.new_slots.size
    # bf16 k, v read; fp8 codes written; one int32 slot per token
    assert bench.store_bytes(w) == T * w.num_kv_heads * w.head_dim * (2 * 2 + 2 * 1) + 4 * T


def test_profile_figures_follow_the_kernel_sources(tmp_path):
    """Counter figures are read only while the kernel sources they were taken on
    are unchanged (the hash line of the summary matches)."""
    p = tmp_path / "summary.md"
    p.write_text("text\n"
                 f"sources_sha256 decode: {bench.sources_sha256('decode')}\n"
                 "traffic_bytes_per_launch w3/decode: 3900000000\n"
                 "sources_sha256 prefill: 0000\n"
                 "traffic_bytes_per_launch w4/prefill: 113000000\n")
    assert bench.profile_figure(str(p), "traffic_bytes_per_launch", 3, "decode") == 3.9e9
    assert bench.profile_figure(str(p), "traffic_bytes_per_launch", 2, "decode") is None
    assert bench.profile_figure(str(p), "traffic_bytes_per_launch", 4, "prefill") is None
    assert bench.profile_figure(str(tmp_path / "missing.md"), "traffic_bytes_per_launch", 3, "decode") is None
    # pa_store_decode runs the decode kernel and then the store kernel
    assert bench.sources_sha256("decode") != bench.sources_sha256("store_decode")
    assert bench.sources_sha256("decode") != bench.sources_sha256("prefill")

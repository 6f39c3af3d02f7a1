"""GPU parity of pa_prefill_varlen (causal varlen chunked prefill over the paged
cache, MFMA) against the CPU oracle, plus invariants. Tolerance: element-wise
|gpu - oracle| <= 1e-2 + 1e-2*|oracle| for a bf16 cache, 3e-2 for an fp8 cache
(the oracle reads the same fp8 bytes; float32 accumulation on the GPU)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import GpuCase, dev_bf16, dev_i32, host_bits
from tests.util import assert_close, bf16_f64, oracle_pools, relabel_blocks

pytestmark = pytest.mark.gpu

TOL = (1e-2, 1e-2)
TOL_FP8 = (3e-2, 3e-2)


def _oracle_prefill(w, kc, vc, seqs=None):
    return oracle.attention.prefill(w.pq, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k, w.p_block_tables,
                                    w.scale, w.block_size, w.k_scale, w.v_scale, seqs=seqs)


CASES = [
    dict(seed=301, Hq=4, Hkv=1, D=128, bs=16, prefill=[(0, 1), (0, 17), (0, 64), (0, 65), (16, 16)]),
    dict(seed=302, Hq=8, Hkv=2, D=128, bs=64, prefill=[(100, 30), (37, 200), (0, 300), (256, 64)]),
    dict(seed=303, Hq=32, Hkv=8, D=128, bs=256, prefill=[(0, 512), (768, 512), (1000, 77)]),
    dict(seed=304, Hq=16, Hkv=8, D=64, bs=32, prefill=[(5, 250), (0, 129), (300, 1)]),
    dict(seed=305, Hq=8, Hkv=1, D=64, bs=128, prefill=[(0, 40), (200, 33), (64, 70)]),
    dict(seed=306, Hq=2, Hkv=2, D=128, bs=16, prefill=[(0, 300), (513, 260)]),
]


@pytest.mark.parametrize("cfg", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_prefill_small(cfg):
    print(f"case {cfg}", flush=True)
    w = W.custom(context_lens=(), **cfg)
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    got = bf16_f64(host_bits(case.prefill()))
    ma, mr = assert_close(got, _oracle_prefill(w, kc, vc), *TOL, what="prefill")
    print(f"max_abs={ma:.3e} max_rel={mr:.3e}")


def test_prefill_equal_lengths_and_many_sequences():
    """Workgroups take sequences longest first, ties by index: equal-length
    sequences each get their own workgroups; past the ranked limit (256
    sequences) they are taken by index. Every row against the oracle."""
    rng = np.random.default_rng(330)
    for pf in ([(40, 24)] * 5 + [(0, 64)] * 3 + [(64, 1)],
               [(int(rng.integers(0, 40)), int(rng.integers(1, 9))) for _ in range(300)],
               # the ranked limit exactly, and one past it: each sequence's query
               # offset and length come from the ranking pass, or from global memory
               [(int(rng.integers(0, 30)), int(rng.integers(1, 6))) for _ in range(256)],
               [(int(rng.integers(0, 30)), int(rng.integers(1, 6))) for _ in range(257)]):
        w = W.custom(seed=331, Hq=4, Hkv=2, D=64, bs=16, context_lens=(), prefill=pf)
        print(f"{len(pf)} sequences", flush=True)
        case = GpuCase(w)
        kc, vc = oracle_pools(w)
        got = bf16_f64(host_bits(case.prefill()))
        assert_close(got, _oracle_prefill(w, kc, vc), *TOL, what=f"{len(pf)} sequences")



@pytest.mark.parametrize("kv,bs", [("bf16", 16), ("bf16", 256), ("fp8", 64)])
def test_prefill_rows_without_keys(kv, bs):
    """Fewer keys than queries: query i sits at position Lk-Lq+i, so the first
    Lq-Lk rows see no key and are zeros, next to rows of the same workgroup that
    do see keys (the running-max rescale must leave a column with no key yet
    untouched); a sequence with no keys at all gives zero rows."""
    w = W.custom(seed=349, Hq=8, Hkv=2, D=128, bs=bs, context_lens=(), kv_dtype=kv,
                 prefill=[(0, 100), (0, 70), (40, 90), (0, 5), (10, 300)])
    lk = np.diff(w.cu_seqlens_k).astype(np.int64)
    lk[0], lk[1], lk[3] = 60, 0, 2
    w.cu_seqlens_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    print(f"{kv} block {bs}: keys per sequence {lk.tolist()}", flush=True)
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    got = bf16_f64(host_bits(case.prefill()))
    assert_close(got, _oracle_prefill(w, kc, vc), *(TOL_FP8 if kv == "fp8" else TOL), what="prefill")
    q0, q1 = int(w.cu_seqlens_q[1]), int(w.cu_seqlens_q[2])
    assert not np.any(got[q0:q1]) and not np.any(got[:40]) and not np.any(got[260:263])

FP8_CASES = [
    dict(seed=321, Hq=4, Hkv=1, D=128, bs=16, prefill=[(0, 1), (0, 17), (0, 64), (0, 65), (16, 16)]),
    dict(seed=322, Hq=8, Hkv=2, D=128, bs=64, prefill=[(100, 30), (37, 200), (0, 300)]),
    dict(seed=323, Hq=16, Hkv=8, D=64, bs=32, prefill=[(5, 250), (0, 129), (300, 1)]),
    dict(seed=324, Hq=8, Hkv=1, D=64, bs=256, prefill=[(0, 40), (700, 33), (64, 270)]),
]


@pytest.mark.parametrize("cfg", FP8_CASES, ids=[f"fp8case{i}" for i in range(len(FP8_CASES))])
def test_prefill_fp8_small(cfg):
    """fp8 (E4M3) cache with per-head scales: every row against the oracle on the same bytes."""
    print(f"fp8 case {cfg}", flush=True)
    w = W.custom(context_lens=(), kv_dtype="fp8", **cfg)
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    got = bf16_f64(host_bits(case.prefill()))
    ma, mr = assert_close(got, _oracle_prefill(w, kc, vc), *TOL_FP8, what="fp8 prefill")
    print(f"max_abs={ma:.3e} max_rel={mr:.3e}")


def test_prefill_fp8_matches_fp8_decode():
    """A one-row prefill over an fp8 cache equals the fp8 decode of the same rows to
    bf16 rounding (both widen the same bytes exactly and fold the same scales)."""
    w = W.custom(seed=325, Hq=16, Hkv=4, D=128, bs=64, context_lens=(1, 100, 700), kv_dtype="fp8")
    case = GpuCase(w)
    dec = bf16_f64(host_bits(case.decode()))
    import paged_kv_cache_store_amd as pa
    S = w.num_seqs
    cu_k = np.concatenate([[0], np.cumsum(w.context_lens)])
    pre = pa.prefill_varlen(case.q, case.k_cache, case.v_cache, dev_i32(np.arange(S + 1)), dev_i32(cu_k),
                            case.block_tables, float(w.scale), 1, int(w.context_lens.max()),
                            k_scale=case.k_scale, v_scale=case.v_scale)
    np.testing.assert_allclose(bf16_f64(host_bits(pre)), dec, rtol=2 ** -7, atol=2e-3)


def test_prefill_long_context_small_blocks():
    """33000 cached keys in 16-token blocks: the workgroup reads more blocks than
    its in-LDS window of block ids holds, so the window moves during the loop."""
    for kv in ("bf16", "fp8"):
        w = W.custom(seed=330, Hq=4, Hkv=1, D=64, bs=16, context_lens=(), prefill=[(33000, 8), (40, 24)],
                     kv_dtype=kv)
        case = GpuCase(w)
        kc, vc = oracle_pools(w)
        got = bf16_f64(host_bits(case.prefill()))
        ma, mr = assert_close(got, _oracle_prefill(w, kc, vc), *(TOL if kv == "bf16" else TOL_FP8),
                              what=f"long small-block prefill {kv}")
        print(f"[{kv}] max_abs={ma:.3e} max_rel={mr:.3e}")


def _score_ramp(w, kind, R=12.0, seed=0):
    """Rewrite the prefill queries and keys so that the scores of a sequence follow
    `kind` along the key positions: q = u + noise for the G query heads of a KV
    head, k(p) = r(p) u + noise with u in {-1, +1}^D, so that score(p) is about
    r(p) sqrt(D) (natural log units) and varies by up to R sqrt(D) log2(e) bits:
    rise (the maximum keeps moving up), fall (the first keys dominate) or spikes
    (1 % of the keys at R)."""
    rng = np.random.default_rng(seed)
    Hkv, G, D = w.num_kv_heads, w.num_q_heads // w.num_kv_heads, w.head_dim
    u = rng.choice([-1.0, 1.0], size=(Hkv, D))
    tq = w.pq.shape[0]
    q = np.repeat(u, G, axis=0)[None] + 0.25 * rng.standard_normal((tq, w.num_q_heads, D))
    w.pq = W.f32_to_bf16_bits(q.astype(np.float32))
    fk = W.bf16_bits_to_f32(w.fill_k).astype(np.float64)
    nk = W.bf16_bits_to_f32(w.new_k).astype(np.float64)
    fo = no = 0
    for i in range(w.cu_seqlens_q.size - 1):
        chunk = int(w.cu_seqlens_q[i + 1] - w.cu_seqlens_q[i])
        L = int(w.cu_seqlens_k[i + 1] - w.cu_seqlens_k[i])
        prefix = L - chunk
        pos = np.arange(L, dtype=np.float64)
        if kind == "rise":
            r = R * pos / max(L - 1, 1)
        elif kind == "fall":
            r = R * (1.0 - pos / max(L - 1, 1))
        else:
            r = np.where(rng.random(L) < 0.01, R, 0.0)
        kk = r[:, None, None] * u[None] + 0.25 * rng.standard_normal((L, Hkv, D))
        fk[fo:fo + prefix] = kk[:prefix]
        nk[no:no + chunk] = kk[prefix:]
        fo += prefix
        no += chunk
    w.fill_k = W.f32_to_bf16_bits(fk.astype(np.float32))
    w.new_k = W.f32_to_bf16_bits(nk.astype(np.float32))
    if w.kv_dtype == "fp8":
        w.k_scale = W._amax_scale(w.fill_k, w.new_k)
    return w


@pytest.mark.parametrize("kind", ["rise", "fall", "spikes"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_wide_score_range(kind, kv):
    """Scores spread over ~160 bits along a sequence: the softmax reference has to
    follow the maximum (exp2 of the raw offsets would overflow fp32), and keys far
    below it must not disturb the result."""
    print(f"score ramp {kind} {kv}", flush=True)
    for cfg in (dict(seed=341, Hq=32, Hkv=8, D=128, bs=256, prefill=[(700, 300), (0, 512), (1500, 40)]),
                dict(seed=342, Hq=4, Hkv=2, D=64, bs=16, prefill=[(200, 130), (0, 77)])):
        w = _score_ramp(W.custom(context_lens=(), kv_dtype=kv, **cfg), kind, seed=cfg["seed"])
        case = GpuCase(w)
        kc, vc = oracle_pools(w)
        got = bf16_f64(host_bits(case.prefill()))
        assert np.isfinite(got).all()
        ma, mr = assert_close(got, _oracle_prefill(w, kc, vc), *(TOL if kv == "bf16" else TOL_FP8),
                              what=f"prefill, scores {kind}, {kv}")
        print(f"[D{w.head_dim} {kind} {kv}] max_abs={ma:.3e} max_rel={mr:.3e}")


def test_mixed_chunked_prefill_workload():
    """Full mixed step: store of 4344 tokens, prefill of the 8 chunks (all rows checked),
    decode of the 248 sequences (all checked)."""
    w = W.make(4)
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    pre = bf16_f64(host_bits(case.prefill()))
    ma, mr = assert_close(pre, _oracle_prefill(w, kc, vc), *TOL, what="mixed prefill")
    print(f"[mixed prefill] max_abs={ma:.3e} max_rel={mr:.3e}")
    dec = bf16_f64(host_bits(case.decode()))
    ref = oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.block_size)
    ma, mr = assert_close(dec, ref, *TOL, what="mixed decode")
    print(f"[mixed decode] max_abs={ma:.3e} max_rel={mr:.3e}")
    assert np.array_equal(host_bits(case.k_cache), kc) and np.array_equal(host_bits(case.v_cache), vc)


def test_mixed_chunked_prefill_fp8_workload():
    """The same mixed step over an fp8 cache: all prefill rows, all 248 decode rows,
    every pool byte."""
    w = W.make(6)
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    pre = bf16_f64(host_bits(case.prefill()))
    ma, mr = assert_close(pre, _oracle_prefill(w, kc, vc), *TOL_FP8, what="fp8 mixed prefill")
    print(f"[fp8 mixed prefill] max_abs={ma:.3e} max_rel={mr:.3e}")
    dec = bf16_f64(host_bits(case.decode()))
    ref = oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.block_size,
                                  w.k_scale, w.v_scale)
    ma, mr = assert_close(dec, ref, *TOL_FP8, what="fp8 mixed decode")
    print(f"[fp8 mixed decode, {w.num_seqs} sequences] max_abs={ma:.3e} max_rel={mr:.3e}")
    assert np.array_equal(host_bits(case.k_cache), kc) and np.array_equal(host_bits(case.v_cache), vc)


def test_chunk_equals_tail_of_full_prefill_bit_identical():
    """Prefill of a 96-token chunk on a 160-token cached prefix gives the last 96 rows of
    the prefill of all 256 tokens (same per-row arithmetic)."""
    p, c = 160, 96
    w = W.custom(seed=310, Hq=8, Hkv=2, D=128, bs=64, context_lens=(), prefill=[(p, c)])
    case = GpuCase(w)
    chunk = host_bits(case.prefill())
    rng = np.random.default_rng(1)
    qfull = np.concatenate([W.f32_to_bf16_bits(rng.standard_normal((p, 8, 128)).astype(np.float32)), w.pq])
    import paged_kv_cache_store_amd as pa
    full = pa.prefill_varlen(dev_bf16(qfull), case.k_cache, case.v_cache, dev_i32([0, p + c]),
                             dev_i32([0, p + c]), case.p_block_tables, float(w.scale), p + c, p + c)
    assert np.array_equal(host_bits(full)[p:], chunk)


def test_prefill_block_permutation_bit_identical():
    w = W.custom(seed=311, Hq=8, Hkv=2, D=128, bs=32, context_lens=(), prefill=[(70, 100), (0, 33)])
    a = host_bits(GpuCase(w).prefill())
    b = host_bits(GpuCase(relabel_blocks(w, seed=2)).prefill())
    assert np.array_equal(a, b)


def test_decode_matches_one_row_prefill():
    w = W.custom(seed=312, Hq=16, Hkv=4, D=128, bs=64, context_lens=(1, 100, 700))
    case = GpuCase(w)
    dec = bf16_f64(host_bits(case.decode()))
    import paged_kv_cache_store_amd as pa
    S = w.num_seqs
    cu_k = np.concatenate([[0], np.cumsum(w.context_lens)])
    pre = pa.prefill_varlen(case.q, case.k_cache, case.v_cache, dev_i32(np.arange(S + 1)), dev_i32(cu_k),
                            case.block_tables, float(w.scale), 1, int(w.context_lens.max()))
    np.testing.assert_allclose(bf16_f64(host_bits(pre)), dec, rtol=2 ** -7, atol=2e-3)


def test_prefill_guard_bands_and_determinism():
    w = W.custom(seed=313, Hq=8, Hkv=2, D=64, bs=16, context_lens=(), prefill=[(20, 45)])
    case = GpuCase(w)
    Tq, Hq, D = w.pq.shape
    buf = torch.full((Tq + 2, Hq, D), -7.0, dtype=torch.bfloat16, device="cuda")
    case.prefill(out=buf[1:Tq + 1])
    first = host_bits(buf)
    case.prefill(out=buf[1:Tq + 1])
    assert np.array_equal(first, host_bits(buf))
    sentinel = host_bits(torch.full((Hq, D), -7.0, dtype=torch.bfloat16))
    assert np.array_equal(first[0], sentinel) and np.array_equal(first[Tq + 1], sentinel)


# ---------------------------------------------------------------- packed keys/values (no block table)
PACKED = [
    dict(seed=340, Hq=4, Hkv=1, D=128, bs=16, prefill=[(0, 1), (0, 17), (0, 64), (0, 65), (16, 16)]),
    dict(seed=341, Hq=8, Hkv=2, D=128, bs=64, prefill=[(100, 30), (37, 200), (0, 300), (256, 64)]),
    dict(seed=342, Hq=32, Hkv=8, D=128, bs=256, prefill=[(0, 512), (768, 512), (1000, 77)]),
    dict(seed=343, Hq=16, Hkv=8, D=64, bs=32, prefill=[(5, 250), (0, 129), (300, 1)]),
    dict(seed=344, Hq=8, Hkv=1, D=64, bs=128, prefill=[(0, 40), (200, 33), (64, 70)]),
]


def _packed_kv(w):
    """Each sequence's Lk keys/values in logical order, sequences one after the
    other ([Tk, Hkv, D] bf16 bits), taken from the generator's token lists."""
    from tests.util import logical_kv, slot_index
    idx = slot_index(w)
    ks, vs = [], []
    for s in range(len(w.cu_seqlens_k) - 1):
        lk = int(w.cu_seqlens_k[s + 1] - w.cu_seqlens_k[s])
        K, V = logical_kv(w, w.p_block_tables[s], lk, idx)
        ks.append(K)
        vs.append(V)
    return np.concatenate(ks), np.concatenate(vs)


def _identity_pool(w, K, V):
    """Oracle pool holding the packed keys with sequence s in consecutive blocks
    from block first[s] (an identity block table per sequence)."""
    bs = w.block_size
    S = len(w.cu_seqlens_k) - 1
    lens = np.diff(w.cu_seqlens_k)
    nblk = -(-lens // bs)
    first = np.concatenate([[0], np.cumsum(nblk)])
    ks, vs = oracle.cache.pool_shapes(int(first[-1]) + 1, w.num_kv_heads, bs, w.head_dim)
    kc = np.full(ks, W.BF16_NAN, np.uint16)
    vc = np.full(vs, W.BF16_NAN, np.uint16)
    slots = np.concatenate([first[s] * bs + np.arange(lens[s]) for s in range(S)]).astype(np.int32)
    oracle.cache.store(K, V, slots, kc, vc, bs)
    table = np.zeros((S, max(1, int(nblk.max()))), np.int32)
    for s in range(S):
        table[s, :nblk[s]] = first[s] + np.arange(nblk[s])
    return kc, vc, table


@pytest.mark.parametrize("cfg", PACKED, ids=[f"packed{i}" for i in range(len(PACKED))])
def test_prefill_packed_kv(cfg):
    """block_tables = NULL: keys/values packed [Tk, Hkv, D] by cu_seqlens_k.
    Every row against the oracle (fed the same keys through an identity-table
    pool), and bit-identical to the paged call over the same keys."""
    import paged_kv_cache_store_amd as pa
    print(f"case {cfg}", flush=True)
    w = W.custom(context_lens=(), **cfg)
    K, V = _packed_kv(w)
    kd, vd = dev_bf16(K), dev_bf16(V)
    q = dev_bf16(w.pq)
    cu_q, cu_k = dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k)
    got = pa.prefill_varlen(q, kd, vd, cu_q, cu_k, None, float(w.scale), w.max_seqlen_q, w.max_seqlen_k)
    torch.cuda.synchronize()
    kc, vc, table = _identity_pool(w, K, V)
    ref = oracle.attention.prefill(w.pq, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k, table, w.scale,
                                   w.block_size)
    ma, mr = assert_close(bf16_f64(host_bits(got)), ref, *TOL, what="packed prefill")
    print(f"max_abs={ma:.3e} max_rel={mr:.3e}")
    paged = GpuCase(w).prefill()
    assert np.array_equal(host_bits(got), host_bits(paged))


def test_prefill_packed_mixed_step_shapes():
    """The mixed step's 8 chunks (512 new tokens on prefixes 0..1792, 32/8
    heads, D 128) with packed keys/values: every row against the oracle."""
    import paged_kv_cache_store_amd as pa
    w = W.make(4)
    K, V = _packed_kv(w)
    got = pa.prefill_varlen(dev_bf16(w.pq), dev_bf16(K), dev_bf16(V), dev_i32(w.cu_seqlens_q),
                            dev_i32(w.cu_seqlens_k), None, float(w.scale), w.max_seqlen_q, w.max_seqlen_k)
    torch.cuda.synchronize()
    kc, vc, table = _identity_pool(w, K, V)
    ref = oracle.attention.prefill(w.pq, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k, table, w.scale,
                                   w.block_size)
    ma, mr = assert_close(bf16_f64(host_bits(got)), ref, *TOL, what="packed mixed-step prefill")
    print(f"[packed mixed prefill] max_abs={ma:.3e} max_rel={mr:.3e}")

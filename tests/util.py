"""Helpers shared by the tests (no attention arithmetic here)."""
import math

import numpy as np

import workloads as W


def slot_index(w):
    """dict slot -> (which list, row) over the workload's cached and new tokens."""
    idx = {}
    for i, s in enumerate(w.fill_slots.tolist()):
        idx[s] = ("fill", i)
    for i, s in enumerate(w.new_slots.tolist()):
        if s >= 0:
            idx[s] = ("new", i)
    return idx


def logical_kv(w, table_row, length, idx=None):
    """bf16 bit patterns [length, Hkv, D] of K and V at logical positions 0..length-1,
    looked up by slot in the generator's token lists (independent of oracle.cache)."""
    idx = idx if idx is not None else slot_index(w)
    bs = w.block_size
    K = np.empty((length, w.num_kv_heads, w.head_dim), np.uint16)
    V = np.empty_like(K)
    for j in range(length):
        which, r = idx[int(table_row[j // bs]) * bs + j % bs]
        K[j] = (w.fill_k if which == "fill" else w.new_k)[r]
        V[j] = (w.fill_v if which == "fill" else w.new_v)[r]
    return K, V


def bf16_f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def close_report(got, ref, atol, rtol):
    """Element-wise |got-ref| <= atol + rtol*|ref|; returns (ok, max_abs, max_rel>=1e-3)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    ok = bool(np.all(err <= atol + rtol * np.abs(ref))) and not np.isnan(got).any()
    big = np.abs(ref) >= 1e-3
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    return ok, float(err.max()) if err.size else 0.0, max_rel


def assert_close(got, ref, atol, rtol, what=""):
    ok, ma, mr = close_report(got, ref, atol, rtol)
    assert ok, f"{what}: max_abs={ma:.3e} max_rel={mr:.3e} (atol={atol}, rtol={rtol})"
    return ma, mr


def poisoned_pools(w, kv_dtype=None):
    """Oracle pools filled with NaN patterns (bf16 0x7FC0 / fp8 0x7F)."""
    import oracle
    kv_dtype = kv_dtype or w.kv_dtype
    ks, vs = oracle.cache.pool_shapes(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, kv_dtype)
    if kv_dtype == "fp8":
        return np.full(ks, W.FP8_NAN, np.uint8), np.full(vs, W.FP8_NAN, np.uint8)
    return np.full(ks, W.BF16_NAN, np.uint16), np.full(vs, W.BF16_NAN, np.uint16)


def oracle_pools(w):
    """Oracle pools after writing every cached and new token of the workload."""
    import oracle
    kc, vc = poisoned_pools(w)
    oracle.cache.store(w.fill_k, w.fill_v, w.fill_slots, kc, vc, w.block_size, w.k_scale, w.v_scale)
    oracle.cache.store(w.new_k, w.new_v, w.new_slots, kc, vc, w.block_size, w.k_scale, w.v_scale)
    return kc, vc


def relabel_blocks(w, seed=0):
    """Same workload with physical block ids renamed by a random permutation."""
    import copy
    rng = np.random.default_rng(seed)
    pi = rng.permutation(w.num_blocks).astype(np.int64)
    bs = w.block_size
    w2 = copy.copy(w)

    def rs(sl):
        sl = np.asarray(sl, np.int64)
        return np.where(sl >= 0, pi[np.maximum(sl, 0) // bs] * bs + np.maximum(sl, 0) % bs, sl).astype(np.int32)

    w2.fill_slots = rs(w.fill_slots)
    w2.new_slots = rs(w.new_slots)
    w2.block_tables = pi[w.block_tables].astype(np.int32)
    if w.p_block_tables is not None:
        w2.p_block_tables = pi[w.p_block_tables].astype(np.int32)
    w2.poison_block = int(pi[w.poison_block])
    w2.unused_blocks = np.sort(pi[w.unused_blocks]).astype(np.int32)
    return w2


def oracle_decode_threads(w, kc, vc, seqs=None):
    """oracle.attention.decode of the given sequences (default: all), the
    sequences split over host threads; each call fills only its own rows, so
    the sum of the partial results is the oracle's result."""
    import concurrent.futures
    import os

    import oracle
    seqs = list(range(w.num_seqs)) if seqs is None else list(seqs)
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(seqs)))
    # longest sequences first, dealt round-robin so the threads get equal work
    order = sorted(seqs, key=lambda s: -int(w.context_lens[s]))
    parts = [order[i::workers] for i in range(workers)]

    def run(part):
        return oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                       w.block_size, w.k_scale, w.v_scale, seqs=part)

    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(run, [p for p in parts if p]))
    return np.sum(outs, axis=0)

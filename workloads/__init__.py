"""Seeded synthetic inputs for the paged KV-cache path.

This module only draws numbers and lays out tables: context lengths, the
physical block assignment (a seeded permutation of the pool), block tables,
slot numbers of the tokens to be written, and bf16 query/key/value draws.
It holds none of the attention or quantisation arithmetic; both the CPU
oracle (``oracle/``) and the HIP path consume what it returns.

The five workloads are the attention shapes of the pages' benchmark runs
(Qwen3-0.6B with 256 sequences, Qwen3-8B with 1024 sequences, input/output
lengths drawn from 100 to 1024 tokens — "DeepSeek复刻vLLM反超原版：AI推理新标杆",
section 性能对决; chunked prefill mixed with decode — "nano-vllm-lite：深入理解
LLM推理机制的教育级开源项目", 核心技术改进 §2; FP8 KV cache — same page, §3).

Recipe (each reading of the pages it rests on is stated where it is used):
* seed = 1000 + workload number; independent sub-streams
  ``default_rng(SeedSequence([seed, k]))`` with k = 0 lengths, 1 block
  permutation, 5 choice of prefix sharers; value draws use
  ``SeedSequence([seed, k, c])`` for chunk c of 2**22 values with k = 2
  decode queries, 102 prefill queries, 3 cached keys, 4 cached values,
  6 new keys, 7 new values;
* "uniform in [a, b]" = integers, both ends included;
* bf16 ~ N(0,1) = float32 standard-normal draws rounded to nearest-even bf16;
* the pool has ceil(1.25 x blocks needed) blocks; logical blocks, taken in
  (sequence, block) order, receive physical ids perm[0], perm[1], ...; the
  next unused id is the "poison" block that pads every block table;
* a decode sequence's context length counts its newest token, whose K/V is
  written by the step's store; every older position is "cached" and is
  written once during set-up.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)

_STREAM_LENGTHS, _STREAM_PERM, _STREAM_Q, _STREAM_K, _STREAM_V = 0, 1, 2, 3, 4
_STREAM_SHARERS, _STREAM_NEW_K, _STREAM_NEW_V = 5, 6, 7


def _rng(seed: int, k: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, k]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_normal(seed: int, stream: int, shape, chunk: int = 1 << 22) -> np.ndarray:
    """bf16 bit patterns of N(0,1) draws. Chunk c of the flattened array comes from
    its own sub-stream SeedSequence([seed, stream, c]), so chunks are drawn in
    parallel threads and the result does not depend on the thread count."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)

    def fill(c):
        lo, hi = c * chunk, min(n, (c + 1) * chunk)
        rng = np.random.default_rng(np.random.SeedSequence([seed, stream, c]))
        out[lo:hi] = f32_to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))

    nchunks = (n + chunk - 1) // chunk
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        workers = max(1, min(16, len(os.sched_getaffinity(0)), nchunks))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclasses.dataclass
class Workload:
    """One synthetic batch. Arrays are numpy; bf16 values are uint16 bit patterns."""
    name: str
    number: int
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str                      # "bf16" or "fp8"
    scale: np.float32                  # softmax scale (fp32)
    poison_block: int                  # unused block that pads block tables
    unused_blocks: np.ndarray          # int32, every block no table refers to
    # K/V already in the cache before the step (written during set-up)
    fill_slots: np.ndarray             # int32 [Tf]
    fill_k: np.ndarray                 # uint16 [Tf, Hkv, D]
    fill_v: np.ndarray
    # K/V written by the step's store (one per decode sequence, plus chunk tokens)
    new_slots: np.ndarray              # int32 [T]
    new_k: np.ndarray                  # uint16 [T, Hkv, D]
    new_v: np.ndarray
    # decode part
    q: np.ndarray                      # uint16 [S, Hq, D]
    block_tables: np.ndarray           # int32 [S, MB]
    context_lens: np.ndarray           # int32 [S]
    partition_size: int = 0            # 0 = library's choice
    # fp8 scales (per KV head), None for a bf16 cache
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    # prefill part (chunked prefill on a cached prefix); None when absent
    pq: Optional[np.ndarray] = None            # uint16 [Tq, Hq, D]
    cu_seqlens_q: Optional[np.ndarray] = None  # int32 [P+1]
    cu_seqlens_k: Optional[np.ndarray] = None  # int32 [P+1]
    p_block_tables: Optional[np.ndarray] = None  # int32 [P, MBp]
    shared_blocks: Optional[np.ndarray] = None   # physical ids shared by several tables

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def has_prefill(self) -> bool:
        return self.pq is not None

    @property
    def max_seqlen_q(self) -> int:
        return int(np.diff(self.cu_seqlens_q).max())

    @property
    def max_seqlen_k(self) -> int:
        return int(np.diff(self.cu_seqlens_k).max())


class _Pool:
    """Hands out physical block ids in the order of a seeded permutation."""

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.perm = rng.permutation(num_blocks).astype(np.int32)
        self.next = 0

    def take(self) -> int:
        b = int(self.perm[self.next])
        self.next += 1
        return b


def _build(number, name, *, seed, Hq, Hkv, D, bs, seqs, prefill=None, kv_dtype="bf16",
           num_blocks=None, sharers=(), shared_prefix_blocks=0, partition_size=0):
    """seqs: list of (context_len) for decode sequences.
    prefill: list of (prefix_len, chunk_len) for chunked-prefill sequences.
    sharers: indices into seqs whose first `shared_prefix_blocks` logical blocks
    point at one common run of physical blocks."""
    prefill = prefill or []
    sharers = set(int(s) for s in sharers)
    # tokens each sequence needs room for
    p_total = [p + c for (p, c) in prefill]
    all_lens = p_total + list(seqs)
    nblk = [math.ceil(n / bs) for n in all_lens]
    needed = sum(nblk) - max(0, len(sharers) - 1) * shared_prefix_blocks
    if num_blocks is None:
        num_blocks = math.ceil(1.25 * needed)
    assert num_blocks > needed, "pool must keep at least one unused block"
    pool = _Pool(num_blocks, _rng(seed, _STREAM_PERM))

    tables = []
    shared = None
    P = len(prefill)
    for i, n in enumerate(nblk):
        row = []
        is_sharer = (i - P) in sharers
        for j in range(n):
            if is_sharer and j < shared_prefix_blocks:
                if shared is None:
                    shared = [pool.take() for _ in range(shared_prefix_blocks)]
                row.append(shared[j])
            else:
                row.append(pool.take())
        tables.append(row)
    assert pool.next == needed
    poison = int(pool.perm[pool.next])
    unused = np.sort(pool.perm[pool.next:]).astype(np.int32)

    def slots(i, lo, hi):
        """slot numbers of logical positions lo..hi-1 of sequence i"""
        pos = np.arange(lo, hi, dtype=np.int64)
        return np.asarray(tables[i], dtype=np.int64)[pos // bs] * bs + pos % bs

    # cached positions (set-up) and new positions (the step), in sequence order
    fill, new = [], []
    shared_done = False
    for i in range(len(all_lens)):
        if i < P:
            prefix, chunk = prefill[i]
            fill.append(slots(i, 0, prefix))
            new.append(slots(i, prefix, prefix + chunk))
        else:
            ctx = all_lens[i]
            start = 0
            if (i - P) in sharers:
                if shared_done:
                    start = shared_prefix_blocks * bs
                shared_done = True
            fill.append(slots(i, start, max(start, ctx - 1)))
    for i in range(P, len(all_lens)):   # decode tokens after all chunk tokens
        if all_lens[i] > 0:
            new.append(slots(i, all_lens[i] - 1, all_lens[i]))
    fill = np.concatenate(fill) if fill else np.zeros(0, np.int64)
    new = np.concatenate(new) if new else np.zeros(0, np.int64)
    fill = fill.astype(np.int32)
    new = new.astype(np.int32)
    both = np.concatenate([fill, new])
    assert np.unique(both).size == both.size, "slot numbers must be distinct"
    assert both.size == 0 or (both.min() >= 0 and both.max() < num_blocks * bs)

    S = len(seqs)
    mb = max([nblk[i] for i in range(P, P + S)] or [1])
    bt = np.full((S, mb), poison, dtype=np.int32)
    for s in range(S):
        bt[s, :nblk[P + s]] = tables[P + s]
    w = Workload(
        name=name, number=number, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        block_size=bs, num_blocks=num_blocks, kv_dtype=kv_dtype,
        scale=np.float32(1.0 / math.sqrt(D)), poison_block=poison, unused_blocks=unused,
        fill_slots=fill, fill_k=bf16_normal(seed, _STREAM_K, (fill.size, Hkv, D)),
        fill_v=bf16_normal(seed, _STREAM_V, (fill.size, Hkv, D)),
        new_slots=new, new_k=bf16_normal(seed, _STREAM_NEW_K, (new.size, Hkv, D)),
        new_v=bf16_normal(seed, _STREAM_NEW_V, (new.size, Hkv, D)),
        q=np.empty((S, Hq, D), np.uint16), block_tables=bt,
        context_lens=np.asarray(seqs, dtype=np.int32).reshape(S), partition_size=partition_size,
        shared_blocks=None if shared is None else np.asarray(shared, np.int32))
    if P:
        tq = sum(c for (_, c) in prefill)
        w.pq = bf16_normal(seed, _STREAM_Q + 100, (tq, Hq, D))
        w.cu_seqlens_q = np.concatenate([[0], np.cumsum([c for (_, c) in prefill])]).astype(np.int32)
        w.cu_seqlens_k = np.concatenate([[0], np.cumsum(p_total)]).astype(np.int32)
        mbp = max(nblk[:P])
        pbt = np.full((P, mbp), poison, dtype=np.int32)
        for i in range(P):
            pbt[i, :nblk[i]] = tables[i]
        w.p_block_tables = pbt
    w.q = bf16_normal(seed, _STREAM_Q, (S, Hq, D))
    if kv_dtype == "fp8":
        # calibration recipe for the synthetic data: per KV head, the largest
        # magnitude drawn for the pool divided by the largest e4m3 value (448)
        w.k_scale = _amax_scale(w.fill_k, w.new_k)
        w.v_scale = _amax_scale(w.fill_v, w.new_v)
    return w


def _amax_scale(a: np.ndarray, b: np.ndarray, chunk: int = 1 << 16) -> np.ndarray:
    H = a.shape[1]
    # bf16 magnitudes order like their bit patterns with the sign bit cleared
    mbits = np.zeros(H, dtype=np.uint16)
    for arr in (a, b):
        for lo in range(0, arr.shape[0], chunk):
            part = arr[lo:lo + chunk] & np.uint16(0x7FFF)
            mbits = np.maximum(mbits, part.max(axis=(0, 2)))
    amax = bf16_bits_to_f32(mbits)
    sc = (amax / np.float32(448.0)).astype(np.float32)
    sc[amax == 0] = np.float32(1.0)
    return sc


def _lengths(seed: int, n: int, lo: int, hi: int) -> list:
    return [int(x) for x in _rng(seed, _STREAM_LENGTHS).integers(lo, hi, size=n, endpoint=True)]


def tiny_decode(seed: int = 1001) -> Workload:
    """4 sequences, contexts {1,17,64,200}, 4 Q / 2 KV heads, D 64, block 16, pool of 64."""
    return _build(1, "tiny decode", seed=seed, Hq=4, Hkv=2, D=64, bs=16,
                  seqs=[1, 17, 64, 200], num_blocks=64)


def qwen3_06b_decode(seed: int = 1002, num_seqs: int = 256) -> Workload:
    """Qwen3-0.6B-shaped decode layer: contexts U[100,1024], 16 Q / 8 KV heads, D 128, block 256."""
    return _build(2, "qwen3-0.6b decode", seed=seed, Hq=16, Hkv=8, D=128, bs=256,
                  seqs=_lengths(seed, num_seqs, 100, 1024))


def qwen3_8b_decode(seed: int = 1003, num_seqs: int = 1024, share_frac: float = 0.3) -> Workload:
    """Qwen3-8B-shaped decode layer: contexts U[100,2048], 32 Q / 8 KV heads, D 128,
    block 256; 30% of sequences share a 512-token (two-block) prefix."""
    lens = _lengths(seed, num_seqs, 100, 2048)
    eligible = np.flatnonzero(np.asarray(lens) >= 513)
    k = min(int(round(share_frac * num_seqs)), eligible.size)
    sharers = np.sort(_rng(seed, _STREAM_SHARERS).choice(eligible, size=k, replace=False))
    return _build(3, "qwen3-8b decode, shared prefix", seed=seed, Hq=32, Hkv=8, D=128, bs=256,
                  seqs=lens, sharers=sharers, shared_prefix_blocks=2)


def mixed_chunked_prefill(seed: int = 1004, num_chunks: int = 8, chunk: int = 512,
                          num_decode: int = 248) -> Workload:
    """8 prefill chunks of 512 new tokens on cached prefixes 0,256,...,1792 plus 248
    decode sequences with contexts U[100,2048]; Qwen3-8B attention shapes, block 256."""
    return _build(4, "mixed chunked prefill + decode", seed=seed, Hq=32, Hkv=8, D=128, bs=256,
                  seqs=_lengths(seed, num_decode, 100, 2048),
                  prefill=[(256 * i, chunk) for i in range(num_chunks)])


def fp8_long_decode(seed: int = 1005, num_seqs: int = 64, lo: int = 8192, hi: int = 32768) -> Workload:
    """FP8-e4m3 KV long-context decode: contexts U[8192,32768], 32 Q / 8 KV heads, D 128,
    block 256, per-KV-head scales, 1024-token partitions."""
    return _build(5, "fp8 long-context decode", seed=seed, Hq=32, Hkv=8, D=128, bs=256,
                  seqs=_lengths(seed, num_seqs, lo, hi), kv_dtype="fp8", partition_size=1024)


def mixed_chunked_prefill_fp8(seed: int = 1006) -> Workload:
    """The mixed chunked-prefill + decode step over an FP8-e4m3 KV cache (per-KV-head
    scales); same shapes and length recipe as the bf16 one."""
    return _build(6, "mixed chunked prefill + decode, fp8 KV", seed=seed, Hq=32, Hkv=8, D=128, bs=256,
                  seqs=_lengths(seed, 248, 100, 2048), prefill=[(256 * i, 512) for i in range(8)],
                  kv_dtype="fp8")


WORKLOADS = {1: tiny_decode, 2: qwen3_06b_decode, 3: qwen3_8b_decode,
             4: mixed_chunked_prefill, 5: fp8_long_decode, 6: mixed_chunked_prefill_fp8}


def make(number: int, **kw) -> Workload:
    return WORKLOADS[number](**kw)


def custom(*, seed=7, Hq=4, Hkv=2, D=64, bs=16, context_lens=(1, 5, 33), prefill=None,
           kv_dtype="bf16", partition_size=0, sharers=(), shared_prefix_blocks=0,
           num_blocks=None) -> Workload:
    """Small ad-hoc workload with the same recipe (edge cases, parity sweeps)."""
    return _build(0, "custom", seed=seed, Hq=Hq, Hkv=Hkv, D=D, bs=bs, seqs=list(context_lens),
                  prefill=prefill, kv_dtype=kv_dtype, partition_size=partition_size,
                  sharers=sharers, shared_prefix_blocks=shared_prefix_blocks,
                  num_blocks=num_blocks)


def _prefix_digest(tokens) -> list:
    """64-bit digest of every prefix tokens[:p+1] (for seeding per-position draws)."""
    out = []
    h = 1469598103934665603
    for t in tokens:
        h ^= (int(t) & 0xFFFFFFFF) + 0x9E3779B97F4A7C15
        h = (h * 1099511628211) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 29
        out.append(h)
    return out


def prefix_kv(tokens, num_kv_heads: int, head_dim: int, seed: int = 77):
    """bf16 K and V rows [len(tokens), Hkv, D] where position p's values depend
    only on tokens[:p+1]: sequences with equal prefixes get equal K/V there, as a
    model's KV cache does (what prefix caching relies on)."""
    d = _prefix_digest(tokens)
    K = np.empty((len(tokens), num_kv_heads, head_dim), np.uint16)
    V = np.empty_like(K)
    for p, h in enumerate(d):
        rng = np.random.default_rng(np.random.SeedSequence([seed, h & 0xFFFFFFFF, h >> 32]))
        x = rng.standard_normal((2, num_kv_heads, head_dim), dtype=np.float32)
        K[p] = f32_to_bf16_bits(x[0])
        V[p] = f32_to_bf16_bits(x[1])
    return K, V


def prefix_q(tokens, num_q_heads: int, head_dim: int, seed: int = 78):
    """bf16 query rows [len(tokens), Hq, D], position p's depending on tokens[:p+1]."""
    d = _prefix_digest(tokens)
    Q = np.empty((len(tokens), num_q_heads, head_dim), np.uint16)
    for p, h in enumerate(d):
        rng = np.random.default_rng(np.random.SeedSequence([seed, h & 0xFFFFFFFF, h >> 32]))
        Q[p] = f32_to_bf16_bits(rng.standard_normal((num_q_heads, head_dim), dtype=np.float32))
    return Q


_STREAM_NORM_X, _STREAM_NORM_R, _STREAM_NORM_W = 200, 201, 202


def norm_inputs(seed: int, num_tokens: int, hidden: int):
    """Inputs of a residual add + RMSNorm as bf16 bits: x [T, H] ~ N(0,1) (a
    layer's output), r [T, H] ~ 4·N(0,1) (the residual stream, larger than one
    layer's output), w [H] ~ 1 + N(0,1)/4 (a trained norm weight stays near 1)."""
    x = bf16_normal(seed, _STREAM_NORM_X, (num_tokens, hidden))
    r = bf16_normal(seed, _STREAM_NORM_R, (num_tokens, hidden))
    r = f32_to_bf16_bits(bf16_bits_to_f32(r) * np.float32(4.0))        # exact: power of two
    rng = np.random.default_rng(np.random.SeedSequence([seed, _STREAM_NORM_W]))
    w = f32_to_bf16_bits(1.0 + 0.25 * rng.standard_normal(hidden).astype(np.float32))
    return x, r, w


# Shapes of the norm workloads: the residual streams of Qwen3-8B (hidden 4096)
# over the tokens of the mixed chunked-prefill step, and of Qwen3-0.6B (1024)
# over the tokens of its decode step.
NORM_WORKLOADS = {
    "qwen3-8b mixed step (4344 tokens x 4096)": (4344, 4096),
    "qwen3-0.6b decode step (256 tokens x 1024)": (256, 1024),
}

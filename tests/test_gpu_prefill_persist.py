"""The persistent prefill launch (bf16 pool, blocks of at least 64 tokens): each
resident workgroup runs a run of work items, starting the next item's copies
during the current item's last step. Its output must not depend on how many
workgroups are resident: at every count, down to one workgroup that runs every
item back to back, it equals the one-workgroup-per-item kernel bit for bit, and
both match the oracle (element-wise |gpu - oracle| <= 1e-2 + 1e-2*|oracle|)."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import GpuCase, host_bits
from tests.util import assert_close, bf16_f64, oracle_pools

pytestmark = pytest.mark.gpu

TOL = (1e-2, 1e-2)
SLOTS = (0, 1, 2, 3, 7, 8, 13)


@pytest.fixture
def set_slots():
    import paged_kv_cache_store_amd as pa
    yield pa.prefill_set_slots
    pa.prefill_set_slots(0)


def _oracle(w):
    kc, vc = oracle_pools(w)
    return oracle.attention.prefill(w.pq, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k, w.p_block_tables,
                                    w.scale, w.block_size, w.k_scale, w.v_scale)


def _check_all_slots(w, set_slots, slots=SLOTS):
    case = GpuCase(w)
    set_slots(-1)
    ref = host_bits(case.prefill())   # one workgroup per work item
    for n in slots:
        set_slots(n)
        got = host_bits(case.prefill())
        diff = np.flatnonzero(got.reshape(-1) != ref.reshape(-1))
        assert diff.size == 0, f"slots={n}: {diff.size} values differ, first at flat index {diff[:4]}"
    ma, mr = assert_close(bf16_f64(ref), _oracle(w), *TOL, what="prefill")
    print(f"max_abs={ma:.3e} max_rel={mr:.3e}")


CASES = [
    # one-tile items between long ones, two query heads per KV head, 64-token blocks
    dict(seed=341, Hq=8, Hkv=2, D=128, bs=64, prefill=[(0, 1), (0, 33), (130, 5), (0, 64), (700, 300), (63, 2),
                                                       (1, 1)]),
    # the mixed step's shapes (four heads per KV head, 256-token blocks), shorter
    dict(seed=342, Hq=32, Hkv=8, D=128, bs=256, prefill=[(256 * i, 512) for i in range(4)] + [(0, 7), (1000, 1)]),
    dict(seed=343, Hq=16, Hkv=8, D=64, bs=128, prefill=[(5, 250), (0, 129), (300, 1), (17, 3)]),
    # eight query heads per KV head: 16 rows per work item
    dict(seed=344, Hq=8, Hkv=1, D=128, bs=64, prefill=[(0, 200), (64, 64), (3, 61)]),
    # one query head per KV head: 128 rows per work item, waves with different rows
    dict(seed=345, Hq=4, Hkv=4, D=64, bs=64, prefill=[(0, 300), (100, 150), (0, 2)]),
]


@pytest.mark.parametrize("cfg", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_persistent_every_slot_count(cfg, set_slots):
    print(f"case {cfg}", flush=True)
    _check_all_slots(W.custom(context_lens=(), **cfg), set_slots)


def test_persistent_many_sequences(set_slots):
    """Sequences up to the ranked limit (256), many short items per workgroup;
    past the limit the one-workgroup-per-item kernel runs whatever the setting,
    so the output is the same too."""
    rng = np.random.default_rng(346)
    for n in (256, 300):
        pf = [(int(rng.integers(0, 200)), int(rng.integers(1, 40))) for _ in range(n)]
        print(f"{n} sequences", flush=True)
        w = W.custom(seed=347, Hq=8, Hkv=2, D=64, bs=64, context_lens=(), prefill=pf)
        _check_all_slots(w, set_slots, slots=(0, 5, 64))


def test_persistent_rows_without_keys(set_slots):
    """Sequences with fewer keys than queries (the first Lq-Lk rows see no key)
    and with no keys at all: those rows are zeros, items whose rows all see no
    key are written as zeros without reading the pool."""
    w = W.custom(seed=348, Hq=8, Hkv=2, D=128, bs=64, context_lens=(),
                 prefill=[(0, 100), (0, 70), (40, 90), (0, 5), (10, 300)])
    lk = np.diff(w.cu_seqlens_k).astype(np.int64)
    lk[0] = 60      # 100 queries on 60 keys
    lk[1] = 0       # no keys
    lk[3] = 2       # 5 queries on 2 keys
    w.cu_seqlens_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    print("keys per sequence", lk.tolist(), flush=True)
    _check_all_slots(w, set_slots)
    case = GpuCase(w)
    got = bf16_f64(host_bits(case.prefill()))
    q0, q1 = int(w.cu_seqlens_q[1]), int(w.cu_seqlens_q[2])
    assert not np.any(got[q0:q1]), "a sequence with no keys must give zero rows"


def test_persistent_mixed_step_full_size(set_slots):
    """The mixed step's 8 chunks (1024 work items over the resident workgroups):
    the default launch equals the one-workgroup-per-item kernel bit for bit."""
    w = W.make(4)
    case = GpuCase(w)
    set_slots(-1)
    ref = host_bits(case.prefill())
    for n in (0, 100):
        set_slots(n)
        assert np.array_equal(host_bits(case.prefill()), ref), f"slots={n}"


def test_persistent_long_context_window_refill(set_slots):
    """Items whose keys span more block ids than one LDS window holds (256 ids
    of 64-token blocks: 16384 keys): the item's window moves forward while it
    runs, next to items whose windows were filled ahead."""
    w = W.custom(seed=350, Hq=8, Hkv=2, D=128, bs=64, context_lens=(),
                 prefill=[(20000, 40), (17000, 100), (100, 30), (16380, 9)])
    _check_all_slots(w, set_slots, slots=(0, 1, 3))


def test_persistent_random_shapes(set_slots):
    """Seeded random batches (head groupings, head sizes, block sizes, prefix and
    chunk lengths, now and then fewer keys than queries): the persistent launch
    at several resident-workgroup counts equals one workgroup per item bit for
    bit; the oracle checks one batch in four."""
    rng = np.random.default_rng(351)
    for trial in range(24):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        bs = int(rng.choice([64, 128, 256]))
        nseq = int(rng.integers(1, 13))
        pf = [(int(rng.integers(0, 700)), int(rng.integers(1, 260))) for _ in range(nseq)]
        w = W.custom(seed=352 + trial, Hq=hkv * g, Hkv=hkv, D=d, bs=bs, context_lens=(), prefill=pf)
        if rng.random() < 0.3:
            lk = np.diff(w.cu_seqlens_k).astype(np.int64)
            i = int(rng.integers(0, nseq))
            lk[i] = int(rng.integers(0, lk[i] + 1))
            w.cu_seqlens_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        print(f"trial {trial}: G={g} Hkv={hkv} D={d} bs={bs} chunks={pf} lk={np.diff(w.cu_seqlens_k).tolist()}",
              flush=True)
        case = GpuCase(w)
        set_slots(-1)
        ref = host_bits(case.prefill())
        for n in (0, 1, 3, 7):
            set_slots(n)
            got = host_bits(case.prefill())
            assert np.array_equal(got, ref), f"trial {trial}, slots={n}"
        if trial % 4 == 0:
            assert_close(bf16_f64(ref), _oracle(w), *TOL, what=f"trial {trial}")


def test_pool_end_block(set_slots):
    """A sequence whose last keys sit in the pool's last physical block, with
    its last 64-key tile running past the context inside that block: the tile
    copies read only that block's bytes (blocks of 64 and 256 tokens, both
    launch forms, against the oracle). The pool has one block to spare, the
    seeds place a sequence's final block last."""
    import math
    pf = [(0, 1), (37, 100), (200, 61), (5, 3), (64, 64)]
    for seed, bs, seq in ((351, 64, 2), (351, 256, 1)):
        needed = sum(math.ceil((p + c) / bs) for p, c in pf)
        w = W.custom(seed=seed, Hq=8, Hkv=2, D=128, bs=bs, context_lens=(), prefill=pf, num_blocks=needed + 1)
        lk = sum(pf[seq])
        assert w.p_block_tables[seq, math.ceil(lk / bs) - 1] == w.num_blocks - 1 and lk % 64 != 0
        print(f"seed {seed} block {bs}: sequence {seq} ends in block {w.num_blocks - 1}", flush=True)
        _check_all_slots(w, set_slots, slots=(0, 1))

"""GPU parity of pa_store_kv and pa_decode against the CPU oracle (through the C ABI).

Store: bit-exact (bf16 bits; fp8 codes) over whole pools, NaN sentinels included.
Decode: element-wise |gpu - oracle| <= atol + rtol*|oracle| with atol = rtol = 1e-2
for a bf16 cache and 3e-2 for fp8 (oracle on the same fp8 bytes, float64).
Every workload is checked in full: every sequence's output and every pool byte.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import GpuCase, host_bits
from tests.util import (assert_close, bf16_f64, oracle_decode_threads, oracle_pools, poisoned_pools,
                        relabel_blocks)

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1e-2), "fp8": (3e-2, 3e-2)}


def _oracle_decode(w, kc, vc, seqs=None):
    return oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                   w.block_size, w.k_scale, w.v_scale, seqs=seqs)


def _check_pools_equal(case, kc, vc, blocks=None):
    gk = case.k_cache if blocks is None else case.k_cache[torch.as_tensor(blocks, device="cuda").long()]
    gv = case.v_cache if blocks is None else case.v_cache[torch.as_tensor(blocks, device="cuda").long()]
    ok_k = host_bits(gk)
    ok_v = host_bits(gv)
    rk = kc if blocks is None else kc[blocks]
    rv = vc if blocks is None else vc[blocks]
    nk = np.count_nonzero(ok_k != rk)
    nv = np.count_nonzero(ok_v != rv)
    assert nk == 0 and nv == 0, f"pool bytes differ: K {nk}, V {nv}"


# ---------------------------------------------------------------- small workloads, whole pools
EDGE = [
    dict(seed=101, Hq=4, Hkv=2, D=64, bs=16, context_lens=(0, 1, 15, 16, 17, 63, 64, 65, 200)),
    dict(seed=102, Hq=8, Hkv=8, D=128, bs=32, context_lens=(1, 31, 32, 33, 300)),
    dict(seed=103, Hq=16, Hkv=2, D=128, bs=64, context_lens=(5, 127, 128, 129, 700)),
    dict(seed=104, Hq=16, Hkv=4, D=64, bs=128, context_lens=(255, 256, 257, 1023, 1024, 1025),
         partition_size=256),
    dict(seed=105, Hq=32, Hkv=8, D=128, bs=256,
         context_lens=(1, 255, 256, 257, 511, 512, 513, 1100), partition_size=256),
    dict(seed=106, Hq=32, Hkv=8, D=128, bs=256, context_lens=(1, 17, 300, 1024, 1025, 3000),
         kv_dtype="fp8", partition_size=1024),
    dict(seed=107, Hq=8, Hkv=4, D=64, bs=16, context_lens=(1, 16, 17, 100), kv_dtype="fp8"),
    dict(seed=108, Hq=8, Hkv=1, D=64, bs=64, context_lens=(2000, 3), kv_dtype="fp8", partition_size=256),
    dict(seed=109, Hq=4, Hkv=4, D=128, bs=16, context_lens=(4096, 1, 77), partition_size=512),
    # with the cases above, every (G, D, dtype) the decode kernels are built for
    # (G 1/2/4/8: one set of 4x4x4 MFMA columns with padding, or two sets)
    dict(seed=110, Hq=16, Hkv=2, D=128, bs=32, context_lens=(3, 64, 65, 450), kv_dtype="fp8"),
    dict(seed=111, Hq=4, Hkv=4, D=128, bs=64, context_lens=(1, 129, 700), kv_dtype="fp8"),
    dict(seed=112, Hq=16, Hkv=4, D=64, bs=256, context_lens=(2, 255, 600), kv_dtype="fp8",
         partition_size=256),
    dict(seed=113, Hq=16, Hkv=2, D=64, bs=16, context_lens=(7, 64, 300)),
    dict(seed=114, Hq=4, Hkv=2, D=128, bs=128, context_lens=(1, 128, 129, 1500), partition_size=512),
    dict(seed=115, Hq=4, Hkv=4, D=64, bs=32, context_lens=(1, 33, 64, 250)),
    dict(seed=116, Hq=8, Hkv=4, D=128, bs=64, context_lens=(1, 64, 65, 900), kv_dtype="fp8"),
    dict(seed=117, Hq=2, Hkv=2, D=64, bs=128, context_lens=(3, 128, 129, 1000), kv_dtype="fp8",
         partition_size=512),
]


@pytest.mark.parametrize("cfg", EDGE, ids=[f"edge{i}" for i in range(len(EDGE))])
def test_store_and_decode_small(cfg):
    w = W.custom(**cfg)
    print(f"case {cfg}", flush=True)
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    _check_pools_equal(case, kc, vc)
    for ps in sorted({w.partition_size, 0, 256, 4096}):
        got = bf16_f64(host_bits(case.decode(partition_size=ps)))
        ref = _oracle_decode(w, kc, vc)
        assert_close(got, ref, *TOL[w.kv_dtype], what=f"P={ps}")


def test_tiny_decode_workload():
    w = W.make(1)
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    _check_pools_equal(case, kc, vc)
    got = bf16_f64(host_bits(case.decode()))
    ma, mr = assert_close(got, _oracle_decode(w, kc, vc), *TOL["bf16"], what="tiny")
    print(f"[tiny decode] max_abs={ma:.3e} max_rel={mr:.3e}")


# ---------------------------------------------------------------- full-size workloads
@pytest.fixture(scope="module")
def qwen3_06b():
    w = W.make(2)
    return w, GpuCase(w)


def test_qwen3_06b_store_bitexact(qwen3_06b):
    w, case = qwen3_06b
    kc, vc = oracle_pools(w)
    _check_pools_equal(case, kc, vc)


def test_qwen3_06b_decode_all_sequences(qwen3_06b):
    w, case = qwen3_06b
    kc, vc = oracle_pools(w)
    got = bf16_f64(host_bits(case.decode()))
    ma, mr = assert_close(got, _oracle_decode(w, kc, vc), *TOL["bf16"], what="qwen3-0.6b")
    print(f"[qwen3-0.6b decode] max_abs={ma:.3e} max_rel={mr:.3e}")


def _fused_case(w):
    """Pools holding the cached context only, and the step's newest tokens as
    pa_store_decode takes them."""
    from tests.gpu_util import dev_bf16, dev_i32
    case = GpuCase(w, store_new=False)
    k, v, slots = _newest_per_sequence(w)
    return case, dev_bf16(k), dev_bf16(v), dev_i32(slots)


def _store_decode(case, k, v, slots, partition_size=None):
    w = case.w
    ps = w.partition_size if partition_size is None else partition_size
    return case.pa.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                          float(w.scale), w.max_context_len, k_scale=case.k_scale, v_scale=case.v_scale,
                          partition_size=ps, new_k=k, new_v=v, slot_mapping=slots)


def test_qwen3_06b_store_decode_full():
    """The headline step as timed: pa_store_decode over the Qwen3-0.6B layer, every
    sequence against the oracle, every pool byte against the oracle's store."""
    w = W.make(2)
    case, k, v, slots = _fused_case(w)
    got = bf16_f64(host_bits(_store_decode(case, k, v, slots)))
    kc, vc = oracle_pools(w)
    _check_pools_equal(case, kc, vc)
    ma, mr = assert_close(got, _oracle_decode(w, kc, vc), *TOL["bf16"], what="qwen3-0.6b fused")
    print(f"[qwen3-0.6b store+decode] max_abs={ma:.3e} max_rel={mr:.3e}")


@pytest.fixture(scope="module", params=[3, 5], ids=["qwen3-8b", "fp8-long"])
def full_size(request):
    """Qwen3-8B (1024 sequences, shared prefix) and fp8 long context (64
    sequences, split contexts): the oracle's pools after storing every cached
    and new token, and the oracle's decode of every sequence."""
    w = W.make(request.param)
    print(w.name, flush=True)
    kc, vc = oracle_pools(w)
    ref = oracle_decode_threads(w, kc, vc)
    return w, kc, vc, ref


def test_full_size_store_and_decode_vs_oracle(full_size):
    """pa_store_kv of every token, then pa_decode: whole pools byte for byte and
    every sequence's output against the oracle."""
    w, kc, vc, ref = full_size
    case = GpuCase(w)
    _check_pools_equal(case, kc, vc)
    got = bf16_f64(host_bits(case.decode()))
    ma, mr = assert_close(got, ref, *TOL[w.kv_dtype], what=f"{w.name} decode, all sequences")
    print(f"[{w.name} decode, {w.num_seqs} sequences] max_abs={ma:.3e} max_rel={mr:.3e}")


def test_full_size_store_decode_vs_oracle(full_size):
    """pa_store_decode (newest tokens stored in the decode launch): every
    sequence's output and the whole pools against the oracle."""
    w, kc, vc, ref = full_size
    case, k, v, slots = _fused_case(w)
    got = bf16_f64(host_bits(_store_decode(case, k, v, slots)))
    _check_pools_equal(case, kc, vc)
    ma, mr = assert_close(got, ref, *TOL[w.kv_dtype], what=f"{w.name} store+decode, all sequences")
    print(f"[{w.name} store+decode, {w.num_seqs} sequences] max_abs={ma:.3e} max_rel={mr:.3e}")


@pytest.mark.parametrize("number", [3, 5], ids=["qwen3-8b", "fp8-long"])
def test_store_decode_full_size_matches_two_launches(number):
    """The fused call gives the bits of pa_store_kv + pa_decode, output and pools."""
    w = W.make(number)
    print(w.name, flush=True)
    fused, k, v, slots = _fused_case(w)
    got = host_bits(_store_decode(fused, k, v, slots))
    fk, fv = host_bits(fused.k_cache), host_bits(fused.v_cache)
    del fused
    torch.cuda.empty_cache()
    two = GpuCase(w)
    want = host_bits(two.decode())
    assert np.array_equal(got, want)
    assert np.array_equal(fk, host_bits(two.k_cache)) and np.array_equal(fv, host_bits(two.v_cache))


# ---------------------------------------------------------------- invariants and closed forms
def test_context_one_returns_v_exactly():
    w = W.custom(seed=201, Hq=8, Hkv=2, D=128, bs=16, context_lens=(1, 1, 1))
    case = GpuCase(w)
    out = host_bits(case.decode())
    expect = np.repeat(w.new_v, 4, axis=1)          # query head h reads KV head h // 4
    assert np.array_equal(out, expect)


def test_block_permutation_bit_identical():
    w = W.custom(seed=202, Hq=8, Hkv=2, D=128, bs=32, context_lens=(7, 90, 300, 1500),
                 partition_size=256)
    a = host_bits(GpuCase(w).decode())
    b = host_bits(GpuCase(relabel_blocks(w, seed=4)).decode())
    assert np.array_equal(a, b)


def test_shared_prefix_equals_private_copies_bit_identical():
    w = W.custom(seed=203, Hq=8, Hkv=2, D=128, bs=64, context_lens=(300, 400, 500),
                 sharers=(0, 1, 2), shared_prefix_blocks=2, num_blocks=40)
    case = GpuCase(w)
    shared = host_bits(case.decode())
    bt = w.block_tables.copy()
    free = list(w.unused_blocks[1:])
    for s in (1, 2):
        for j in range(2):
            nb = int(free.pop())
            case.k_cache[nb] = case.k_cache[int(bt[s, j])]
            case.v_cache[nb] = case.v_cache[int(bt[s, j])]
            bt[s, j] = nb
    case.block_tables = torch.from_numpy(bt).cuda()
    private = host_bits(case.decode())
    assert np.array_equal(shared, private)


def test_split_matches_single_partition():
    w = W.custom(seed=204, Hq=32, Hkv=8, D=128, bs=256, context_lens=(3000, 4096, 999, 2500))
    case = GpuCase(w)
    one = bf16_f64(host_bits(case.decode(partition_size=4096)))
    for ps in (256, 512, 1024):
        split = bf16_f64(host_bits(case.decode(partition_size=ps)))
        # same arithmetic up to float32 rounding order, then one bf16 rounding each
        np.testing.assert_allclose(split, one, rtol=2 ** -7, atol=1e-3)


def test_deterministic_and_guard_bands():
    w = W.custom(seed=205, Hq=16, Hkv=8, D=128, bs=256, context_lens=(100, 1024, 3000),
                 partition_size=512)
    case = GpuCase(w)
    S, Hq, D = w.q.shape
    buf = torch.full((S + 2, Hq, D), 1234.0, dtype=torch.bfloat16, device="cuda")
    case.decode(out=buf[1:S + 1])
    first = host_bits(buf)
    case.decode(out=buf[1:S + 1])
    second = host_bits(buf)
    assert np.array_equal(first, second)
    sentinel = host_bits(torch.full((Hq, D), 1234.0, dtype=torch.bfloat16))
    assert np.array_equal(first[0], sentinel) and np.array_equal(first[S + 1], sentinel)


def test_store_skips_negative_and_out_of_range_slots():
    w = W.custom(seed=206, Hq=4, Hkv=2, D=64, bs=16, context_lens=(40, 9))
    case = GpuCase(w, store_new=False)
    before_k, before_v = host_bits(case.k_cache), host_bits(case.v_cache)
    slots = w.new_slots.copy()
    slots[0::2] = -1
    slots[1::2] = w.num_blocks * w.block_size + 5
    case.store(case.new_k, case.new_v, torch.from_numpy(slots).cuda())
    assert np.array_equal(host_bits(case.k_cache), before_k)
    assert np.array_equal(host_bits(case.v_cache), before_v)


def test_store_runs_of_slots_bit_exact():
    """Batches mixing whole aligned runs of 8 slots (written as whole V chunks), an
    unaligned partial run, a run broken by token order, a run holding an invalid
    slot and a run cut by the end of the batch: every pool byte equals the oracle's."""
    import paged_kv_cache_store_amd as pa
    for kv in ("bf16", "fp8"):
        w = W.custom(seed=208, Hq=4, Hkv=2, D=64, bs=16, context_lens=(), num_blocks=12, kv_dtype=kv)
        run = list(range(16, 32))                        # two aligned runs
        part = list(range(37, 43))                       # unaligned partial run
        swapped = list(range(48, 56))
        swapped[3], swapped[4] = swapped[4], swapped[3]  # same slots, order broken
        holed = list(range(64, 72))
        holed[5] = -1                                    # a skipped slot inside a run
        tail = list(range(80, 86))                       # run cut by the end of the batch
        slots = np.array(run + part + swapped + holed + [176, 177] + tail, dtype=np.int32)
        T = slots.size
        rng = np.random.default_rng(9)
        k = W.f32_to_bf16_bits(rng.standard_normal((T, 2, 64)).astype(np.float32))
        v = W.f32_to_bf16_bits(rng.standard_normal((T, 2, 64)).astype(np.float32))
        case = GpuCase(w, store_new=False)
        kc, vc = poisoned_pools(w)
        oracle.cache.store(k, v, slots, kc, vc, w.block_size, w.k_scale, w.v_scale)
        from tests.gpu_util import dev_bf16, dev_i32
        case.store(dev_bf16(k), dev_bf16(v), dev_i32(slots))
        assert np.array_equal(host_bits(case.k_cache), kc), kv
        assert np.array_equal(host_bits(case.v_cache), vc), kv


def _newest_per_sequence(w):
    """The step's new tokens as pa_store_decode takes them: one per sequence, slot
    -1 for an empty sequence (decode-only workloads list them in sequence order)."""
    S = w.q.shape[0]
    live = np.flatnonzero(w.context_lens > 0)
    assert live.size == w.new_slots.size
    k = np.zeros((S,) + w.new_k.shape[1:], np.uint16)
    v = np.zeros_like(k)
    slots = np.full(S, -1, np.int32)
    k[live], v[live], slots[live] = w.new_k, w.new_v, w.new_slots
    return k, v, slots


@pytest.mark.parametrize("cfg", EDGE, ids=[f"edge{i}" for i in range(len(EDGE))])
def test_store_decode_matches_store_then_decode(cfg):
    """pa_store_decode writes the same pool bytes as pa_store_kv and returns the
    same output bits as pa_decode after it, for every partition size; the output
    also meets the oracle's tolerance on its own."""
    import paged_kv_cache_store_amd as pa
    from tests.gpu_util import dev_bf16, dev_i32
    w = W.custom(**cfg)
    print(f"case {cfg}", flush=True)
    k, v, slots = _newest_per_sequence(w)
    two_step = GpuCase(w)
    fused = GpuCase(w, store_new=False)
    kd, vd, sd = dev_bf16(k), dev_bf16(v), dev_i32(slots)
    kc, vc = oracle_pools(w)
    ref = _oracle_decode(w, kc, vc)
    for ps in sorted({w.partition_size, 0, 256, 4096}):
        want = host_bits(two_step.decode(partition_size=ps))
        got = pa.decode(fused.q, fused.k_cache, fused.v_cache, fused.block_tables, fused.context_lens,
                        float(w.scale), w.max_context_len, k_scale=fused.k_scale, v_scale=fused.v_scale,
                        partition_size=ps, new_k=kd, new_v=vd, slot_mapping=sd)
        got = host_bits(got)
        assert np.array_equal(got, want), f"P={ps}: fused output differs from store + decode"
        assert_close(bf16_f64(got), ref, *TOL[w.kv_dtype], what=f"fused P={ps}")
        _check_pools_equal(fused, kc, vc)


def test_store_decode_slot_elsewhere():
    """A slot that is not the newest position's (here: slots of an unused block)
    is written as pa_store_kv writes it; pools and output match store + decode."""
    import paged_kv_cache_store_amd as pa
    from tests.gpu_util import dev_bf16, dev_i32
    for kv in ("bf16", "fp8"):
        w = W.custom(seed=210, Hq=8, Hkv=2, D=128, bs=16, context_lens=(40, 9, 100, 33), kv_dtype=kv)
        k, v, slots = _newest_per_sequence(w)
        spare = int(w.unused_blocks[0]) * w.block_size
        slots[1], slots[3] = spare + 3, spare + 12
        kd, vd, sd = dev_bf16(k), dev_bf16(v), dev_i32(slots)
        two_step = GpuCase(w)
        two_step.store(kd, vd, sd)
        want = host_bits(two_step.decode())
        fused = GpuCase(w)
        got = pa.decode(fused.q, fused.k_cache, fused.v_cache, fused.block_tables, fused.context_lens,
                        float(w.scale), w.max_context_len, k_scale=fused.k_scale, v_scale=fused.v_scale,
                        new_k=kd, new_v=vd, slot_mapping=sd)
        assert np.array_equal(host_bits(got), want), kv
        assert np.array_equal(host_bits(fused.k_cache), host_bits(two_step.k_cache)), kv
        assert np.array_equal(host_bits(fused.v_cache), host_bits(two_step.v_cache)), kv


def test_store_decode_skips_invalid_slots():
    """A slot < 0 or past the pool writes nothing; the decode still runs."""
    import paged_kv_cache_store_amd as pa
    from tests.gpu_util import dev_bf16, dev_i32
    w = W.custom(seed=209, Hq=8, Hkv=2, D=128, bs=16, context_lens=(40, 9, 0))
    k, v, slots = _newest_per_sequence(w)
    case = GpuCase(w, store_new=False)
    before_k, before_v = host_bits(case.k_cache), host_bits(case.v_cache)
    slots[0] = -7
    slots[1] = w.num_blocks * w.block_size
    slots[2] = -1
    out = pa.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                    float(w.scale), w.max_context_len, new_k=dev_bf16(k), new_v=dev_bf16(v),
                    slot_mapping=dev_i32(slots))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(case.k_cache), before_k)
    assert np.array_equal(host_bits(case.v_cache), before_v)
    assert not np.any(bf16_f64(host_bits(out))[2])          # empty sequence: zeros


def test_store_large_batch_patterns_bit_exact():
    """A batch large enough for the tiled store path (64 tokens per workgroup):
    aligned and unaligned runs, runs across a tile edge, order breaks, holes,
    skipped and out-of-range slots, and scattered single tokens, bf16 and fp8;
    every pool byte equals the oracle's."""
    rng = np.random.default_rng(11)
    for kv in ("bf16", "fp8"):
        bs, nb = 16, 1400
        w = W.custom(seed=211, Hq=4, Hkv=2, D=64, bs=bs, context_lens=(), num_blocks=nb, kv_dtype=kv)
        free = rng.permutation(nb)                 # blocks in random order
        slots = []
        for i, blk in enumerate(free[:1100]):
            base = int(blk) * bs
            kind = i % 6
            if kind == 0:                          # whole block in order
                slots += list(range(base, base + bs))
            elif kind == 1:                        # unaligned start, partial
                slots += list(range(base + 3, base + 13))
            elif kind == 2:                        # order broken inside a run
                seg = list(range(base, base + bs))
                seg[5], seg[6] = seg[6], seg[5]
                slots += seg
            elif kind == 3:                        # hole (-1) and an out-of-range slot
                seg = list(range(base, base + bs))
                seg[2] = -1
                seg[11] = nb * bs + 7
                slots += seg
            elif kind == 4:                        # a few scattered tokens
                slots += [base + int(o) for o in rng.choice(bs, 3, replace=False)]
            else:                                  # block in reverse order
                slots += list(range(base + bs - 1, base - 1, -1))
        slots = np.array(slots, dtype=np.int32)
        T = slots.size
        assert T > 256 * 64 // 2, T                # the tiled path: at least 256 workgroups
        k = W.f32_to_bf16_bits(rng.standard_normal((T, 2, 64)).astype(np.float32))
        v = W.f32_to_bf16_bits(rng.standard_normal((T, 2, 64)).astype(np.float32))
        from tests.gpu_util import dev_bf16, dev_i32
        case = GpuCase(w, store_new=False)
        kc, vc = poisoned_pools(w)
        # the library skips slots past the pool as it skips negative ones
        oracle.cache.store(k, v, np.where(slots < nb * bs, slots, -1), kc, vc, w.block_size,
                           w.k_scale, w.v_scale)
        case.store(dev_bf16(k), dev_bf16(v), dev_i32(slots))
        assert np.array_equal(host_bits(case.k_cache), kc), kv
        assert np.array_equal(host_bits(case.v_cache), vc), kv


def test_wrapper_rejects_bad_arguments():
    import paged_kv_cache_store_amd as pa
    w = W.custom(seed=207, Hq=4, Hkv=2, D=64, bs=16, context_lens=(5,))
    case = GpuCase(w)
    with pytest.raises(ValueError):
        pa.decode(case.q.float(), case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                  0.125, 5)
    with pytest.raises(pa.PaError):
        pa.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, 0.125, 5,
                  partition_size=100)


def test_longest_first_order_many_sequences():
    """From 128 sequences on, a kernel ranks the sequences longest first before
    the decode. Many equal lengths, empty sequences, split and whole contexts:
    every sequence against the oracle, and each sequence's output bit-identical
    when the batch is given in reverse order or below the ranking threshold."""
    rng = np.random.default_rng(120)
    lens = [0] * 5 + [1] * 10 + [64] * 40 + [65] * 20 + rng.integers(1, 3000, 125).tolist()
    lens = [int(x) for x in rng.permutation(lens)]
    w = W.custom(seed=120, Hq=8, Hkv=2, D=64, bs=32, context_lens=tuple(lens))
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    ref = _oracle_decode(w, kc, vc)
    outs = {}
    for ps in (0, 1024):
        got = host_bits(case.decode(partition_size=ps))
        assert_close(bf16_f64(got), ref, *TOL["bf16"], what=f"P={ps}")
        outs[ps] = got
    # the same sequences in reverse batch order: same bits per sequence
    import paged_kv_cache_store_amd as pa
    from tests.gpu_util import dev_bf16, dev_i32
    rev = pa.decode(dev_bf16(w.q[::-1]), case.k_cache, case.v_cache, dev_i32(w.block_tables[::-1]),
                    dev_i32(w.context_lens[::-1]), float(w.scale), w.max_context_len)
    assert np.array_equal(host_bits(rev)[::-1], outs[0])
    # 100 sequences (no ranking kernel): same bits for those sequences
    sub = np.arange(100)
    few = pa.decode(dev_bf16(w.q[sub]), case.k_cache, case.v_cache, dev_i32(w.block_tables[sub]),
                    dev_i32(w.context_lens[sub]), float(w.scale), w.max_context_len)
    assert np.array_equal(host_bits(few), outs[0][sub])


def test_longest_first_order_beyond_register_keys():
    """More than 4096 sequences: the ranking keeps the first 4096 bucket keys in
    registers and recomputes the rest; every sequence against the oracle."""
    rng = np.random.default_rng(121)
    lens = rng.integers(1, 40, 5000).tolist()
    lens[4321] = 1500                       # one long context: the ranking runs
    lens[17] = 0
    w = W.custom(seed=121, Hq=2, Hkv=1, D=64, bs=16, context_lens=tuple(int(x) for x in lens))
    case = GpuCase(w)
    kc, vc = oracle_pools(w)
    got = bf16_f64(host_bits(case.decode(partition_size=0)))
    assert_close(got, _oracle_decode(w, kc, vc), *TOL["bf16"], what="5000 sequences")

"""The host block manager (allocation, free/reuse, prefix caching, fork and
copy-on-write) on the CPU, through the C ABI."""
import random

import pytest

pa = pytest.importorskip("paged_kv_cache_store_amd")


def test_allocation_and_release():
    bm = pa.BlockManager(10, 4, prefix_caching=False)
    a, c = bm.add_sequence(list(range(9)))          # 3 blocks
    assert c == 0 and bm.info(a) == (9, 3) and bm.num_free_blocks == 7
    b, _ = bm.add_sequence(list(range(9)))          # no caching: private blocks
    ta, tb = bm.block_table(a, 3), bm.block_table(b, 3)
    assert not set(ta) & set(tb)
    assert bm.slots(a, 0, 9) == [ta[p // 4] * 4 + p % 4 for p in range(9)]
    bm.free(a)
    assert bm.num_free_blocks == 7 and all(bm.refcount(x) == 0 for x in ta)
    with pytest.raises(pa.PaError):
        bm.free(a)                                    # unknown id


def test_prefix_hits_reuse_full_blocks_only():
    bm = pa.BlockManager(32, 4)
    sys_prompt = [7, 3, 9, 1, 4, 4, 2, 8, 6, 5]       # 2 full blocks + 2 tokens
    a, c = bm.add_sequence(sys_prompt + [11, 12])
    assert c == 0
    b, c = bm.add_sequence(sys_prompt + [21, 22, 23])
    assert c == 8                                    # the two full blocks
    ta, tb = bm.block_table(a, 3), bm.block_table(b, 4)
    assert ta[:2] == tb[:2] and ta[2] != tb[2]
    assert bm.refcount(ta[0]) == 2 and bm.refcount(ta[2]) == 1
    # a different first block: no hit at all, even if later blocks match
    d, c = bm.add_sequence([0] + sys_prompt[1:] + [11, 12])
    assert c == 0 and not set(bm.block_table(d, 3)) & set(ta)


def test_freed_cached_blocks_are_reused_until_handed_out():
    bm = pa.BlockManager(6, 4)
    prompt = list(range(100, 112))                   # 3 full blocks
    a, _ = bm.add_sequence(prompt)
    t = bm.block_table(a, 3)
    bm.free(a)
    assert bm.num_free_blocks == 6
    b, c = bm.add_sequence(prompt + [1])             # hits all 3 cached free blocks
    assert c == 12 and bm.block_table(b, 4)[:3] == t
    bm.free(b)
    # fill the pool with unrelated sequences: cached blocks get handed out again
    x, _ = bm.add_sequence(list(range(24)))
    bm.free(x)
    y, c = bm.add_sequence(prompt)
    assert c == 0


def test_out_of_blocks_changes_nothing():
    bm = pa.BlockManager(4, 4)
    a, _ = bm.add_sequence(list(range(12)))
    with pytest.raises(pa.PaError) as e:
        bm.add_sequence(list(range(50, 58)))
    assert e.value.status == -6 and bm.num_free_blocks == 1
    slot, cow = bm.append_token(a, 99)               # fits in the last block? 12 % 4 == 0 -> new block
    assert cow is None and bm.num_free_blocks == 0
    with pytest.raises(pa.PaError):
        bm.add_sequence([1])


def test_append_fills_then_hashes_blocks():
    bm = pa.BlockManager(16, 4)
    a, _ = bm.add_sequence([5, 6])
    toks = [5, 6]
    for t in [7, 8, 9]:
        slot, cow = bm.append_token(a, t)
        toks.append(t)
        assert cow is None
        row = bm.block_table(a, 2)
        assert slot == row[(len(toks) - 1) // 4] * 4 + (len(toks) - 1) % 4
    # the first block became full while decoding: another prompt with it hits
    b, c = bm.add_sequence([5, 6, 7, 8, 1])
    assert c == 4 and bm.block_table(b, 2)[0] == bm.block_table(a, 2)[0]


def test_fork_copy_on_write():
    bm = pa.BlockManager(16, 4)
    a, _ = bm.add_sequence([1, 2, 3, 4, 5, 6])       # last block holds 2 tokens
    f = bm.fork(a)
    ta = bm.block_table(a, 2)
    assert bm.block_table(f, 2) == ta and bm.refcount(ta[1]) == 2
    slot, cow = bm.append_token(f, 70)
    assert cow is not None and cow[0] == ta[1]
    tf = bm.block_table(f, 2)
    assert tf[0] == ta[0] and tf[1] == cow[1] and slot == cow[1] * 4 + 2
    assert bm.refcount(ta[1]) == 1
    slot_a, cow_a = bm.append_token(a, 80)           # a owns its block alone now
    assert cow_a is None and slot_a == ta[1] * 4 + 2


def test_random_operations_keep_invariants():
    rng = random.Random(5)
    bm = pa.BlockManager(64, 4)
    live = {}
    for step in range(600):
        op = rng.random()
        try:
            if op < 0.3 or not live:
                prefix = [1, 2, 3, 4, 5, 6, 7, 8][:rng.choice([0, 4, 8])]
                toks = prefix + [rng.randrange(50) for _ in range(rng.randrange(1, 10))]
                sid, cached = bm.add_sequence(toks)
                live[sid] = list(toks)
                assert cached % 4 == 0 and cached <= len(toks)
            elif op < 0.75:
                sid = rng.choice(list(live))
                t = rng.randrange(50)
                bm.append_token(sid, t)
                live[sid].append(t)
            elif op < 0.85:
                sid = rng.choice(list(live))
                live[bm.fork(sid)] = list(live[sid])
            else:
                sid = rng.choice(list(live))
                bm.free(sid)
                del live[sid]
        except pa.PaError as e:
            assert e.status == -6
        # invariants: refcounts equal table membership; free count matches
        owners = {}
        for sid, toks in live.items():
            n, nb = bm.info(sid)
            assert n == len(toks) and nb == -(-n // 4)
            for b in bm.block_table(sid, nb):
                owners[b] = owners.get(b, 0) + 1
        assert all(bm.refcount(b) == owners.get(b, 0) for b in range(64))
        assert bm.num_free_blocks == sum(1 for b in range(64) if owners.get(b, 0) == 0)
        # a block shared by several sequences holds the same tokens in each
        seen = {}
        for sid, toks in live.items():
            for j, b in enumerate(bm.block_table(sid, -(-len(toks) // 4))):
                content = tuple(toks[4 * j:4 * j + 4])
                if b in seen:
                    assert seen[b] == content
                else:
                    seen[b] = content

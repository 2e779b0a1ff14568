"""The native block manager (host only): allocation, reference counts, prefix
reuse, appends, eviction of cached blocks, and the tables / slots it builds."""
import numpy as np
import pytest

import oracle
import paged_kv_gqa_mapping_amd as pkv

needs_lib = pytest.mark.skipif(not __import__("os").path.exists(pkv.library_path), reason="libpkv.so not built")
pytestmark = needs_lib


def test_allocate_free_and_refcounts():
    bm = pkv.BlockManager(8, 4)
    assert bm.allocate(1, list(range(9))) == 0
    t1 = bm.block_table(1)
    assert len(t1) == 3 and bm.num_free_blocks == 5
    assert all(bm.refcount(b) == 1 for b in t1)
    bm.free(1)
    assert bm.num_free_blocks == 8 and all(bm.refcount(b) == 0 for b in range(8))
    with pytest.raises(pkv.PkvError):
        bm.free(1)


def test_prefix_blocks_are_shared_and_partial_blocks_are_not():
    bm = pkv.BlockManager(16, 4)
    a = [5, 6, 7, 8, 9, 10, 11, 12, 13]       # 2 full blocks + 1 token
    b = [5, 6, 7, 8, 9, 10, 11, 12, 13, 14]   # same 2 full blocks, different tail
    assert bm.allocate(1, a) == 0
    assert bm.allocate(2, b) == 8             # both full blocks found in the cache
    ta, tb = bm.block_table(1), bm.block_table(2)
    assert list(ta[:2]) == list(tb[:2]) and ta[2] != tb[2]
    assert bm.refcount(ta[0]) == 2 and bm.refcount(ta[2]) == 1
    # a different first block breaks the chain even if later blocks are equal
    c = [0, 6, 7, 8, 9, 10, 11, 12]
    assert bm.allocate(3, c) == 0
    assert set(bm.block_table(3)).isdisjoint(ta)


def test_cached_blocks_survive_free_until_reused():
    bm = pkv.BlockManager(4, 2)
    bm.allocate(1, [1, 2, 3, 4])   # blocks for [1,2] and [3,4], both registered
    t1 = list(bm.block_table(1))
    bm.free(1)
    assert bm.num_free_blocks == 4
    assert bm.allocate(2, [1, 2, 3, 4, 9]) == 4   # both found although free
    assert list(bm.block_table(2))[:2] == t1
    bm.free(2)
    # four fresh blocks evict the cached ones (oldest free first)
    bm.allocate(3, [7, 7, 7, 7, 7, 7, 7, 7])
    bm.free(3)
    assert bm.allocate(4, [1, 2, 3, 4]) == 0


def test_append_fills_blocks_and_registers_them():
    bm = pkv.BlockManager(8, 4)
    bm.allocate(1, [1, 2, 3])
    slots = [bm.append(1, t) for t in (4, 5, 6, 7, 8, 9)]
    table = bm.block_table(1)
    assert bm.seq_len(1) == 9 and len(table) == 3
    assert slots == [oracle.slot_of(table, p, 4) for p in range(3, 9)]
    # the two blocks completed by appends are reusable as a prefix
    assert bm.allocate(2, [1, 2, 3, 4, 5, 6, 7, 8, 100]) == 8


def test_out_of_blocks_changes_nothing():
    bm = pkv.BlockManager(3, 4)
    bm.allocate(1, list(range(8)))
    assert not bm.can_allocate(list(range(100, 108)))
    with pytest.raises(pkv.OutOfBlocks):
        bm.allocate(2, list(range(100, 108)))
    assert bm.num_free_blocks == 1
    with pytest.raises(pkv.PkvError):
        bm.seq_len(2)
    assert bm.can_allocate([0, 1, 2, 3, 50])  # prefix hit + one fresh block
    bm.allocate(2, [0, 1, 2, 3, 50])
    assert bm.num_free_blocks == 0
    bm.append(2, 51)
    bm.append(2, 52)
    bm.append(2, 53)               # fills the tail block
    with pytest.raises(pkv.OutOfBlocks):
        bm.append(2, 54)           # would need a new block
    assert bm.seq_len(2) == 8


def test_prefix_cache_off_shares_nothing():
    bm = pkv.BlockManager(8, 2, prefix_cache=False)
    bm.allocate(1, [1, 2, 3, 4])
    assert bm.allocate(2, [1, 2, 3, 4]) == 0
    assert set(bm.block_table(1)).isdisjoint(bm.block_table(2))


def test_slot_mapping_and_padded_table():
    bm = pkv.BlockManager(32, 8)
    bm.allocate(7, list(range(30)))
    t = bm.block_table(7, width=6, pad=31)
    assert list(t[4:]) == [31, 31]
    s = bm.slot_mapping(7, 5, 20)
    assert list(s) == [oracle.slot_of(t, p, 8) for p in range(5, 25)]
    with pytest.raises(pkv.PkvError):
        bm.slot_mapping(7, 25, 10)
    with pytest.raises(pkv.PkvError):
        bm.block_table(7, width=2)


def test_create_rejects_slot_overflow():
    with pytest.raises(pkv.PkvError):
        pkv.BlockManager(1 << 24, 256)


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(0)
    bs, nb = 4, 64
    bm = pkv.BlockManager(nb, bs)
    live = {}
    order = []  # allocation order of the live sequences
    prefixes = [list(rng.integers(0, 50, size=8)) for _ in range(3)]
    next_id = 0
    preempted = 0
    for step in range(600):
        op = rng.random()
        if op < 0.35 or not live:
            toks = list(prefixes[rng.integers(0, 3)]) + list(rng.integers(0, 50, size=rng.integers(0, 10)))
            ok = bm.can_allocate(toks)
            try:
                bm.allocate(next_id, toks)
                assert ok
                live[next_id] = list(toks)
                order.append(next_id)
            except pkv.OutOfBlocks:
                assert not ok
                if live and rng.random() < 0.5:
                    # scheduler response: preempt the newest sequence, then retry once
                    victim, cached = bm.preempt()
                    assert victim == order[-1] and 0 <= cached <= len(live[victim])
                    order.pop()
                    del live[victim]
                    preempted += 1
                    if bm.can_allocate(toks):
                        bm.allocate(next_id, toks)
                        live[next_id] = list(toks)
                        order.append(next_id)
            next_id += 1
        elif op < 0.75:
            sid = list(live)[rng.integers(0, len(live))]
            t = int(rng.integers(0, 50))
            try:
                slot = bm.append(sid, t)
                live[sid].append(t)
                table = bm.block_table(sid)
                assert slot == oracle.slot_of(table, len(live[sid]) - 1, bs)
            except pkv.OutOfBlocks:
                pass
        else:
            sid = list(live)[rng.integers(0, len(live))]
            bm.free(sid)
            del live[sid]
            order.remove(sid)
        # invariants: refcounts equal the number of tables holding a block; shared
        # blocks are full blocks holding the same tokens in every holder
        holders = {}
        for sid, toks in live.items():
            table = bm.block_table(sid)
            assert bm.seq_len(sid) == len(toks) and len(table) == -(-len(toks) // bs)
            for j, b in enumerate(table):
                holders.setdefault(int(b), []).append(tuple(toks[j * bs:(j + 1) * bs]))
        for b in range(nb):
            assert bm.refcount(b) == len(holders.get(b, []))
        for b, contents in holders.items():
            if len(contents) > 1:
                assert len(set(contents)) == 1 and len(contents[0]) == bs
        assert bm.num_free_blocks == nb - len(holders)
    assert preempted > 0


def test_exhaust_preempt_retry():
    """Pool runs out -> the most recently allocated sequence is preempted (its
    blocks freed, registered blocks kept in the prefix cache) -> the allocation
    that failed succeeds; the victim re-allocated later reuses what the cache
    still holds (page "Nano-vLLM Architecture and Performance", Key Features,
    preemption on exhausted KV cache)."""
    bs = 4
    bm = pkv.BlockManager(10, bs)
    shared = [1, 2, 3, 4, 5, 6, 7, 8]                      # two full blocks
    p1 = shared + [9, 10]                                   # 3 blocks, 2 shared later
    p2 = shared + [20, 21, 22]                              # shares p1's 2 full blocks
    p3 = [30 + i for i in range(13)]                        # 4 blocks (3 full + 1 partial)
    assert bm.allocate(1, p1) == 0
    assert bm.allocate(2, p2) == 8
    assert bm.allocate(3, p3) == 0
    assert bm.num_free_blocks == 10 - 3 - 1 - 4
    p4 = [50 + i for i in range(12)]                        # needs 3 blocks, 2 are free
    assert not bm.can_allocate(p4)
    with pytest.raises(pkv.OutOfBlocks):
        bm.allocate(4, p4)
    assert bm.num_free_blocks == 2                          # the failed call changed nothing
    t3 = bm.block_table(3)
    victim, cached = bm.preempt()
    assert victim == 3                                      # the most recent allocation
    assert cached == 12                                     # its 3 full blocks stay registered
    assert bm.num_free_blocks == 6 and all(bm.refcount(b) == 0 for b in t3)
    with pytest.raises(pkv.PkvError):
        bm.seq_len(3)
    assert bm.allocate(4, p4) == 0                          # the retry succeeds
    # the shared prefix is untouched by the preemption
    t1, t2 = bm.block_table(1), bm.block_table(2)
    assert list(t1[:2]) == list(t2[:2]) and bm.refcount(t1[0]) == 2
    # p4 took 3 of the 6 free blocks, oldest first: the 2 never-used blocks and the
    # victim's partial block (freed first, being its last); its 3 full blocks stay cached
    assert sorted(set(bm.block_table(4)) & set(t3)) == [t3[3]]
    bm.free(1)                                              # returns p1's own tail block only
    assert bm.refcount(t1[0]) == 1 and bm.num_free_blocks == 4
    assert bm.allocate(3, p3) == 12                         # the victim comes back, 12 tokens cached
    assert list(bm.block_table(3)[:3]) == list(t3[:3])
    assert bm.num_free_blocks == 0


def test_append_exhaustion_preempts_the_newest():
    bm = pkv.BlockManager(4, 2)
    bm.allocate(1, [1, 2])                                  # 1 full block
    bm.allocate(2, [3, 4, 5])                               # 2 blocks
    bm.allocate(3, [6])                                     # 1 block; pool now empty
    assert bm.num_free_blocks == 0
    bm.append(3, 7)                                         # fills seq 3's block: no new block
    with pytest.raises(pkv.OutOfBlocks):
        bm.append(1, 8)                                     # seq 1 needs a new block
    assert bm.seq_len(1) == 2
    victim, cached = bm.preempt()
    assert victim == 3 and cached == 2                      # its block was completed by the append
    slot = bm.append(1, 8)
    assert slot // 2 in bm.block_table(1) and bm.seq_len(1) == 3
    victim, _ = bm.preempt()
    assert victim == 2
    victim, _ = bm.preempt()
    assert victim == 1
    with pytest.raises(pkv.PkvError):
        bm.preempt()                                        # nothing left
    assert bm.num_free_blocks == 4

"""C++ allocator (through the C ABI) == pool oracle, bit for bit -- CPU only.

Compares block tables, lengths, slots, copy pairs, the free stack, the
counters and the error class after every operation, on the course
notebook's page trace and on random operation sequences.
"""

import json
import os
import random

import numpy as np
import pytest

import paged_kv_cache_202_amd as pkv
from oracle.pool import PagedPool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvnb_contract.json")


def snapshot(pool: pkv.PagedKVPool, names=None):
    ids = pool.seq_ids()
    seqs = {}
    for i in ids:
        key = names[i] if names else str(i)
        seqs[key] = {"length": pool.seq_length(i), "blocks": list(pool.page_table(i))}
    snap = {"sequences": dict(sorted(seqs.items(), key=lambda kv: repr(kv[0])))}
    snap.update(pool.stats())
    return snap


def test_notebook_trace_through_the_abi():
    trace = json.load(open(GOLDEN))["paged"]["trace"]
    names = {0: "A", 1: "B"}
    pool = pkv.PagedKVPool(8, 4)
    pool.seq_create(0)
    slots, cow = pool.alloc(0, 6)
    assert slots.tolist() == [0, 1, 2, 3, 4, 5] and cow == []
    pool.validate()
    assert snapshot(pool, names) == trace["after_a"]
    pool.fork(0, 1, 6)
    assert snapshot(pool, names) == trace["after_share"]
    slots, cow = pool.alloc(1, 3)
    assert cow == [(1, 2)] and slots.tolist() == [10, 11, 12]
    assert snapshot(pool, names) == trace["after_b_append"]
    pool.free(0)
    pool.validate()
    assert snapshot(pool, names) == trace["after_a_release"]


def test_error_classes_and_no_partial_mutation():
    pool = pkv.PagedKVPool(2, 4)
    with pytest.raises(KeyError):
        pool.alloc(99, 1)
    pool.seq_create(1)
    with pytest.raises(pkv.SequenceExists):
        pool.seq_create(1)
    pool.alloc(1, 6)
    before = (snapshot(pool), pool.free_stack())
    with pytest.raises(MemoryError):
        pool.alloc(1, 3)
    assert (snapshot(pool), pool.free_stack()) == before
    with pytest.raises(pkv.InvalidArgument):
        pool.fork(1, 2, 7)
    with pytest.raises(pkv.InvalidArgument):
        pool.alloc(1, -1)
    with pytest.raises(pkv.InvalidArgument):
        pool.truncate(1, 7)
    with pytest.raises(pkv.InvalidArgument):
        pkv.PagedKVPool(3, 2, initial_free_stack=[0, 0, 1])
    with pytest.raises(pkv.InvalidArgument):
        pkv.PagedKVPool(1 << 28, 16)  # slots would overflow int32
    pool.validate()


def test_lecture_pins_through_the_abi():
    pool = pkv.PagedKVPool(128, 16)
    pool.seq_create(7)
    pool.alloc(7, 2048)
    assert len(pool.page_table(7)) == 128
    assert pool.stats()["internal_waste_tokens"] == 0
    with pytest.raises(MemoryError):
        pool.alloc(7, 1)
    pool.free(7)
    assert len(pool.free_stack()) == 128


def test_block_tables_pad_and_reject():
    pool = pkv.PagedKVPool(16, 4, initial_free_stack=np.random.default_rng(3).permutation(16))
    for s, n in ((0, 5), (1, 9), (2, 1)):
        pool.seq_create(s)
        pool.alloc(s, n)
    tables, lens = pool.block_tables([2, 0, 1], 3)
    assert lens.tolist() == [1, 5, 9]
    assert tables[0, 1:].tolist() == [-1, -1] and tables[1, 2] == -1
    assert tables[2].tolist() == list(pool.page_table(1))
    with pytest.raises(pkv.InvalidArgument):
        pool.block_tables([1], 2)


def test_batch_alloc_matches_sequential_appends():
    stack = np.random.default_rng(9).permutation(12)
    a = pkv.PagedKVPool(12, 4, initial_free_stack=stack)
    o = PagedPool(12, 4, initial_free_stack=stack.tolist())
    for s in range(3):
        a.seq_create(s)
        o.create(s)
    a.fork(0, 3, 0)
    o.share_prefix(0, 3, 0)
    slots, pairs = a.alloc_batch([0, 1, 2, 3], [3, 5, 0, 2])
    expect = []
    for s, n in zip([0, 1, 2, 3], [3, 5, 0, 2]):
        expect += o.append(s, n)[0]
    assert slots.tolist() == expect and pairs.shape == (0, 2)
    assert a.last_batch_done == 4


def test_failing_batch_changes_nothing():
    """[KVNB §5] preflight: a batch that runs out of blocks at its k-th member
    leaves every table, count and the free stack as they were (the members
    before it are not applied either)."""
    stack = np.random.default_rng(9).permutation(12)
    a = pkv.PagedKVPool(12, 4, initial_free_stack=stack)
    for s in range(3):
        a.seq_create(s)
    a.alloc(0, 6)          # blocks for 6 tokens: the last one partial
    a.fork(0, 3, 6)        # ... and shared
    before = (snapshot(a), a.free_stack())
    # 10 free blocks. First batch: sequence 1 takes 3, sequence 3 a copy of
    # the shared tail + 1, sequence 2 six (11). Last: sequence 3 copies, so
    # sequence 0's tail is no longer shared and needs no copy; then sequence
    # 3 grows by 10 blocks (11).
    for ids, ns in (([1, 3, 2], [12, 6, 21]), ([1, 2], [3, 40]), ([3, 0, 3], [2, 2, 40])):
        with pytest.raises(MemoryError):
            a.alloc_batch(ids, ns)
        assert a.last_batch_done == 0
        assert (snapshot(a), a.free_stack()) == before
        a.validate()
    with pytest.raises(KeyError):  # an unknown id late in the batch
        a.alloc_batch([1, 2, 99], [1, 1, 1])
    assert (snapshot(a), a.free_stack()) == before
    with pytest.raises(pkv.InvalidArgument):
        a.alloc_batch([1, 2], [1, -1])
    assert (snapshot(a), a.free_stack()) == before
    # the same batch fits once it asks for exactly the free blocks
    a.alloc_batch([1, 3, 2], [12, 6, 20])
    assert a.stats()["free_blocks"] == 0
    a.validate()


@pytest.mark.parametrize("seed", range(30))
def test_random_batches_all_or_nothing(seed):
    """Random batches over shared partial tails (copies whose counts change
    within the batch) and repeated ids: a batch succeeds exactly when the
    same appends one by one would all succeed, with the same slots, pairs
    and free stack; otherwise nothing changes."""
    import copy

    rnd = random.Random(7000 + seed)
    bs = rnd.choice([2, 4, 16])
    nblocks = rnd.randint(6, 40)
    stack = np.random.default_rng(seed).permutation(nblocks).tolist()
    lib = pkv.PagedKVPool(nblocks, bs, initial_free_stack=stack)
    ora = PagedPool(nblocks, bs, initial_free_stack=stack)
    lib.seq_create(0)
    ora.create(0)
    n0 = rnd.randint(1, 3 * bs)
    lib.alloc(0, n0)
    ora.append(0, n0)
    live = [0]
    for c in range(1, rnd.randint(2, 6)):
        p = rnd.randint(0, ora.sequence_length(0))
        lib.fork(0, c, p)
        ora.share_prefix(0, c, p)
        live.append(c)
    for _ in range(12):
        ids = [rnd.choice(live) for _ in range(rnd.randint(1, 6))]
        ns = [rnd.randint(0, 2 * bs) for _ in ids]
        trial = copy.deepcopy(ora)
        try:
            expect_slots, expect_pairs = [], []
            for s, n in zip(ids, ns):
                sl, cw = trial.append(s, n)
                expect_slots += sl
                expect_pairs += cw
        except MemoryError:
            before = (snapshot(lib), lib.free_stack())
            with pytest.raises(MemoryError):
                lib.alloc_batch(ids, ns)
            assert (snapshot(lib), lib.free_stack()) == before
        else:
            slots, pairs = lib.alloc_batch(ids, ns)
            assert slots.tolist() == expect_slots
            assert [tuple(x) for x in pairs.tolist()] == expect_pairs
            ora = trial
        lib.validate()
        assert lib.free_stack() == ora.free
        assert snapshot(lib) == ora.snapshot()


@pytest.mark.parametrize("seed", range(40))
def test_random_operations_bit_exact(seed):
    rnd = random.Random(1000 + seed)
    bs = rnd.choice([1, 2, 4, 16])
    nblocks = rnd.randint(2, 48)
    stack = np.random.default_rng(seed).permutation(nblocks).tolist() if seed % 2 else None
    lib = pkv.PagedKVPool(nblocks, bs, initial_free_stack=stack)
    ora = PagedPool(nblocks, bs, initial_free_stack=stack)
    live, next_id = [], 0
    for step in range(250):
        op = rnd.random()
        if op < 0.12 or not live:
            lib.seq_create(next_id)
            ora.create(next_id)
            live.append(next_id)
            next_id += 1
        elif op < 0.55:
            s = rnd.choice(live)
            n = rnd.randint(0, 3 * bs + 2)
            try:
                expect = ora.append(s, n)
            except MemoryError:
                with pytest.raises(MemoryError):
                    lib.alloc(s, n)
            else:
                slots, cow = lib.alloc(s, n)
                assert slots.tolist() == expect[0] and cow == expect[1]
        elif op < 0.7:
            s = rnd.choice(live)
            p = rnd.randint(0, ora.sequence_length(s))
            lib.fork(s, next_id, p)
            ora.share_prefix(s, next_id, p)
            live.append(next_id)
            next_id += 1
        elif op < 0.85:
            s = rnd.choice(live)
            n = rnd.randint(0, ora.sequence_length(s))
            lib.truncate(s, n)
            ora.truncate(s, n)
        else:
            s = rnd.choice(live)
            lib.free(s)
            ora.release(s)
            live.remove(s)
        lib.validate()
        assert lib.free_stack() == ora.free
        assert snapshot(lib) == ora.snapshot()
    if live:
        tables, lens = lib.block_tables(live, max(1, max(len(ora.page_table(s)) for s in live)))
        et, el = ora.block_tables(live, tables.shape[1])
        assert tables.tolist() == et and lens.tolist() == el

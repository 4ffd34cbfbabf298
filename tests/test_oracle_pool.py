"""Pins for the pool oracle (``oracle.pool``) -- CPU only.

Each pin comes from outside the oracle: values the course notebook prints
(its SHA-checked contract and its asserts), closed forms, or a brute-force
content model that checks what the allocator must guarantee (every sequence
reads back exactly the tokens written to it or inherited from its parent).
"""

import json
import math
import os
import random

import numpy as np
import pytest

from oracle.geometry import expected_paged_waste, naive_preallocation_waste
from oracle.pool import PagedPool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvnb_contract.json")


@pytest.fixture(scope="module")
def contract():
    with open(GOLDEN) as f:
        return json.load(f)


def test_notebook_trace_snapshots(contract):
    """[KVNB §6] page trace at block size 4 with 8 blocks, all four snapshots."""
    trace = contract["paged"]["trace"]
    pool = PagedPool(8, 4)
    pool.create("A")
    pool.append("A", 6)
    pool.validate()
    assert pool.snapshot() == trace["after_a"]
    pool.share_prefix("A", "B", 6)
    pool.validate()
    assert pool.snapshot() == trace["after_share"]
    pool.append("B", 3)
    pool.validate()
    assert pool.snapshot() == trace["after_b_append"]
    assert pool.page_table("A")[-1] != pool.page_table("B")[1]
    pool.release("A")
    pool.validate()
    assert pool.snapshot() == trace["after_a_release"]


def test_trace_slots_and_cow_pairs():
    """Slots and the copy pair implied by the same trace (block*bs + offset)."""
    pool = PagedPool(8, 4)
    pool.create("A")
    slots, cow = pool.append("A", 6)
    assert slots == [0, 1, 2, 3, 4, 5] and cow == []
    pool.share_prefix("A", "B", 6)
    slots, cow = pool.append("B", 3)
    # B's shared partial block 1 is replaced by block 2 (offsets 2, 3), then
    # block 3 takes the last token at offset 0.
    assert cow == [(1, 2)]
    assert slots == [2 * 4 + 2, 2 * 4 + 3, 3 * 4 + 0]


def test_negative_cases_leave_state_unchanged():
    """[KVNB §9] unknown id, duplicate id, OOM without mutation, prefix > length."""
    pool = PagedPool(2, 4)
    with pytest.raises(KeyError):
        pool.append("missing", 1)
    pool.create("x")
    with pytest.raises(ValueError):
        pool.create("x")
    pool.append("x", 6)
    before = pool.snapshot()
    free_before = list(pool.free)
    with pytest.raises(MemoryError):
        pool.append("x", 3)
    assert pool.snapshot() == before and pool.free == free_before
    with pytest.raises(ValueError):
        pool.share_prefix("x", "y", 7)
    with pytest.raises(ValueError):
        pool.append("x", -1)
    with pytest.raises(TypeError):
        pool.create(["unhashable"])
    pool.validate()


@pytest.mark.parametrize("action,payload", [("release", 1), ("append", 5)])
def test_short_child_survives_parent(action, payload):
    """[KVNB §9] a short child keeps its token when the parent leaves or copies."""
    pool = PagedPool(4, 4)
    pool.create("parent")
    pool.append("parent", 3)
    pool.share_prefix("parent", "child", 1)
    if action == "release":
        pool.release("parent")
    else:
        pool.append("parent", 1)
    assert pool.stats()["physical_payload_tokens"] == payload
    pool.append("child", 2)
    pool.validate()


def test_lecture_core_private_pages():
    """[KVNB] lecture core: 2048 tokens fill 128 blocks; 2049 is refused unchanged."""
    pool = PagedPool(128, 16)
    pool.create("a")
    pool.append_to("a", 2048)
    assert len(pool.page_table("a")) == 128
    assert pool.stats()["internal_waste_tokens"] == 0
    before = (list(pool.free), pool.snapshot())
    with pytest.raises(MemoryError):
        pool.append_to("a", 2049)
    assert before == (list(pool.free), pool.snapshot())
    with pytest.raises(ValueError):
        pool.append_to("a", 10)  # cannot shorten
    pool.release("a")
    assert len(pool.free) == 128


def test_waste_closed_forms(contract):
    """[KVNB §6] expected paged waste and naive reservation waste."""
    paged = contract["paged"]
    assert math.isclose(expected_paged_waste(2048, 16),
                        paged["expected_paged_waste_fraction"], abs_tol=1e-12)
    assert math.isclose(naive_preallocation_waste(32768, 2048),
                        paged["naive_waste_fraction"], abs_tol=1e-12)


def test_demo_tails_below_block_size():
    """[KVNB demo] Demo 1: 500 lengths in [64, 4096]; every tail wastes < 16 slots."""
    rng = np.random.default_rng(20260801)
    lengths = rng.integers(64, 4097, size=500)
    pool = PagedPool(int(sum((lengths + 15) // 16)), 16)
    for i, n in enumerate(lengths):
        pool.create(i)
        pool.append(i, int(n))
    st = pool.stats()
    assert st["free_blocks"] == 0
    assert st["internal_waste_tokens"] == int(sum(-(-lengths // 16) * 16 - lengths))
    for i, n in enumerate(lengths):
        assert len(pool.page_table(i)) * 16 - int(n) < 16
    pool.validate()


def test_custom_free_stack_pops_from_end():
    pool = PagedPool(4, 2, initial_free_stack=[2, 0, 3, 1])
    pool.create(0)
    slots, _ = pool.append(0, 3)
    assert pool.page_table(0) == (1, 3)
    assert slots == [2, 3, 6]
    with pytest.raises(ValueError):
        PagedPool(3, 2, initial_free_stack=[0, 0, 1])


def test_truncate_keeps_shared_partial_block():
    """[KVNB] exercise: truncate returns blocks past the length; shared tail stays."""
    pool = PagedPool(8, 4)
    pool.create("p")
    pool.append("p", 10)  # blocks 0, 1, 2 (2 in the last)
    pool.share_prefix("p", "c", 6)  # c: blocks 0, 1 (1 shared, partial for c)
    pool.truncate("p", 5)  # p keeps 0, 1; block 2 goes back
    assert pool.page_table("p") == (0, 1)
    assert pool.free[-1] == 2
    pool.validate()
    _, cow = pool.append("p", 1)  # block 1 shared and partial -> copy
    assert cow == [(1, 2)]  # the block freed by the truncate is on top
    pool.validate()
    with pytest.raises(ValueError):
        pool.truncate("p", 7)


class ContentModel:
    """Brute force: device memory as slot -> label; checks what each sequence reads."""

    def __init__(self, pool: PagedPool):
        self.pool = pool
        self.mem = {}
        self.expect = {}  # seq -> list of labels of its logical tokens
        self.next_label = 0

    def append(self, s, n):
        slots, cow = self.pool.append(s, n)
        bs = self.pool.block_size
        for src, dst in cow:  # the device copies whole blocks before writing
            for off in range(bs):
                if src * bs + off in self.mem:
                    self.mem[dst * bs + off] = self.mem[src * bs + off]
        labels = list(range(self.next_label, self.next_label + n))
        self.next_label += n
        assert len(slots) == n and len(set(slots)) == n
        for slot, lab in zip(slots, labels):
            self.mem[slot] = lab
        self.expect[s] = self.expect.get(s, []) + labels

    def fork(self, src, dst, p):
        self.pool.share_prefix(src, dst, p)
        self.expect[dst] = list(self.expect[src][:p])

    def release(self, s):
        self.pool.release(s)
        del self.expect[s]

    def truncate(self, s, n):
        self.pool.truncate(s, n)
        self.expect[s] = self.expect[s][:n]

    def check(self):
        bs = self.pool.block_size
        for s, labels in self.expect.items():
            table = self.pool.page_table(s)
            got = [self.mem.get(table[t // bs] * bs + t % bs) for t in range(len(labels))]
            assert got == labels, f"sequence {s} reads back other tokens"


@pytest.mark.parametrize("seed", range(12))
def test_random_ops_content_and_invariants(seed):
    rnd = random.Random(seed)
    bs = rnd.choice([1, 2, 4, 16])
    nblocks = rnd.randint(4, 40)
    stack = np.random.default_rng(seed).permutation(nblocks).tolist() if seed % 2 else None
    pool = PagedPool(nblocks, bs, initial_free_stack=stack)
    model = ContentModel(pool)
    live = []
    next_id = 0
    for _ in range(300):
        op = rnd.random()
        try:
            if op < 0.15 or not live:
                pool.create(next_id)
                model.expect[next_id] = []
                live.append(next_id)
                next_id += 1
            elif op < 0.55:
                s = rnd.choice(live)
                before = pool.snapshot()
                try:
                    model.append(s, rnd.randint(0, 3 * bs + 1))
                except MemoryError:
                    assert pool.snapshot() == before
            elif op < 0.7:
                s = rnd.choice(live)
                p = rnd.randint(0, pool.sequence_length(s))
                model.fork(s, next_id, p)
                live.append(next_id)
                next_id += 1
            elif op < 0.85:
                s = rnd.choice(live)
                model.truncate(s, rnd.randint(0, pool.sequence_length(s)))
            else:
                s = rnd.choice(live)
                model.release(s)
                live.remove(s)
        finally:
            pool.validate()
        model.check()

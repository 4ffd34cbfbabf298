"""Float64-free integer oracle: the paged block pool (test infrastructure).

Restates the page pool of [KVNB §5] ("Page pool: prefix sharing and
copy-on-write") in plain Python, and adds the two outputs the pool on that
page leaves implicit: the slot of every appended token (slot = physical block
id * block size + offset, [NeuralOps] "Block Table" / continuous-batching
"slot mapping") and the copy-on-write pairs (old block, replacement) that a
device copy must perform.

Rules taken from the page, in its order:

* The free list starts as the ids N-1, ..., 0 and blocks are taken from its
  end, so block 0 is handed out first. A caller may supply another initial
  order (a seeded shuffle); it is still taken from the end.
* append(seq, n): check n >= 0 and that seq exists; count the blocks needed
  (one extra if the last block is partial and shared, then enough new blocks
  for what does not fit in the last block's room); refuse with MemoryError,
  changing nothing, if fewer are free; then, if the last block is partial:
  copy it first when it is shared (drop one reference, take a replacement),
  fill its room; then take new blocks for the rest.
* share_prefix(src, dst, p): dst gets src's first ceil(p / bs) blocks, each
  gaining one reference; dst's length is p.
* release(seq): drop one reference per table entry in table order; a block
  whose count reaches zero goes back on the end of the free list.
* Fill of a block: the most any live sequence stores in it,
  min(bs, len - j*bs) for table position j; counters follow from fills.
* validate(): the invariants of [KVNB §5] ``validate``.

``truncate`` is the exercise of [KVNB] "Exercises" (truncate for the page
pool): blocks past the new length are released in table order; a shared
partial block keeps its references, so the next append copies it.
"""

from __future__ import annotations

import math
from typing import Hashable, Iterable


class PoolError(Exception):
    """Base for the pool's error classes."""


class PagedPool:
    """Plain restatement of the page-pool simulator, with slots and COW pairs."""

    def __init__(self, total_blocks: int, block_size: int = 16,
                 initial_free_stack: Iterable[int] | None = None) -> None:
        if not _is_int(total_blocks) or total_blocks <= 0:
            raise ValueError("total_blocks must be a positive integer")
        if not _is_int(block_size) or block_size <= 0:
            raise ValueError("block_size must be a positive integer")
        self.total_blocks = total_blocks
        self.block_size = block_size
        if initial_free_stack is None:
            stack = list(range(total_blocks - 1, -1, -1))
        else:
            stack = [int(b) for b in initial_free_stack]
            if sorted(stack) != list(range(total_blocks)):
                raise ValueError("initial free stack must be a permutation of 0..N-1")
        self.free = stack  # taken from the end
        self.refs = [0] * total_blocks
        self.seqs: dict[Hashable, list] = {}  # id -> [length, blocks]

    # -- queries --------------------------------------------------------
    def _seq(self, seq_id):
        if seq_id not in self.seqs:
            raise KeyError(f"unknown sequence: {seq_id!r}")
        return self.seqs[seq_id]

    def sequence_length(self, seq_id) -> int:
        return self._seq(seq_id)[0]

    def page_table(self, seq_id) -> tuple[int, ...]:
        return tuple(self._seq(seq_id)[1])

    def fills(self) -> list[int]:
        """Per physical block: the most tokens any live sequence keeps in it."""
        bs = self.block_size
        fill = [0] * self.total_blocks
        for length, blocks in self.seqs.values():
            for j, b in enumerate(blocks):
                fill[b] = max(fill[b], min(bs, length - j * bs))
        return fill

    def stats(self) -> dict[str, int]:
        fill = self.fills()
        allocated = self.total_blocks - len(self.free)
        capacity = allocated * self.block_size
        payload = sum(f for b, f in enumerate(fill) if self.refs[b])
        logical = sum(length for length, _ in self.seqs.values())
        return {
            "allocated_blocks": allocated,
            "free_blocks": len(self.free),
            "physical_capacity_tokens": capacity,
            "physical_payload_tokens": payload,
            "logical_tokens": logical,
            "internal_waste_tokens": capacity - payload,
            "sharing_savings_tokens": logical - payload,
        }

    def snapshot(self) -> dict:
        items = sorted(self.seqs.items(), key=lambda kv: repr(kv[0]))
        snap = {"sequences": {str(k): {"length": v[0], "blocks": list(v[1])}
                              for k, v in items}}
        snap.update(self.stats())
        return snap

    def block_tables(self, seq_ids, max_blocks: int):
        """Row-major [n, max_blocks] int table padded with -1, and lengths."""
        tables, lens = [], []
        for s in seq_ids:
            length, blocks = self._seq(s)
            if len(blocks) > max_blocks:
                raise ValueError("max_blocks is smaller than a page table")
            tables.append(list(blocks) + [-1] * (max_blocks - len(blocks)))
            lens.append(length)
        return tables, lens

    # -- mutations ------------------------------------------------------
    def create(self, seq_id) -> None:
        hash(seq_id)  # raises TypeError for unhashable ids
        if seq_id in self.seqs:
            raise ValueError(f"sequence already exists: {seq_id!r}")
        self.seqs[seq_id] = [0, []]

    def blocks_needed(self, seq_id, n: int) -> int:
        length, blocks = self._seq(seq_id)
        if n == 0:
            return 0
        bs = self.block_size
        used_in_last = length % bs
        room = 0
        extra = 0
        if blocks and used_in_last:
            room = bs - used_in_last
            if self.refs[blocks[-1]] > 1:
                extra = 1  # private copy of the shared partial last block
        rest = max(0, n - room)
        return extra + math.ceil(rest / bs)

    def _take(self) -> int:
        b = self.free.pop()
        self.refs[b] = 1
        return b

    def append(self, seq_id, n: int):
        """Grow ``seq_id`` by ``n`` tokens; return (slots, cow_pairs)."""
        if not _is_int(n) or n < 0:
            raise ValueError("token count must be a non-negative integer")
        state = self._seq(seq_id)
        need = self.blocks_needed(seq_id, n)
        if need > len(self.free):
            raise MemoryError(f"need {need} free blocks, {len(self.free)} remain")
        slots: list[int] = []
        cow: list[tuple[int, int]] = []
        if n == 0:
            return slots, cow
        bs = self.block_size
        length, blocks = state
        used_in_last = length % bs
        if blocks and used_in_last:
            last = blocks[-1]
            if self.refs[last] > 1:
                self.refs[last] -= 1
                fresh = self._take()
                blocks[-1] = fresh
                cow.append((last, fresh))
            take = min(n, bs - used_in_last)
            for k in range(take):
                slots.append(blocks[-1] * bs + used_in_last + k)
            length += take
            n -= take
        while n:
            take = min(n, bs)
            b = self._take()
            blocks.append(b)
            for k in range(take):
                slots.append(b * bs + k)
            length += take
            n -= take
        state[0] = length
        return slots, cow

    def append_to(self, seq_id, total: int):
        """Grow a sequence to ``total`` tokens (refusing to shrink it)."""
        if not _is_int(total) or total < 0:
            raise ValueError("total must be a non-negative integer")
        cur = self.sequence_length(seq_id)
        if total < cur:
            raise ValueError("append_to cannot shorten a sequence")
        return self.append(seq_id, total - cur)

    def share_prefix(self, src, dst, prefix: int) -> None:
        length, blocks = self._seq(src)
        if not _is_int(prefix) or prefix < 0:
            raise ValueError("prefix must be a non-negative integer")
        if prefix > length:
            raise ValueError("prefix exceeds source length")
        if dst in self.seqs:
            raise ValueError(f"target sequence already exists: {dst!r}")
        hash(dst)
        count = math.ceil(prefix / self.block_size)
        shared = list(blocks[:count])
        for b in shared:
            self.refs[b] += 1
        self.seqs[dst] = [prefix, shared]

    def release(self, seq_id) -> None:
        _, blocks = self._seq(seq_id)
        for b in blocks:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free.append(b)
        del self.seqs[seq_id]

    def truncate(self, seq_id, new_length: int) -> None:
        state = self._seq(seq_id)
        if not _is_int(new_length) or not 0 <= new_length <= state[0]:
            raise ValueError("new length must lie in [0, length]")
        keep = math.ceil(new_length / self.block_size)
        for b in state[1][keep:]:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free.append(b)
        del state[1][keep:]
        state[0] = new_length

    # -- invariants -----------------------------------------------------
    def validate(self) -> None:
        n = self.total_blocks
        if len(set(self.free)) != len(self.free):
            raise AssertionError("free list contains duplicates")
        if any(b < 0 or b >= n for b in self.free):
            raise AssertionError("free list contains an invalid block id")
        expect = [0] * n
        for length, blocks in self.seqs.values():
            if length < 0:
                raise AssertionError("negative sequence length")
            if len(blocks) != math.ceil(length / self.block_size):
                raise AssertionError("page-table length does not match length")
            if len(set(blocks)) != len(blocks):
                raise AssertionError("a sequence references a block twice")
            for b in blocks:
                if b < 0 or b >= n:
                    raise AssertionError("page table holds an invalid block id")
                expect[b] += 1
        free = set(self.free)
        fill = self.fills()
        for b in range(n):
            if self.refs[b] != expect[b]:
                raise AssertionError("reference count does not match page tables")
            if self.refs[b] == 0:
                if b not in free or fill[b] != 0:
                    raise AssertionError("unreferenced block is not clean and free")
            else:
                if b in free:
                    raise AssertionError("referenced block is on the free list")
                if not 1 <= fill[b] <= self.block_size:
                    raise AssertionError("referenced block has an invalid fill")
        st = self.stats()
        if st["logical_tokens"] < st["physical_payload_tokens"]:
            raise AssertionError("physical payload exceeds logical payload")


def _is_int(x) -> bool:
    return isinstance(x, int) and not isinstance(x, bool)

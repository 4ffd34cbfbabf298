"""Integer oracle: the paged block pool (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module; the library never does.

What it models is the page pool of the course page "Module 10. KV Caches and
Efficient Inference", notebook "KV cache and serving: bytes, pages, and
ceilings", section 5 "Page pool: prefix sharing and copy-on-write" (cited
below as [KVNB §5]), plus the two outputs that pool leaves implicit: the slot
of every appended token (block id * block size + offset, the slot mapping of
"NeuralOps v1.3.4", Paged KV Cache Engine) and the copy-on-write pairs (old
block, private replacement) that a device copy must carry out.

The state is written as rules rather than as a procedure:

* A sequence of length L owns a table of exactly ceil(L / bs) block ids; its
  token t lives in slot table[t // bs] * bs + t % bs.
* A block's reference count is the number of table entries naming it; a block
  is on the free stack exactly when nothing names it. The stack starts as
  N-1, ..., 0 (or a caller's permutation) and its top (the end of the list)
  is handed out next.
* Growing a sequence from L to L' = L + n tokens needs ceil(L'/bs) - ceil(L/bs)
  new table entries, plus one private replacement when n > 0 and the last
  block is partial (L % bs != 0) and named by another table too ([KVNB §5]:
  a writer into a shared partial block copies it first). The whole count is
  checked against the free stack before anything changes, so a refused append
  leaves the pool as it was ([KVNB §5] preflight). The replacement is taken
  first, then the new entries in table order.
* Forking a child with a prefix of p tokens gives it the parent's first
  ceil(p / bs) entries; releasing or truncating drops entries (in table order),
  and blocks nobody names any more go back on the stack in that order.
* A block's fill is the largest number of tokens any table keeps in it; the
  counters of [KVNB §5] follow from the fills.

``truncate`` is the exercise of the same page ("Exercises": truncate for the
page pool): entries past ceil(new_length / bs) are dropped; a kept shared
partial block stays shared, so the next append copies it.
"""

from __future__ import annotations

from typing import Hashable, Iterable


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _is_int(x) -> bool:
    return isinstance(x, int) and not isinstance(x, bool)


class PagedPool:
    """The page pool with slots and copy-on-write pairs, in plain Python."""

    def __init__(self, total_blocks: int, block_size: int = 16,
                 initial_free_stack: Iterable[int] | None = None) -> None:
        if not _is_int(total_blocks) or total_blocks <= 0:
            raise ValueError("the pool needs a positive whole number of blocks")
        if not _is_int(block_size) or block_size <= 0:
            raise ValueError("block size must be a positive whole number")
        self.total_blocks = total_blocks
        self.block_size = block_size
        if initial_free_stack is None:
            order = list(reversed(range(total_blocks)))
        else:
            order = [int(b) for b in initial_free_stack]
            if sorted(order) != list(range(total_blocks)):
                raise ValueError("a custom free stack must hold each block id once")
        self.free = order  # the end of the list is handed out next
        self.refs = [0] * total_blocks
        self._len: dict[Hashable, int] = {}
        self._table: dict[Hashable, list[int]] = {}

    # -- reading the state ---------------------------------------------
    def _known(self, seq_id) -> None:
        if seq_id not in self._len:
            raise KeyError(f"no sequence with id {seq_id!r}")

    def sequence_length(self, seq_id) -> int:
        self._known(seq_id)
        return self._len[seq_id]

    def page_table(self, seq_id) -> tuple[int, ...]:
        self._known(seq_id)
        return tuple(self._table[seq_id])

    def slot(self, seq_id, t: int) -> int:
        """Physical slot of logical token t of a sequence."""
        bs = self.block_size
        return self._table[seq_id][t // bs] * bs + t % bs

    def fills(self) -> list[int]:
        """Per block: the most tokens that any table keeps in it."""
        bs = self.block_size
        fill = [0] * self.total_blocks
        for seq_id, table in self._table.items():
            length = self._len[seq_id]
            for j, b in enumerate(table):
                fill[b] = max(fill[b], min(bs, length - j * bs))
        return fill

    def stats(self) -> dict[str, int]:
        fill = self.fills()
        n_free = len(self.free)
        allocated = self.total_blocks - n_free
        payload = sum(fill[b] for b in range(self.total_blocks) if self.refs[b] > 0)
        logical = sum(self._len.values())
        return {
            "allocated_blocks": allocated,
            "free_blocks": n_free,
            "physical_capacity_tokens": allocated * self.block_size,
            "physical_payload_tokens": payload,
            "logical_tokens": logical,
            "internal_waste_tokens": allocated * self.block_size - payload,
            "sharing_savings_tokens": logical - payload,
        }

    def snapshot(self) -> dict:
        """Sequences (sorted by the repr of their ids) and the counters."""
        ids = sorted(self._len, key=repr)
        out = {"sequences": {str(i): {"length": self._len[i], "blocks": list(self._table[i])}
                             for i in ids}}
        out.update(self.stats())
        return out

    def block_tables(self, seq_ids, max_blocks: int):
        """Row-major [n, max_blocks] table padded with -1, and the lengths."""
        rows, lens = [], []
        for s in seq_ids:
            table = self.page_table(s)
            if len(table) > max_blocks:
                raise ValueError(f"sequence {s!r} owns {len(table)} blocks > {max_blocks}")
            rows.append(list(table) + [-1] * (max_blocks - len(table)))
            lens.append(self._len[s])
        return rows, lens

    # -- changing the state --------------------------------------------
    def create(self, seq_id) -> None:
        hash(seq_id)  # an unhashable id raises TypeError
        if seq_id in self._len:
            raise ValueError(f"id {seq_id!r} is taken")
        self._len[seq_id] = 0
        self._table[seq_id] = []

    def _needs_copy(self, seq_id, n: int) -> bool:
        """A write of n > 0 tokens lands in a partial last block someone else names."""
        length = self._len[seq_id]
        return (n > 0 and length % self.block_size != 0
                and self.refs[self._table[seq_id][-1]] > 1)

    def blocks_needed(self, seq_id, n: int) -> int:
        """Free blocks an append of n tokens consumes (new entries + a copy)."""
        self._known(seq_id)
        length = self._len[seq_id]
        grow = _ceil_div(length + n, self.block_size) - _ceil_div(length, self.block_size)
        return grow + int(self._needs_copy(seq_id, n))

    def _pop(self) -> int:
        b = self.free.pop()
        self.refs[b] = 1
        return b

    def _unref(self, blocks) -> None:
        """Drop one reference per id (in order); unnamed blocks go on the stack."""
        for b in blocks:
            self.refs[b] -= 1
        self.free.extend(b for b in blocks if self.refs[b] == 0)

    def append(self, seq_id, n: int):
        """Grow a sequence by n tokens. Returns (slots of the new tokens,
        copy-on-write pairs (old block, replacement))."""
        if not _is_int(n) or n < 0:
            raise ValueError("an append needs a whole number of tokens >= 0")
        self._known(seq_id)
        need = self.blocks_needed(seq_id, n)
        if need > len(self.free):
            raise MemoryError(f"append wants {need} blocks; the pool has {len(self.free)}")
        length = self._len[seq_id]
        table = self._table[seq_id]
        pairs = []
        if self._needs_copy(seq_id, n):
            old = table[-1]
            self.refs[old] -= 1  # still named by another table, so never freed here
            table[-1] = self._pop()
            pairs.append((old, table[-1]))
        grow = need - len(pairs)
        table.extend(self._pop() for _ in range(grow))
        self._len[seq_id] = length + n
        return [self.slot(seq_id, t) for t in range(length, length + n)], pairs

    def append_to(self, seq_id, total: int):
        """Grow a sequence to ``total`` tokens (never shortens it)."""
        if not _is_int(total) or total < 0:
            raise ValueError("a target length must be a whole number >= 0")
        have = self.sequence_length(seq_id)
        if total < have:
            raise ValueError(f"sequence {seq_id!r} already holds {have} > {total} tokens")
        return self.append(seq_id, total - have)

    def share_prefix(self, src, dst, prefix: int) -> None:
        """Fork: dst names src's first ceil(prefix / bs) blocks; its length is prefix."""
        self._known(src)
        if not _is_int(prefix) or prefix < 0:
            raise ValueError("a prefix must be a whole number of tokens >= 0")
        if prefix > self._len[src]:
            raise ValueError(f"prefix {prefix} is longer than sequence {src!r}")
        if dst in self._len:
            raise ValueError(f"fork target {dst!r} is taken")
        hash(dst)
        shared = self._table[src][:_ceil_div(prefix, self.block_size)]
        for b in shared:
            self.refs[b] += 1
        self._len[dst] = prefix
        self._table[dst] = list(shared)

    def release(self, seq_id) -> None:
        self._known(seq_id)
        self._unref(self._table.pop(seq_id))
        del self._len[seq_id]

    def truncate(self, seq_id, new_length: int) -> None:
        self._known(seq_id)
        if not _is_int(new_length) or not 0 <= new_length <= self._len[seq_id]:
            raise ValueError(f"a new length must lie in [0, {self._len[seq_id]}]")
        keep = _ceil_div(new_length, self.block_size)
        table = self._table[seq_id]
        dropped = table[keep:]
        del table[keep:]
        self._unref(dropped)
        self._len[seq_id] = new_length

    # -- invariants (the rule list of [KVNB §5] validate) --------------
    def validate(self) -> None:
        """Raise AssertionError naming the first broken rule."""
        n, bs = self.total_blocks, self.block_size
        seen = set()
        for b in self.free:
            if not 0 <= b < n:
                raise AssertionError(f"free stack names id {b} outside the pool")
            if b in seen:
                raise AssertionError(f"free stack names block {b} twice")
            seen.add(b)
        named = [0] * n
        for s, table in self._table.items():
            length = self._len[s]
            if length < 0:
                raise AssertionError(f"sequence {s!r} has a negative length")
            if len(table) != _ceil_div(length, bs):
                raise AssertionError(f"sequence {s!r}: table size disagrees with its length")
            if len(set(table)) != len(table):
                raise AssertionError(f"sequence {s!r} names one block twice")
            for b in table:
                if not 0 <= b < n:
                    raise AssertionError(f"sequence {s!r} names id {b} outside the pool")
            for b in table:
                named[b] += 1
        on_stack = set(self.free)
        fill = self.fills()
        for b in range(n):
            if self.refs[b] != named[b]:
                raise AssertionError(f"block {b}: count {self.refs[b]} but {named[b]} names")
            if named[b] and b in on_stack:
                raise AssertionError(f"block {b} is named and also free")
            if not named[b] and b not in on_stack:
                raise AssertionError(f"block {b} is neither named nor free")
            if named[b] and not 1 <= fill[b] <= bs:
                raise AssertionError(f"block {b} holds {fill[b]} tokens")
        st = self.stats()
        if st["physical_payload_tokens"] > st["logical_tokens"]:
            raise AssertionError("more tokens stored than the sequences hold")

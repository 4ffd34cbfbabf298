"""Pins for the pool oracle's invariant checker (``PagedPool.validate``) -- CPU only.

[KVNB §5] ``validate`` lists the rules a page pool must keep; [KVNB §9]
"Negative tests" asks that broken states are refused. Each case below breaks
exactly one rule of a small, valid pool (the others still hold) and expects
``AssertionError`` naming that rule, so deleting any one check fails its
case. Fills are derived from the tables in this oracle, so a fill outside
[1, block size] and a payload above the logical tokens cannot arise while
the tables are consistent; those two cases hand in fills that disagree with
the tables (the stored fills of the page's own pool could).
"""

import pytest

from oracle.pool import PagedPool


def valid_pool() -> PagedPool:
    """Blocks of 4 slots; a (6 tokens, 2 blocks), b forked from a's first 6
    (sharing both blocks), c (9 tokens, 3 blocks); 3 blocks free."""
    p = PagedPool(10, 4)
    p.create("a")
    p.append("a", 6)
    p.share_prefix("a", "b", 6)
    p.create("c")
    p.append("c", 9)
    p.validate()
    return p


def _free_named_block(p: PagedPool, seq, j: int, new_id: int) -> int:
    """Point table entry j of seq at new_id (taken off the free stack) and
    return the block it named, left unnamed and put on the free stack."""
    old = p._table[seq][j]
    p.free.remove(new_id)
    p._table[seq][j] = new_id
    p.refs[new_id] += 1
    p.refs[old] -= 1
    if p.refs[old] == 0:
        p.free.append(old)
    return old


def corrupt_free_out_of_range(p):
    p.free.append(p.total_blocks + 3)


def corrupt_free_twice(p):
    p.free.append(p.free[0])


def corrupt_negative_length(p):
    p.create("z")
    p._len["z"] = -3  # ceil(-3 / 4) = 0 entries: the table size still agrees


def corrupt_table_size(p):
    p._len["c"] = 13  # 4 entries wanted, 3 held; fills stay within [1, 4]


def corrupt_block_twice(p):
    first = p._table["c"][0]
    _free_named_block(p, "c", 1, p.free[-1])  # keep counts right while editing
    second = p._table["c"][1]
    p._table["c"][1] = first
    p.refs[first] += 1
    p.refs[second] -= 1
    p.free.append(second)


def corrupt_table_out_of_range(p):
    old = p._table["c"][2]
    p._table["c"][2] = p.total_blocks + 1
    p.refs[old] -= 1
    p.free.append(old)


def corrupt_count(p):
    p.refs[p._table["c"][0]] += 1


def corrupt_named_and_free(p):
    p.free.append(p._table["c"][1])


def corrupt_neither(p):
    p.free.pop()  # an unnamed block disappears from the stack


CASES = {
    "free stack names id .* outside": corrupt_free_out_of_range,
    "free stack names block .* twice": corrupt_free_twice,
    "negative length": corrupt_negative_length,
    "table size disagrees": corrupt_table_size,
    "names one block twice": corrupt_block_twice,
    "sequence .* names id .* outside": corrupt_table_out_of_range,
    "count .* but .* names": corrupt_count,
    "named and also free": corrupt_named_and_free,
    "neither named nor free": corrupt_neither,
}


@pytest.mark.parametrize("rule", list(CASES))
def test_each_broken_rule_is_refused(rule):
    p = valid_pool()
    CASES[rule](p)
    with pytest.raises(AssertionError, match=rule):
        p.validate()


class StoredFills(PagedPool):
    """A pool whose fills come from a stored list, as in a pool that keeps
    per-block fill counters beside its tables."""

    stored = None

    def fills(self):
        return list(self.stored) if self.stored is not None else super().fills()


@pytest.mark.parametrize("bad,rule", [(0, "holds 0 tokens"), (5, "holds 5 tokens")])
def test_fill_outside_block_is_refused(bad, rule):
    p = StoredFills(4, 4)
    p.create("a")
    p.append("a", 6)
    fill = p.fills()
    fill[p.page_table("a")[1]] = bad
    p.stored = fill
    with pytest.raises(AssertionError, match=rule):
        p.validate()


def test_payload_above_logical_is_refused():
    p = StoredFills(4, 4)
    p.create("a")
    p.append("a", 1)
    fill = p.fills()
    fill[p.page_table("a")[0]] = 4  # within [1, 4], but 4 stored for 1 token
    p.stored = fill
    with pytest.raises(AssertionError, match="more tokens stored"):
        p.validate()


def test_valid_states_pass():
    """The same pool without corruption, and after every kind of operation."""
    p = valid_pool()
    p.append("b", 3)  # copy of the shared partial block
    p.truncate("a", 2)
    p.release("c")
    p.validate()

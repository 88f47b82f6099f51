"""Hand-worked cases for the page allocator's Python model alone (oracle/pages.py), so that a
mistake the model shared with the C++ allocator would still be caught.  Every expected value
below was worked out by hand from the rules the model states: lowest free page first, copy on
write of a shared partly filled last page, a prefix tree of whole pages, the longest run of
equal pages on lookup, and eviction of the least recently used unshared leaf first (ties broken
by insertion order)."""
from oracle.pages import PageModel


def test_fork_and_copy_on_write_by_hand():
    m = PageModel(8, 4)
    s = m.create()
    assert m.reserve(s, 6) == [] and m.table(s) == [0, 1]        # pages 0, 1 (2 slots of 1 used)
    t = m.fork(s)
    assert m.refs[:3] == [2, 2, 0]
    assert m.reserve(t, 1) == [(1, 2)]                           # t's slot 6 is in shared page 1
    assert m.table(t) == [0, 2] and m.table(s) == [0, 1]
    assert m.refs[:4] == [2, 1, 1, 0]
    assert m.reserve(s, 2) == [] and m.table(s) == [0, 1]        # page 1 is s's alone: no copy
    assert m.reserve(t, 2) == [] and m.table(t) == [0, 2, 3]     # t's slot 8 starts page 3
    m.release(t)
    assert m.refs[:4] == [1, 1, 0, 0] and m.free_count() == 6


def build_tree():
    """Page size 2.  Three sequences inserted at clocks 1, 2, 3:
         a: tokens 1 2 | 3 4 | 5 6      pages 0 1 2
         b: tokens 1 2 | 3 4 | 7 8      pages 3 4 5  (first two pages match a's nodes)
         c: tokens 9 9                  page  6
    Tree: root -> n0 (1 2, page 0) -> n1 (3 4, page 1) -> n2 (5 6, page 2)
                                                       -> n3 (7 8, page 5)
          root -> n4 (9 9, page 6)."""
    m = PageModel(16, 2)
    seqs = {}
    for name, toks in (("a", [1, 2, 3, 4, 5, 6]), ("b", [1, 2, 3, 4, 7, 8]), ("c", [9, 9])):
        sid = m.create()
        m.reserve(sid, len(toks))
        m.prefix_insert(sid, toks)
        seqs[name] = sid
    return m, seqs


def test_prefix_tree_and_longest_match_by_hand():
    m, seqs = build_tree()
    assert m.table(seqs["a"]) == [0, 1, 2] and m.table(seqs["b"]) == [3, 4, 5]
    assert m.table(seqs["c"]) == [6]
    # cache references: n0..n4 hold pages 0, 1, 2, 5, 6 (b's pages 3 and 4 matched a's nodes)
    assert m.refs[:7] == [2, 2, 2, 1, 1, 2, 2]
    assert [x[2] for x in m.nodes] == [0, 1, 2, 5, 6]
    # longest match: 1 2 | 3 4 | 7 8 | 0 0 follows n0, n1, n3 and stops at the fourth page
    sid, matched = m.create_with_prefix([1, 2, 3, 4, 7, 8, 0, 0])
    assert matched == 6 and m.table(sid) == [0, 1, 5]
    # a different second page stops after the first: 1 2 | 3 5
    sid2, matched2 = m.create_with_prefix([1, 2, 3, 5])
    assert matched2 == 2 and m.table(sid2) == [0]
    # an odd trailing token is not a whole page and is never matched
    sid3, matched3 = m.create_with_prefix([9, 9, 9])
    assert matched3 == 2 and m.table(sid3) == [6]
    # no match at all
    sid4, matched4 = m.create_with_prefix([5, 6])
    assert matched4 == 0 and m.table(sid4) == [] and m.length(sid4) == 0


def test_eviction_order_by_hand():
    m, seqs = build_tree()
    for name in ("a", "b", "c"):
        m.release(seqs[name])
    # now only the cache holds pages 0, 1, 2, 5, 6.  Last uses: a's insert (clock 1) made
    # n0, n1, n2; b's (clock 2) touched n0, n1 and made n3; c's (clock 3) made n4.
    assert [x[3] for x in m.nodes] == [2, 2, 1, 2, 3]
    # leaves: n2 (use 1), n3 (use 2), n4 (use 3); n2 goes first
    assert m.evict(1) == 1 and not m.nodes[2][5] and m.refs[2] == 0
    # a lookup through n3 makes it the most recently used leaf (clock 4)
    sid, matched = m.create_with_prefix([1, 2, 3, 4, 7, 8])
    assert matched == 6 and m.nodes[3][3] == 4
    # n3's page is now also held by the new sequence, so it cannot be evicted; n4 (use 3) is
    # the only evictable leaf
    assert m.evict(5) == 1 and not m.nodes[4][5] and m.refs[6] == 0
    m.release(sid)
    # the only leaf now is n3 (use 4); evicting it leaves n1 as the only leaf, then n0
    assert m.evict(1) == 1 and not m.nodes[3][5] and m.nodes[1][5]
    assert m.evict(10) == 2
    assert [x[5] for x in m.nodes] == [False] * 5
    assert m.free_count() == 16

"""Pins for the oracle's visibility rule.

The page's parameter table defines sparse_mode 0 (defaultMask) and 3
(rightDownCausal: lower triangle cut at the bottom-right corner), and
cmp_ratio (keys compressed by that factor).  The reading adopted: entry j
covers original tokens [j*cmp, (j+1)*cmp), and query i of a sequence with
S1 queries over Sk tokens sits at position Sk - S1 + i and sees an entry
only when every token of it is at or before that position.  The brute force
below checks that definition token by token.
"""
import itertools

from tests._helpers import rows_of  # noqa: F401


def brute_visible(mode, cmp, sk, s1, i):
    stored = sk // cmp
    if mode == 0:
        return stored
    pos = sk - s1 + i
    n = 0
    for j in range(stored):
        if all(t <= pos for t in range(j * cmp, (j + 1) * cmp)):
            n += 1
    return n


def test_visible_matches_token_brute_force(ora):
    for mode, cmp, sk, s1 in itertools.product((0, 3), (1, 2, 4, 8, 128), range(0, 41, 3), (1, 2, 3, 5, 9, 50)):
        for i in range(s1):
            assert ora.visible(mode, cmp, sk, s1, i) == brute_visible(mode, cmp, sk, s1, i), (mode, cmp, sk, s1, i)


def test_mode0_equals_mode3_for_single_uncompressed_query(ora):
    for sk in (0, 1, 17, 4096):
        assert ora.visible(0, 1, sk, 1, 0) == ora.visible(3, 1, sk, 1, 0) == sk


def test_causal_growth_and_last_query(ora):
    for cmp in (1, 2, 4, 128):
        sk, s1 = 1000, 37
        v = [ora.visible(3, cmp, sk, s1, i) for i in range(s1)]
        assert all(a <= b for a, b in zip(v, v[1:]))
        assert v[-1] == sk // cmp


def test_long_context_edges(ora):
    # 131072 tokens, 2 queries, 4x compression: 32767 then 32768 entries
    assert ora.visible(3, 4, 131072, 2, 0) == 32767
    assert ora.visible(3, 4, 131072, 2, 1) == 32768
    # the page's aclgraph example shape: s2=512, s1=4, cmp 4
    assert [ora.visible(3, 4, 512, 4, i) for i in range(4)] == [127, 127, 127, 128]


def test_more_queries_than_keys_clamps_to_zero(ora):
    assert ora.visible(3, 1, 3, 10, 0) == 0
    assert ora.visible(3, 1, 3, 10, 6) == 0
    assert ora.visible(3, 1, 3, 10, 7) == 1
    assert ora.visible(3, 1, 3, 10, 9) == 3


def test_row_visible_layouts(ora):
    # BSND with per-batch query counts below S1: unused rows see nothing
    v = ora.row_visible(0, 2, 3, 3, 1, [2, 3], [10, 4])
    assert list(v) == [9, 10, 0, 2, 3, 4]
    # TND prefix sums [2, 5]: batch 0 = rows 0..1, batch 1 = rows 2..4, row 5 unused
    v = ora.row_visible(1, 2, 6, 3, 1, [2, 5], [10, 4])
    assert list(v) == [9, 10, 2, 3, 4, 0]


# --- pre_tokens / next_tokens windows ----------------------------------------
# The page marks both parameters as reserved (only 2^63-1).  The reading pinned
# here: query i sits at position pos = Sk - S1 + i in both modes; token t is
# inside its window when pos - pre <= t <= pos + next; an entry is visible when
# the mode lets the query see it and every token it covers is in the window.

INT64_MAX = (1 << 63) - 1


def brute_window(mode, cmp, sk, s1, i, pre, nxt):
    """The visible entries as a set, token by token in Python integers."""
    pos = sk - s1 + i
    out = set()
    for j in range(sk // cmp):
        toks = range(j * cmp, (j + 1) * cmp)
        if mode == 3 and not all(t <= pos for t in toks):
            continue
        if all(pos - pre <= t <= pos + nxt for t in toks):
            out.add(j)
    return out


def test_window_matches_token_brute_force(ora):
    bounds = (0, 1, 2, 3, 5, 8, 13, 40, INT64_MAX)
    for mode, cmp, sk, s1 in itertools.product((0, 3), (1, 2, 4, 8), (0, 7, 16, 33), (1, 3, 9, 40)):
        for i in range(0, s1, max(1, s1 // 4)):
            for pre, nxt in itertools.product(bounds, bounds):
                want = brute_window(mode, cmp, sk, s1, i, pre, nxt)
                lo, hi = ora.visible_range(mode, cmp, sk, s1, i, pre, nxt)
                assert set(range(lo, hi)) == want, (mode, cmp, sk, s1, i, pre, nxt, lo, hi)


def test_window_defaults_and_special_cases(ora):
    # the defaults cut nothing: [0, visible)
    for mode, cmp, sk, s1, i in ((0, 1, 100, 4, 2), (3, 4, 131072, 2, 0), (3, 1, 3, 10, 8)):
        assert ora.visible_range(mode, cmp, sk, s1, i) == (0, ora.visible(mode, cmp, sk, s1, i))
    # pre = next = 0, no compression: the query's own position only
    assert ora.visible_range(0, 1, 100, 4, 1, 0, 0) == (97, 98)
    assert ora.visible_range(3, 1, 100, 4, 1, 0, 0) == (97, 98)
    # sliding window of 64 tokens over 4x compressed keys: 16 whole entries end at pos
    assert ora.visible_range(3, 4, 131072, 2, 1, 63, 0) == (32752, 32768)
    # next_tokens lets a mode-0 query see later tokens; mode 3 still stops at pos
    assert ora.visible_range(0, 1, 100, 4, 0, 0, 2) == (96, 99)
    assert ora.visible_range(3, 1, 100, 4, 0, 0, 2) == (96, 97)
    # a window that ends before the first stored token, or a query before any key
    assert ora.visible_range(0, 1, 10, 20, 0, 3, 2) == (0, 0)
    assert ora.visible_range(3, 1, 10, 20, 15, 100, 0) == (0, 6)


def test_row_range_layouts(ora):
    # TND prefix sums [2, 5] over lengths [10, 4], window pre = 2: rows see
    # [6, 9), [7, 10), then batch 1 rows at positions 1, 2, 3: [0, 2), [0, 3), [1, 4)
    lo, hi = ora.row_range(1, 2, 6, 3, 1, [2, 5], [10, 4], 2, INT64_MAX)
    assert list(lo) == [6, 7, 0, 0, 1, 0] and list(hi) == [9, 10, 2, 3, 4, 0]

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

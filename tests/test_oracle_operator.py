"""Pins for the whole oracle operator: output layout and padding, paging and
layout invariances, the page's own example shapes, and validation.

Sources (VllmQuantLightningIndexer page): parameter table (sparse_indices,
sparse_values, block_table, stride, layout_query BSND/TND), constraints
(TND prefix sums, block_size), and the two example programs (single-operator
call and graph-mode call), whose shapes and seeds are reused here.  The page
prints no outputs for them; what they pin is that with sparse_count at or
above every row's visible count the indexer returns exactly the visible set.
"""
import numpy as np
import pytest

import synth
from tests._helpers import rows_of


def run(ora, inp, **kw):
    rc, idx, val, sc = ora.indexer(inp, **kw)
    assert rc == 0
    return idx, val, sc


def check_rows(ora, inp, idx, val, sc):
    p = inp["problem"]
    vis = ora.row_visible(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"],
                          inp["aslq"], inp["aslk"])
    k = p["sparse_count"]
    for r in range(rows_of(p)):
        n = min(k, vis[r])
        assert np.all(idx[r, n:] == -1) and np.all(val[r, n:] == -np.inf)
        sel = idx[r, :n]
        assert len(set(sel.tolist())) == n and (n == 0 or (sel.min() >= 0 and sel.max() < vis[r]))
        if sc is not None and n:
            s = sc[r, :vis[r]]
            assert np.array_equal(val[r, :n], s[sel].astype(np.float32))
            assert np.array_equal(sel, np.argsort(-s, kind="stable")[:n])
    return vis


def test_output_layout_and_padding(ora):
    spec = synth.small(batch=3, s1=3, aslk=[150, 40, 0], aslq=[3, 2, 3], block_size=32,
                       sparse_count=64, sparse_mode=3, cmp_ratio=2)
    inp = synth.make_inputs(spec, 21)
    idx, val, sc = run(ora, inp, scores_cols=80)
    vis = check_rows(ora, inp, idx, val, sc)
    # batch 0: 150 tokens, 3 queries, cmp 2 -> floor((148..150)/2) = 74, 74, 75 entries (> k);
    # batch 1: 40 tokens, 2 of 3 queries used -> 19, 20 and an unused row; batch 2 has no keys
    assert list(vis) == [74, 74, 75, 19, 20, 0, 0, 0, 0]
    assert np.all(idx[5] == -1) and np.all(idx[6:] == -1)


def test_paging_invariance(ora):
    """A permuted block table over physically permuted blocks, and a padded
    block stride, give the same result as contiguous identity paging."""
    base = synth.small(batch=2, s1=2, aslk=[200, 130], block_size=16, sparse_count=32, table="identity")
    a = synth.make_inputs(base, 5)
    b = synth.make_inputs(base, 5)
    p = a["problem"]
    nb, bs = p["num_blocks"], p["block_size"]
    perm = np.random.default_rng(1).permutation(nb)         # logical block i stored at perm[i]
    kb = a["key"].reshape(nb, bs * 128)
    pad = 48
    stored = np.zeros((nb, bs * 128 + pad), dtype=np.uint8)
    stored[perm, :bs * 128] = kb
    stored[:, bs * 128:] = 0x7F
    b["key"] = stored.reshape(-1)
    b["problem"]["key_block_stride"] = bs * 128 + pad
    ks = np.zeros_like(a["k_scale"])
    ks[perm] = a["k_scale"]
    b["k_scale"] = ks
    t = a["block_table"].copy()
    t[t >= 0] = perm[t[t >= 0]]
    b["block_table"] = np.ascontiguousarray(t)
    ia, va, sa = run(ora, a, scores_cols=200)
    ib, vb, sb = run(ora, b, scores_cols=200)
    assert np.array_equal(ia, ib) and np.array_equal(va, vb)
    assert np.array_equal(np.nan_to_num(sa, nan=-1), np.nan_to_num(sb, nan=-1))


def test_tnd_equals_bsnd_for_equal_lengths(ora):
    bs_spec = synth.small(batch=3, s1=4, aslk=[90, 70, 120], block_size=16, sparse_count=40,
                          sparse_mode=3)
    a = synth.make_inputs(bs_spec, 2)
    b = dict(a)
    b["problem"] = dict(a["problem"], layout_query=synth.TND, s1=12)
    b["aslq"] = np.array([4, 8, 12], dtype=np.int32)
    ia, va, _ = run(ora, a)
    ib, vb, _ = run(ora, b)
    assert np.array_equal(ia, ib) and np.array_equal(va, vb)


def test_single_operator_example_shape(ora):
    """Shapes and recipe of the page's single-operator example: b=24, s1=4,
    s2=512, block_size=128, identity table, sparse_count=512, mode 0, cmp 1.
    Every row has 512 visible entries, so every index 0..511 comes back."""
    spec = synth.Spec("example1", synth.INT8, synth.BSND, 24, 4, [512] * 24, 128, 512, 0, 1,
                      table="identity")
    inp = synth.make_inputs(spec, 0)
    idx, val, _ = run(ora, inp)
    for r in range(96):
        assert sorted(idx[r].tolist()) == list(range(512))
    assert np.all(np.isfinite(val)) and np.all(val >= 0)


def test_graph_mode_example_shape(ora):
    """The page's graph-mode example: same shape, sparse_mode 3, cmp_ratio 4.
    Visible counts per query are 127, 127, 127, 128 < 512."""
    spec = synth.Spec("example2", synth.INT8, synth.BSND, 24, 4, [512] * 24, 128, 512, 3, 4,
                      table="identity")
    inp = synth.make_inputs(spec, 0)
    idx, val, _ = run(ora, inp)
    for r in range(96):
        n = [127, 127, 127, 128][r % 4]
        assert sorted(idx[r, :n].tolist()) == list(range(n))
        assert np.all(idx[r, n:] == -1) and np.all(val[r, n:] == -np.inf)


def test_fp8_operator_runs_and_is_consistent(ora):
    spec = synth.small(qk=synth.FP8, batch=2, s1=1, aslk=[300, 77], block_size=64, sparse_count=50)
    inp = synth.make_inputs(spec, 4)
    idx, val, sc = run(ora, inp, scores_cols=300)
    check_rows(ora, inp, idx, val, sc)


@pytest.mark.parametrize("field,value,code", [
    ("block_size", 24, 1), ("block_size", 2048, 1), ("sparse_count", 0, 1), ("sparse_count", 2049, 1),
    ("sparse_mode", 1, 1), ("cmp_ratio", 3, 1), ("cmp_ratio", 256, 1), ("scale_dtype", 1, 2)])
def test_validation(ora, field, value, code):
    inp = synth.make_inputs(synth.small(), 1)
    inp["problem"] = dict(inp["problem"], **{field: value})
    rc, *_ = ora.indexer(inp)
    assert rc == code


def test_validation_tables(ora):
    inp = synth.make_inputs(synth.small(aslk=[300, 200], block_size=64), 1)
    inp["problem"] = dict(inp["problem"], max_blocks_per_seq=4)
    inp["block_table"] = np.ascontiguousarray(inp["block_table"][:, :4])
    assert ora.indexer(inp)[0] == 1                     # 300 entries need 5 blocks of 64
    inp = synth.make_inputs(synth.small(layout=synth.TND, s1=6, aslq=[4, 3]), 1)
    assert ora.indexer(inp)[0] == 1                     # prefix sums must not decrease


@pytest.mark.parametrize("mode,cmp,pre,nxt", [(3, 1, 40, 0), (0, 2, 100, 30), (3, 4, 7, 5), (0, 1, 0, 0)])
def test_window_restricts_the_candidates(ora, mode, cmp, pre, nxt):
    """With a window, each row's result is the stable top-k of the unwindowed
    scores restricted to the row's window (entries [lo, hi))."""
    import math
    spec = synth.small(batch=2, s1=5, aslk=[700, 260], block_size=32, sparse_count=24, sparse_mode=mode,
                       cmp_ratio=cmp, pre_tokens=pre, next_tokens=nxt)
    inp = synth.make_inputs(spec, 31)
    full = dict(inp, problem=dict(inp["problem"], pre_tokens=synth.INT64_MAX, next_tokens=synth.INT64_MAX))
    _, _, sc = run(ora, full, scores_cols=800)
    idx, val, _ = run(ora, inp)
    p = inp["problem"]
    lo, hi = ora.row_range(0, 2, 5, mode, cmp, None, inp["aslk"], pre, nxt)
    k = p["sparse_count"]
    for r in range(10):
        cand = list(range(lo[r], hi[r]))
        # Python's sort: score descending, then index ascending
        top = sorted(cand, key=lambda j: (-sc[r, j], j))[:k]
        assert list(idx[r, :len(top)]) == top and np.all(idx[r, len(top):] == -1)
        assert all(val[r, i] == np.float32(sc[r, j]) for i, j in enumerate(top))
        assert all(not math.isnan(sc[r, j]) for j in cand)


def test_window_bounds_validated(ora):
    inp = synth.make_inputs(synth.small(pre_tokens=-1), 0)
    assert ora.indexer(inp)[0] == 1
    inp = synth.make_inputs(synth.small(next_tokens=-5), 0)
    assert ora.indexer(inp)[0] == 1

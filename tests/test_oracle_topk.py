"""Pins for the oracle's top-k (VllmQuantLightningIndexer page, section
功能说明 step 3: keep the Top-k indices).  Reading: larger score first,
equal scores to the lower index.  numpy's stable argsort of the negated
scores is an independent implementation of exactly that order."""
import numpy as np
import pytest


@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (100, 7), (1000, 512), (4096, 2048), (10, 64), (0, 5)])
def test_topk_matches_stable_argsort(ora, n, k):
    rng = np.random.default_rng(n * 31 + k)
    s = rng.integers(0, max(2, n // 4), size=n).astype(np.float64)  # many ties
    got = ora.topk(s, k)
    ref = np.argsort(-s, kind="stable")[:k]
    assert np.array_equal(got, ref)


def test_topk_invariants_continuous(ora):
    rng = np.random.default_rng(7)
    s = rng.standard_normal(3000)
    k = 700
    got = ora.topk(s, k)
    assert len(set(got.tolist())) == k
    assert got.min() >= 0 and got.max() < 3000
    sel = np.zeros(3000, bool)
    sel[got] = True
    assert s[sel].min() >= s[~sel].max()
    assert np.all(np.diff(s[got]) <= 0)


def test_all_equal_scores_take_lowest_indices(ora):
    assert list(ora.topk(np.zeros(50), 8)) == list(range(8))


def test_k_at_least_n_returns_everything(ora):
    rng = np.random.default_rng(3)
    s = rng.standard_normal(37)
    got = ora.topk(s, 64)
    assert sorted(got.tolist()) == list(range(37))

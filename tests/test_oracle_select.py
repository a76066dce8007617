"""Pins of the budget-selection oracle (oracle/select_ref.py), CPU only.

The page prints no worked example; the oracle's block-level definition is
checked against an independent cell-level ranking written with Python's
sorted(), against closed forms, and against the invariants every valid
selection has."""
import numpy as np
import pytest

from oracle import select_ref as R


def test_okey_orders_like_floats():
    vals = np.array([-np.inf, -3.0e38, -1.0, -1e-30, -1e-45, -0.0, 0.0, 1e-45, 1e-30, 1.0,
                     3.0e38, np.inf], dtype=np.float32)
    k = R.okey(vals).astype(np.int64)
    assert np.all(np.diff(k) > 0), k          # strictly increasing, -0 below +0
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(10000) * 10.0 ** rng.integers(-20, 20, 10000)).astype(np.float32)
    x = x[x != 0]
    assert np.array_equal(np.argsort(R.okey(x), kind="stable"), np.argsort(x, kind="stable"))


def cell_level(scores_row, n, B):
    """Independent formulation: every cell carries its block's score; rank
    cells by (score descending, cell ascending) with Python's sorted()."""
    if n <= B:
        return list(range(n))
    ranked = sorted(range(n), key=lambda c: (-float(scores_row[c // 4]), c))
    return sorted(ranked[:B])


@pytest.mark.parametrize("seed", range(12))
def test_matches_cell_level_ranking(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 200))
    B = int(rng.integers(1, 120))
    nb = n // 4 + 1
    # few distinct values -> many ties between blocks; no zeros (the float
    # comparison and the key agree away from -0/+0)
    scores = rng.integers(1, 6, size=nb).astype(np.float32) * rng.choice([-1, 1], size=nb)
    got = R.select_one(scores, n, B)
    assert list(got) == cell_level(scores, n, B)


def test_identity_below_budget():
    scores = np.arange(10, dtype=np.float32)
    for n in (0, 1, 7, 40):
        assert list(R.select_one(scores, n, 40)) == list(range(n))


def test_distinct_scores_take_top_blocks():
    rng = np.random.default_rng(3)
    n, B = 400, 64          # whole blocks only
    nb = n // 4 + 1
    scores = rng.permutation(nb).astype(np.float32)
    top = np.argsort(-scores[:n // 4])[:B // 4]
    expect = np.sort(np.concatenate([np.arange(4 * b, 4 * b + 4) for b in top]))
    assert np.array_equal(R.select_one(scores, n, B), expect)


def test_all_equal_scores_take_first_cells():
    scores = np.full(101, 0.5, dtype=np.float32)
    assert np.array_equal(R.select_one(scores, 399, 37), np.arange(37))


def test_partial_last_block_weighs_its_cells():
    # n = 10: blocks 0, 1 whole, block 2 holds cells 8, 9; it scores highest
    scores = np.array([1.0, 2.0, 9.0], dtype=np.float32)
    assert list(R.select_one(scores, 10, 3)) == [4, 8, 9]
    # n = 8: block 2 holds no cell and is never taken despite its score
    assert list(R.select_one(scores, 8, 5)) == [0, 4, 5, 6, 7]


def test_negative_zero_ranks_below_positive_zero():
    scores = np.array([-0.0, 0.0, -1.0], dtype=np.float32)
    assert list(R.select_one(scores, 12, 4)) == [4, 5, 6, 7]


@pytest.mark.parametrize("seed", range(4))
def test_invariants_and_causal_rows(seed):
    rng = np.random.default_rng(100 + seed)
    S, T, Lmax, B = 3, 4, 300, 50
    lens = np.array([300, 52, 2], dtype=np.int32)
    bs = rng.standard_normal((S, T, R.blocks_per_token(Lmax))).astype(np.float32)
    ids = R.select_budget_ids(bs, lens, T, Lmax, B)
    for s in range(S):
        for t in range(T):
            n = max(0, min(int(lens[s]) - (T - 1 - t), Lmax))
            w = min(n, B)
            row = ids[s, t]
            assert np.all(row[w:] == -1)
            v = row[:w]
            assert np.all(np.diff(v) > 0) and (w == 0 or (v[0] >= 0 and v[-1] < n))
            assert list(v) == cell_level(bs[s, t], n, B)

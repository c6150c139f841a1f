"""Pins for oracle.topk against brute force with Python's sorted()."""
import math

import numpy as np
import pytest

from oracle import topk


def _brute(scores, valid, k, col_to_row=None):
    items = []
    for c, (s, v) in enumerate(zip(scores, valid)):
        if not v:
            continue
        s = float(s)
        if math.isnan(s):
            s = -math.inf
        if s == 0.0:
            s = 0.0  # -0 == +0
        items.append((s, c))
    # highest score first; among equal scores the lower column first
    items = sorted(items, key=lambda t: (-t[0], t[1]))[:k]
    cols = sorted(c for _, c in items)
    rows = [col_to_row[c] if col_to_row is not None else c for c in cols]
    return rows + [-1] * (k - len(rows))


def test_crafted_ties_nan_signed_zero():
    s = np.array([1.0, 2.0, 2.0, np.nan, -0.0, 0.0, -np.inf, 2.0, 0.0, -1.0], dtype=np.float32)
    v = np.ones(len(s), dtype=bool)
    for k in range(1, 12):
        assert list(topk.topk_row(s, v, k)) == _brute(s, v, k), k
    # ties resolve to the lower index: with k=2 the three 2.0s give columns 1 and 2
    assert list(topk.topk_row(s, v, 2)) == [1, 2]
    # NaN ranks with -inf, below every finite score
    assert 3 not in list(topk.topk_row(s, v, 8))
    # -0 and +0 tie: column 4 wins over 5 and 8
    assert list(topk.topk_row(s, v, 5)) == [0, 1, 2, 4, 7]


def test_short_rows_pad_with_minus_one():
    s = np.arange(5, dtype=np.float32)
    v = np.array([1, 1, 0, 1, 0], dtype=bool)
    assert list(topk.topk_row(s, v, 4)) == [0, 1, 3, -1]
    assert list(topk.topk_row(s, np.zeros(5, bool), 3)) == [-1, -1, -1]


def test_all_equal_scores_take_lowest_columns():
    s = np.full(100, 0.5, dtype=np.float32)
    assert list(topk.topk_row(s, np.ones(100, bool), 7)) == list(range(7))


@pytest.mark.parametrize("seed", range(20))
def test_random_small_rows(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 80))
    # few distinct values so ties are common
    s = rng.integers(-4, 5, n).astype(np.float32) * 0.25
    s[rng.random(n) < 0.05] = np.nan
    s[rng.random(n) < 0.05] = -0.0
    v = rng.random(n) < 0.8
    k = int(rng.integers(1, 40))
    assert list(topk.topk_row(s, v, k)) == _brute(s, v, k)


def test_full_and_reindex_validity():
    rng = np.random.default_rng(9)
    scores = rng.standard_normal((3, 40)).astype(np.float32)
    pos = np.array([0, 9, 79])
    out = topk.topk_full(scores, pos, 2, 8)
    for r in range(3):
        nv = (pos[r] + 1) // 2
        assert list(out[r]) == _brute(scores[r], np.arange(40) < nv, 8)
    cand = np.array([[0, 2, 4, -1, -1], [1, 3, -1, -1, -1], [0, 1, 2, 3, 4]])
    out = topk.topk_reindex(scores, pos, 1, cand, 8, 6)
    for r in range(3):
        nv = pos[r] + 1
        rows = np.repeat(cand[r], 8) * 8 + np.tile(np.arange(8), 5)
        valid = (np.repeat(cand[r], 8) >= 0) & (rows < nv)
        assert list(out[r]) == _brute(scores[r], valid, 6, col_to_row=rows)

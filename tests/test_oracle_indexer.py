"""Pins for oracle.indexer: loop evaluation, REINDEX == FULL-then-mask, printed scale."""
import json
import math
import os

import numpy as np
import pytest

from oracle import indexer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _loop_score(q, w, k, scale, relu=True):
    total = 0.0
    for h in range(q.shape[0]):
        d = 0.0
        for i in range(q.shape[1]):
            d += float(q[h, i]) * float(k[i])
        if relu and d < 0:
            d = 0.0
        total += float(w[h]) * d
    return scale * total


def test_scale_printed_forms():
    g = json.load(open(os.path.join(GOLDEN, "indexer_scale.json")))
    for c in g["cases"]:
        assert math.isclose(indexer.indexer_scale(c["heads"], c["dim"]), c["scale"], rel_tol=1e-15)


@pytest.mark.parametrize("relu", [True, False])
def test_full_scores_match_loops(relu):
    rng = np.random.default_rng(5)
    rows, H, D, N, m = 6, 4, 8, 9, 2
    q = rng.standard_normal((rows, H, D))
    w = rng.standard_normal((rows, H))
    plane = rng.standard_normal((N, D))
    pos = np.array([0, 1, 2, 7, 16, 17])
    width = 9
    s = indexer.scores_full(q, w, lambda r: plane, pos, m, 0.3, width, relu=relu)
    for r in range(rows):
        nv = (pos[r] + 1) // m
        for c in range(width):
            if c < nv:
                assert math.isclose(s[r, c], _loop_score(q[r], w[r], plane[c], 0.3, relu), rel_tol=1e-12, abs_tol=1e-12)
            else:
                assert s[r, c] == -np.inf


def test_relu_is_applied_per_head():
    q = np.array([[[1.0, 0.0]], [[1.0, 0.0]]]).reshape(1, 2, 2)
    q[0, 1] = [-1.0, 0.0]
    w = np.array([[1.0, 1.0]])
    plane = np.array([[2.0, 5.0]])
    s_relu = indexer.scores_full(q, w, lambda r: plane, np.array([0]), 1, 1.0, 1, relu=True)
    s_lin = indexer.scores_full(q, w, lambda r: plane, np.array([0]), 1, 1.0, 1, relu=False)
    assert s_relu[0, 0] == 2.0 and s_lin[0, 0] == 0.0


def test_reindex_equals_full_then_mask():
    rng = np.random.default_rng(6)
    rows, H, D, N, br, nb = 4, 3, 5, 61, 8, 5
    q = rng.standard_normal((rows, H, D))
    w = rng.standard_normal((rows, H))
    plane = rng.standard_normal((N, D))
    pos = np.array([60, 33, 7, 0])
    cand = np.array([[0, 3, 5, 7, -1], [1, 2, 4, -1, -1], [0, -1, -1, -1, -1], [0, -1, -1, -1, -1]])
    full = indexer.scores_full(q, w, lambda r: plane, pos, 1, 0.7, N)
    re = indexer.scores_reindex(q, w, lambda r: plane, pos, 1, cand, br, 0.7)
    for r in range(rows):
        nv = pos[r] + 1
        for i in range(nb):
            for t in range(br):
                row = cand[r, i] * br + t
                expect = full[r, row] if (cand[r, i] >= 0 and row < nv) else -np.inf
                assert re[r, i * br + t] == expect


def test_abs_bound_dominates_score():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((4, 16))
    w = rng.standard_normal(4)
    k = rng.standard_normal((10, 16))
    s = indexer.score_rows(q, w, k, 0.1)
    a = indexer.score_abs_bound(q, w, k, 0.1)
    assert np.all(np.abs(s) <= a + 1e-15)


@pytest.mark.parametrize("nan_sign", [1.0, -1.0])
def test_nan_key_gives_nan_score(nan_sign):
    """A NaN dot stays NaN through the per-head ReLU (of either sign bit), so the score is NaN; the
    loop form (ReLU as 'd < 0 -> 0', false for NaN) agrees.  Other columns are unaffected."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 3, 4))
    w = rng.standard_normal((1, 3))
    plane = rng.standard_normal((5, 4))
    plane[2, 1] = np.copysign(np.nan, nan_sign)
    s = indexer.scores_full(q, w, lambda r: plane, np.array([4]), 1, 0.5, 5)
    assert np.isnan(s[0, 2])
    assert math.isnan(_loop_score(q[0], w[0], plane[2], 0.5))
    for c in (0, 1, 3, 4):
        assert math.isclose(s[0, c], _loop_score(q[0], w[0], plane[c], 0.5), rel_tol=1e-12, abs_tol=1e-12)


def test_nan_query_head_gives_nan_row():
    """A NaN in one head of the query makes that head's dot NaN for every key: every valid score is
    NaN, invalid columns stay -inf."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 3, 4))
    q[0, 1, 3] = np.nan
    w = rng.standard_normal((1, 3))
    plane = rng.standard_normal((6, 4))
    s = indexer.scores_full(q, w, lambda r: plane, np.array([3]), 1, 0.5, 6)
    assert np.all(np.isnan(s[0, :4])) and np.all(s[0, 4:] == -np.inf)

"""Pins for oracle.candidates (the FULL layer's hierarchical candidate pool).

Checked against what the pages fix and what follows from it: a pure-Python
brute force of "8-row block max, NaN as -inf, clip to the largest finite
float, newest block pinned, best 2048 ascending", crafted NaN / infinity / tie
rows, the closed-form pool size, and the soundness property of the pool
(every row of the FULL top-k lies in a pool block, so REINDEX over the pool
reproduces FULL).
"""
import math

import numpy as np
import pytest

from oracle import candidates, indexer, topk

FMAX = float(np.finfo(np.float32).max)


def _brute_pool(scores, n_vis, block_rows, n_cand):
    nb = -(-n_vis // block_rows)
    blocks = []
    for b in range(nb):
        best = None
        for c in range(b * block_rows, min((b + 1) * block_rows, n_vis)):
            s = float(scores[c])
            if math.isnan(s):
                s = -math.inf
            elif s > FMAX:
                s = FMAX
            elif s < -FMAX:
                s = -FMAX
            best = s if best is None or s > best else best
        if b == nb - 1:
            best = math.inf
        blocks.append((best, b))
    chosen = sorted(b for _, b in sorted(blocks, key=lambda t: (-t[0], t[1]))[:n_cand])
    return chosen + [-1] * (n_cand - len(chosen))


@pytest.mark.parametrize("seed", range(6))
def test_random_rows_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        n_vis = int(rng.integers(0, 200))
        width = n_vis + int(rng.integers(0, 20))
        s = rng.standard_normal(width).astype(np.float32)
        # coarse values make ties between blocks common
        if seed % 2:
            s = np.round(s * 2) / 2
        n_cand = int(rng.integers(1, 30))
        got = candidates.candidate_pool_row(s, n_vis, 8, n_cand)
        assert list(got) == _brute_pool(s, n_vis, 8, n_cand)


def test_crafted_nan_inf_and_ties():
    B = 2
    # blocks (B = 2): 0:[nan, nan] 1:[-inf, -inf] 2:[+inf, 0] 3:[fmax, 1] 4:[5, nan] 5:[5, 5] 6:[-1, -2] (newest)
    s = np.array([np.nan, np.nan, -np.inf, -np.inf, np.inf, 0, FMAX, 1, 5, np.nan, 5, 5, -1, -2],
                 dtype=np.float32)
    m = candidates.block_maxima_row(s, len(s), B)
    assert m[0] == -np.inf                         # all-NaN block: NaN counts as -inf
    assert m[1] == -FMAX                           # -inf is clipped to the largest finite magnitude
    assert m[2] == FMAX and m[3] == FMAX           # +inf clipped: ties with a real FLT_MAX
    assert m[4] == 5.0                             # NaN ignored beside finite values
    assert m[6] == np.inf                          # newest block pinned
    # order: 6 (pinned), 2, 3 (tie -> lower id), 4, 5 (tie -> lower id), 1, 0
    for k, want in [(1, [6]), (2, [2, 6]), (3, [2, 3, 6]), (4, [2, 3, 4, 6]), (5, [2, 3, 4, 5, 6]),
                    (6, [1, 2, 3, 4, 5, 6]), (7, [0, 1, 2, 3, 4, 5, 6])]:
        assert list(candidates.candidate_pool_row(s, len(s), B, k)) == want
        assert list(candidates.candidate_pool_row(s, len(s), B, k)) == _brute_pool(s, len(s), B, k)
    # the newest block wins even if every score in it is NaN
    s2 = np.array([3.0, 4.0, np.nan], dtype=np.float32)
    assert list(candidates.candidate_pool_row(s2, 3, 2, 1)) == [1]


def test_pool_size_and_newest_block():
    rng = np.random.default_rng(7)
    for n_vis in [0, 1, 7, 8, 9, 63, 64, 65, 1000]:
        s = rng.standard_normal(n_vis + 3)
        for n_cand in [1, 4, 16, 200]:
            pool = candidates.candidate_pool_row(s, n_vis, 8, n_cand)
            nb = -(-n_vis // 8)
            v = pool[pool >= 0]
            assert len(v) == min(n_cand, nb)
            assert np.all(pool[len(v):] == -1) and np.all(np.diff(v) > 0)
            if nb:
                assert (n_vis - 1) // 8 in v          # the newest visible row's block is always kept
                assert v[-1] == nb - 1
            if nb <= n_cand:
                assert list(v) == list(range(nb))     # small histories keep every block


def test_rows_beyond_visibility_never_count():
    s = np.array([0.0] * 8 + [9.0] * 8 + [100.0] * 8, dtype=np.float32)
    # 12 visible rows: blocks 0 and 1 (partly visible, pinned); block 2 is invisible despite its scores
    pool = candidates.candidate_pool(s[None, :], np.array([11]), 1, 8, 4)
    assert list(pool[0]) == [0, 1, -1, -1]
    # ratio 2: pos 23 sees 12 rows as well
    assert list(candidates.candidate_pool(s[None, :], np.array([23]), 2, 8, 4)[0]) == [0, 1, -1, -1]


@pytest.mark.parametrize("seed", range(4))
def test_reindex_over_the_pool_reproduces_full(seed):
    """Soundness of the pool: a FULL top-k row c with k < n_cand lies in a pool block.

    Blocks that outrank c's block each hold a row that outranks c (a higher score,
    or an equal score at a lower column), and at most k-1 rows outrank c; with
    the pinned block that is at most k blocks ahead, so c's block is kept.
    REINDEX over the pool with the same query and weights therefore selects the
    same rows as FULL; its ties also resolve alike, because ascending blocks
    make REINDEX column order equal to row order.  (This holds for any finite
    scores, ties included; clipping infinities can merge ranks.)
    """
    rng = np.random.default_rng(100 + seed)
    H, D, N, k, n_cand = 4, 16, 700, 24, 25
    q = rng.standard_normal((3, H, D))
    w = rng.standard_normal((3, H))
    plane = np.round(rng.standard_normal((N, D)) * 2) / 2   # coarse: equal scores occur
    if seed == 3:
        plane[100:140] = plane[40]                          # many exact ties
    pos = np.array([N - 1, 517, 5])
    tau = indexer.indexer_scale(H, D)
    s_full = indexer.scores_full(q, w, lambda r: plane, pos, 1, tau, N)
    full = topk.topk_full(s_full, pos, 1, k)
    pool = candidates.candidate_pool(s_full, pos, 1, 8, n_cand)
    s_re = indexer.scores_reindex(q, w, lambda r: plane, pos, 1, pool, 8, tau)
    re = topk.topk_reindex(s_re, pos, 1, pool, 8, k)
    assert np.array_equal(full, re)

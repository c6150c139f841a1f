"""Hierarchical candidate pool of the FULL owner layer (oracle; test infrastructure only).

What the pages fix ("DeepSeek-V4.1-Flash 架构解剖", special module "indexer",
fig. 3b, second level; the same page's fig. 3 "candidate blocks";
"DeepSeek-V4.1-Flash 结构说明" §5.2; "万字长文解析DeekSeekV4.1flash" §4 and
appendix A.11):

* the FULL layer's own score row (the same logits its top-512 is taken from)
  is cut into blocks of 8 consecutive rows, the index plane's page height;
* a block's score is the largest score in it, where a NaN counts as -inf and
  every other value is first clipped to the largest finite float;
* the newest block -- the one holding the newest visible row, possibly only
  partly filled -- is pinned to +inf so no other block can outrank it;
* the 2048 best blocks are kept, written in ascending block order and padded
  with -1; the table doubles as a block table for the REINDEX layers.

Readings taken where the pages are silent:

* "clipped to the largest finite float" is read for both signs and in float32
  (the scores' precision): +inf -> FLT_MAX, -inf -> -FLT_MAX, finite values
  unchanged.  NaN -> -inf happens first, so an all-NaN block scores -inf, below
  a block of -inf scores (which scores -FLT_MAX);
* only visible rows (row < floor((pos+1)/m)) take part: blocks 0 ..
  ceil(n_vis/8) - 1 are the candidates and the newest is block
  ceil(n_vis/8) - 1, pinned whether it is full or not;
* ranking among blocks follows the top-k contract (score descending, lower
  block id first on ties).

Pins (tests/test_oracle_candidates.py): pure-Python brute force on small rows,
crafted NaN / +-inf / tie cases, the pool's closed-form size and the newest
block's membership, and the property that makes the pool sound: with fewer
than 2048 selected rows, every row of the FULL top-k lies in a pool block, so
REINDEX over the pool with the same query reproduces the FULL selection.
"""

import numpy as np

from .topk import topk_row

FLT_MAX = float(np.finfo(np.float32).max)


def n_pool_blocks(n_vis, block_rows):
    """Candidate blocks of a row with n_vis visible rows: ceil(n_vis / block_rows)."""
    return (int(n_vis) + int(block_rows) - 1) // int(block_rows)


def block_maxima_row(scores_row, n_vis, block_rows):
    """Block scores of one FULL score row (float64 [ceil(n_vis/B)]), newest block pinned to +inf."""
    nb = n_pool_blocks(n_vis, block_rows)
    s = np.asarray(scores_row, dtype=np.float64)[: int(n_vis)]
    s = np.where(np.isnan(s), -np.inf, np.clip(s, -FLT_MAX, FLT_MAX))
    out = np.empty(nb, dtype=np.float64)
    for b in range(nb):
        out[b] = s[b * block_rows: (b + 1) * block_rows].max()
    if nb > 0:
        out[nb - 1] = np.inf
    return out


def candidate_pool_row(scores_row, n_vis, block_rows, n_cand):
    """The n_cand best blocks of one row: int32 [n_cand], ascending, -1 padded."""
    m = block_maxima_row(scores_row, n_vis, block_rows)
    return topk_row(m, np.ones(m.shape[0], dtype=bool), n_cand)


def candidate_pool(scores, pos, ratio, block_rows, n_cand):
    """Candidate blocks [rows, n_cand] from FULL scores [rows, width]."""
    rows = scores.shape[0]
    out = np.empty((rows, n_cand), dtype=np.int32)
    for r in range(rows):
        nv = min((int(pos[r]) + 1) // int(ratio), scores.shape[1])
        out[r] = candidate_pool_row(scores[r], nv, block_rows, n_cand)
    return out

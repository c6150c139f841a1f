"""Per-row top-k selection with the ordering contract (oracle; test infrastructure only).

What the pages fix: k = 512 per query row; the result is the selected row
indices in ascending order, padded with -1 when the row has fewer than k valid
columns ("DeepSeek-V4.1-Flash 架构解剖", fig. 2d REUSE: selected [rows, 512]
ascending, -1 filled; special module "indexer": a -1 means the history is
shorter than 512 rows, never "an empty pick").

Readings taken where the pages are silent:

* ranking is by score descending, ties broken by the lower column index;
* NaN ranks as -inf (the pages state this for the block maxima of the
  candidate-pool stage, fig. 3b); -0 and +0 are equal scores;
* only valid columns are candidates: FULL columns c < floor((pos+1)/m),
  REINDEX columns whose candidate block is not -1 and whose row is visible;
* the output lists the chosen columns in increasing column order, mapped to
  plane rows (identity for FULL, cand[i]*B + t for REINDEX, which is
  increasing in the column when candidate blocks are ascending).

Pins (tests/test_oracle_topk.py): brute force with Python's ``sorted`` on
crafted ties, NaN, +-0, -inf and short rows, plus random small rows.
"""

import numpy as np


def topk_row(scores, valid, k, col_to_row=None):
    """Top-k of one score row; returns int32 [k], ascending, -1 padded."""
    scores = np.asarray(scores, dtype=np.float64)
    valid = np.asarray(valid, dtype=bool)
    cols = np.nonzero(valid)[0]
    s = scores[cols].copy()
    s[np.isnan(s)] = -np.inf
    order = np.lexsort((cols, -s))           # primary: score descending; then column ascending
    chosen = np.sort(cols[order[:k]])
    if col_to_row is not None:
        chosen = np.asarray(col_to_row, dtype=np.int64)[chosen]
    out = np.full(k, -1, dtype=np.int32)
    out[: chosen.shape[0]] = chosen
    return out


def topk_full(scores, pos, ratio, k):
    """FULL top-k over [rows, width] scores with validity c < floor((pos+1)/ratio)."""
    rows, width = scores.shape
    out = np.empty((rows, k), dtype=np.int32)
    cols = np.arange(width)
    for r in range(rows):
        nv = (int(pos[r]) + 1) // int(ratio)
        out[r] = topk_row(scores[r], cols < nv, k)
    return out


def topk_reindex(scores, pos, ratio, cand, block_rows, k):
    """REINDEX top-k: columns map to plane rows through the candidate blocks."""
    rows, width = scores.shape
    out = np.empty((rows, k), dtype=np.int32)
    for r in range(rows):
        nv = (int(pos[r]) + 1) // int(ratio)
        c = np.asarray(cand[r], dtype=np.int64)
        prow = np.repeat(c, block_rows) * block_rows + np.tile(np.arange(block_rows), c.shape[0])
        valid = (np.repeat(c, block_rows) >= 0) & (prow < nv)
        out[r] = topk_row(scores[r], valid, k, col_to_row=prow)
    return out

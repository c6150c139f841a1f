"""Lightning-indexer scores, FULL and REINDEX (oracle; test infrastructure only).

Definition.  For query row r with indexer heads h < H_I, per-head query
qI[r,h,:] (dimension D_I), head weights w[r,h] and an index-key row k[c,:]:

    score[r,c] = tau_I * sum_h w[r,h] * ReLU(<qI[r,h,:], k[c,:]>),
    tau_I = D_I^-1/2 * H_I^-1/2.

* The weighted head sum, the raw (activation-free) weights and the two
  inverse square roots come from the anatomy page ("DeepSeek-V4.1-Flash
  架构解剖", special module "indexer", fig. 3b and the score formula under it)
  and from the V4-Pro page ("DeepSeek-V4-Pro 架构解剖", special module
  "indexer", score formula, which has 64 heads).
* The per-head ReLU is the long essay's indexer pseudo-code
  ("万字长文解析DeekSeekV4.1flash", appendix A.15.2) and the overview's decode
  walk-through ("DeepSeek-V4.1 模型结构（0）", decode walk-through: dot, ReLU,
  head-weighted sum).  The anatomy formula omits it; reading taken: ReLU on,
  with a switch kept for tests.
* FULL scores every visible row c < floor((pos+1)/m) of the plane; each row
  computes only up to its visible length (anatomy page, fig. 3b).
* REINDEX re-scores only candidate rows: column i*B + t of the score row is
  plane row cand[r,i]*B + t (B = 8 rows per block), valid iff cand[r,i] != -1
  and that row is visible (anatomy page, fig. 2c REINDEX and fig. 3b second
  stage; essay appendix A.15.2: gather first, then score).
* Columns that are not valid hold -inf.
* An FP8 query's per-(token, head) scale is folded into w upstream (anatomy
  page, fig. 3b: "the FP32 scale is folded into w"), so ``w`` here is the
  effective weight and ``qI`` the decoded query codes.

Pins (tests/test_oracle_indexer.py): pure-Python loop evaluation on tiny
inputs; REINDEX equals FULL-then-mask; the scale helper against the printed
32-head form 1/(sqrt(128)*sqrt(32)).
"""

import math

import numpy as np

from .geometry import n_visible


def indexer_scale(heads, dim):
    """tau_I = dim^-1/2 * heads^-1/2."""
    return 1.0 / (math.sqrt(dim) * math.sqrt(heads))


def score_rows(q_row, w_row, krows, scale, relu=True):
    """Scores of one query row against the given key rows (float64 [C])."""
    q_row = np.asarray(q_row, dtype=np.float64)          # [H, D]
    w_row = np.asarray(w_row, dtype=np.float64)          # [H]
    krows = np.asarray(krows, dtype=np.float64)          # [C, D]
    dots = krows @ q_row.T                                # [C, H]
    if relu:
        dots = np.maximum(dots, 0.0)
    return scale * (dots @ w_row)


def scores_full(q, w, plane_of_row, pos, ratio, scale, width, relu=True):
    """FULL scores [rows, width]; ``plane_of_row(r)`` gives row r's decoded plane [N, D]."""
    rows = q.shape[0]
    out = np.full((rows, width), -np.inf, dtype=np.float64)
    for r in range(rows):
        nv = int(n_visible(pos[r], ratio))
        assert nv <= width
        if nv == 0:
            continue
        plane = plane_of_row(r)
        out[r, :nv] = score_rows(q[r], w[r], plane[:nv], scale, relu)
    return out


def reindex_rows(cand_row, block_rows, nv):
    """Plane row of each REINDEX column, and whether the column is valid."""
    cand_row = np.asarray(cand_row, dtype=np.int64)
    nb = cand_row.shape[0]
    rows = np.repeat(cand_row, block_rows) * block_rows + np.tile(np.arange(block_rows), nb)
    valid = (np.repeat(cand_row, block_rows) >= 0) & (rows < nv)
    return rows, valid


def scores_reindex(q, w, plane_of_row, pos, ratio, cand, block_rows, scale, relu=True):
    """REINDEX scores [rows, n_blocks*block_rows]."""
    rows, nb = cand.shape
    width = nb * block_rows
    out = np.full((rows, width), -np.inf, dtype=np.float64)
    for r in range(rows):
        nv = int(n_visible(pos[r], ratio))
        prow, valid = reindex_rows(cand[r], block_rows, nv)
        if not valid.any():
            continue
        plane = plane_of_row(r)
        cols = np.nonzero(valid)[0]
        out[r, cols] = score_rows(q[r], w[r], plane[prow[cols]], scale, relu)
    return out


def score_abs_bound(q_row, w_row, krows, scale):
    """A = tau_I * sum_h |w_h| * sum_d |q_hd * k_d| per key row: the scale of rounding error."""
    q_row = np.abs(np.asarray(q_row, dtype=np.float64))
    krows = np.abs(np.asarray(krows, dtype=np.float64))
    return scale * ((krows @ q_row.T) @ np.abs(np.asarray(w_row, dtype=np.float64)))

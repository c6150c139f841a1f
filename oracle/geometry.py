"""Integer geometry of one CSA2 query: which rows it may see (oracle; test infrastructure only).

* Compressed rows.  Row j of an owner plane with compression ratio m pools
  tokens j*m .. j*m+m-1 and is stored already rotated at position j*m
  ("DeepSeek-V4.1-Flash 结构说明", section 4.1 and section 6.2).  It becomes
  visible only once the query has reached the last token of its group
  (same page, section 4.1: the group-causal mask).  Reading: the query at
  ``pos`` completes the group containing ``pos`` itself, so row j is visible
  iff (j+1)*m - 1 <= pos, i.e. j < floor((pos+1)/m).  The anatomy page
  ("DeepSeek-V4.1-Flash 架构解剖", special module "indexer", the visible-prefix
  paragraph) states the same closed form, min((pos+1)/ratio, 512) slots.
* SWA window.  Each layer keeps a 128-slot ring; the query sees its causal
  window of the last W positions including itself, min(pos+1, W) entries
  (anatomy page, fig. 2a WINDOW; structure page section 4.4 step 4).  In
  decode, slot s of the ring holds position a(s) = pos - ((pos - s) mod W)
  (the ring is overwritten at start_pos mod 128, structure page section 4.4
  step 3); a slot whose position would be negative has never been written and
  is masked.
* Linear window (prefill chunk).  Row t of a linear SWA array holds position
  pos0 + t; the query at pos sees positions max(0, pos-W+1) .. pos.

Pins (tests/test_oracle_geometry.py): the closed forms are compared against a
brute-force simulation of ring writes and of the group-completion rule, and the
property that no token is ever invisible to both branches is checked
exhaustively for small windows and ratios.
"""

import numpy as np


def n_visible(pos, ratio):
    """Number of compressed rows visible to a query at absolute position ``pos``."""
    pos = np.asarray(pos, dtype=np.int64)
    return (pos + 1) // int(ratio)


def ring_slot_positions(pos, window):
    """Absolute position held by each ring slot for a decode query at ``pos``; -1 if unwritten."""
    pos = int(pos)
    out = np.empty(window, dtype=np.int64)
    for s in range(window):
        a = pos - ((pos - s) % window)
        out[s] = a if a >= 0 else -1
    return out


def linear_window_positions(pos, window):
    """Positions a prefill query at ``pos`` sees in its own sliding window (ascending)."""
    pos = int(pos)
    return np.arange(max(0, pos - window + 1), pos + 1, dtype=np.int64)


def compressed_rows_covering(pos_token, ratio):
    """Compressed row that pools absolute token ``pos_token``."""
    return int(pos_token) // int(ratio)

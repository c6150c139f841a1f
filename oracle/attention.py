"""Single-softmax sink attention over SWA + selected compressed rows (oracle; test infrastructure only).

Definition (one query row, head h, entry multiset S):

    s_j   = tau * <q_h, kv_j>,                          tau = D^-1/2
    out_h = sum_{j in S} e^{s_j} kv_j / (e^{sink_h} + sum_{j in S} e^{s_j})

* K and V are the same stored row; one KV head is shared by all query heads
  ("DeepSeek-V4.1-Flash 架构解剖", "四种层合并出来的是什么形状": the kernel takes a
  single KV tensor, 64 heads share the same N <= 128 + 512 rows).
* SWA rows and selected compressed rows form one entry set and one softmax,
  with no gating and no de-duplication ("DeepSeek-V4.1-Flash 结构说明",
  section 4.1; "万字长文解析DeekSeekV4.1flash", section 5.5).
* attn_sink adds one unscaled logit per head to the denominator only, with no
  value vector ("DeepSeek-V4-Pro 架构解剖", attention merge, fig. 2d formula;
  anatomy page, shared-path figure: attn_sink only in the denominator).
* tau = 1/sqrt(512) for D = 512, no YaRN temperature (anatomy page, shared
  path: softmax temperature 1/sqrt(512); structure page section 6.3).
* After the weighted sum the rope tail is rotated back at the query's own
  position (anatomy page, "出来之后"; structure page section 6.1).
* The query arrives already rotated (anatomy page, shared path: Q and the SWA
  KV are rotated together upstream).

Entries: the SWA entries the geometry module marks valid, then every selected
index with 0 <= idx < floor((pos+1)/m) (the group-causal mask); -1 padding and
out-of-range indices are skipped.  An empty entry set gives a zero output
(reading: it cannot occur, the query always sees itself through its window).

The softmax is evaluated stably by subtracting M = max(sink_h, max_j s_j) from
every exponent, which leaves the defined value unchanged.

Pins (tests/test_oracle_attention.py): equality with dense masked attention
when k covers every visible row (scipy softmax with an appended sink column);
plain softmax attention from torch's scaled_dot_product_attention when the
sink is -inf; probability mass plus sink mass equals 1; closed forms for a
single entry, constant rows and q = 0; difference from two separate softmaxes
added together; multiset semantics of repeated indices.
"""

import numpy as np

from .geometry import n_visible, ring_slot_positions, linear_window_positions
from .rope import rotate_tail


def sink_softmax_weights(q, rows, sink, tau):
    """Probabilities p[h, j] over the entries and the sink mass p_sink[h]."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    if rows.shape[0] == 0:
        return np.zeros((q.shape[0], 0)), np.ones(q.shape[0])
    s = tau * (q @ rows.T)                                       # [H, E]
    m = np.maximum(sink, s.max(axis=1))
    e = np.exp(s - m[:, None])
    es = np.exp(sink - m)
    denom = es + e.sum(axis=1)
    return e / denom[:, None], es / denom


def sink_attention(q, rows, sink, tau):
    """out[h, :] for one query row over the entry rows [E, D]."""
    rows = np.asarray(rows, dtype=np.float64)
    if rows.shape[0] == 0:
        return np.zeros_like(np.asarray(q, dtype=np.float64))
    p, _ = sink_softmax_weights(q, rows, sink, tau)
    return p @ rows


def entries_decode(pos, idx_row, main_plane, ring, ratio):
    """Entry rows for a decode query: valid ring slots, then valid selected rows."""
    window = ring.shape[0]
    slot_pos = ring_slot_positions(pos, window)
    parts = [ring[slot_pos >= 0]]
    nv = int(n_visible(pos, ratio))
    idx = np.asarray(idx_row, dtype=np.int64)
    sel = idx[(idx >= 0) & (idx < nv)]
    parts.append(main_plane[sel])
    return np.concatenate(parts, axis=0)


def entries_prefill(pos, idx_row, main_plane, swa_linear, swa_pos0, window, ratio):
    """Entry rows for a prefill query whose SWA source is a linear array starting at swa_pos0."""
    wpos = linear_window_positions(pos, window)
    t = wpos - int(swa_pos0)
    t = t[(t >= 0) & (t < swa_linear.shape[0])]
    parts = [swa_linear[t]]
    nv = int(n_visible(pos, ratio))
    idx = np.asarray(idx_row, dtype=np.int64)
    sel = idx[(idx >= 0) & (idx < nv)]
    parts.append(main_plane[sel])
    return np.concatenate(parts, axis=0)


def attend(q, pos, rows, sink, tau, freqs):
    """Sink attention of one query row followed by the inverse rotation of the rope tail."""
    out = sink_attention(q, rows, sink, tau)
    return rotate_tail(out, pos, freqs, inverse=True)


def decode(q, pos, idx, main_of_row, ring_of_row, sink, tau, freqs, ratio):
    """Whole decode call: q [rows, H, D] -> out [rows, H, D] (float64)."""
    out = np.empty(q.shape, dtype=np.float64)
    for r in range(q.shape[0]):
        rows = entries_decode(pos[r], idx[r], main_of_row(r), ring_of_row(r), ratio)
        out[r] = attend(q[r], pos[r], rows, sink, tau, freqs)
    return out


def prefill(q, pos, idx, main_plane, swa_linear, swa_pos0, window, sink, tau, freqs, ratio):
    """Whole prefill call over one sequence: q [rows, H, D] -> out [rows, H, D] (float64)."""
    out = np.empty(q.shape, dtype=np.float64)
    for r in range(q.shape[0]):
        rows = entries_prefill(pos[r], idx[r], main_plane, swa_linear, swa_pos0, window, ratio)
        out[r] = attend(q[r], pos[r], rows, sink, tau, freqs)
    return out

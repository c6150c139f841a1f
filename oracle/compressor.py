"""The FULL layer's write path: compressor, main row and index key (oracle; test infrastructure only).

What one FULL owner layer writes for the tokens of a step, float64:

1. Projections of each token's hidden row: kv = wkv . x and, at ratio 2, the
   gate score = wgate . x (both [512]; "DeepSeek-V4.1-Flash 架构解剖", special
   module "compressor": wkv / wgate, pooling in FP32).
2. Pooling ("万字长文解析DeekSeekV4.1flash" appendix A.15.1, §6.3): groups of
   ``ratio`` consecutive positions [j*m, j*m + m - 1] with no overlap; per
   channel, a softmax over the group's positions of the gate scores weights the
   kv values.  At ratio 1 the group is one token and the weight is 1 (no gate).
   The absolute-position bias of the previous generation is all zeros and left
   out (anatomy page, "ape 在这里是一串零").
3. RMSNorm of the pooled latent with a learned weight (appendix A.15.1).
4. Main row: the normalised latent with its last 64 dims rotated at the
   group's first position j*m ("DeepSeek-V4.1-Flash 结构说明" §4: a compressed
   entry is rotated at the position of its group's first token).
5. Index key: wk . (normalised latent before rotation) [128], then k_norm,
   then the same rotation of its last 64 dims (anatomy page, special module
   "indexer", key side; special module "compressor": the indexer's wk reads the
   pre-rotation latent, the two branches fork after the RMSNorm).  k_norm is
   read as an RMSNorm with a learned weight like the pages' other norms (the
   pages name it without its form).
6. Incomplete groups: at ratio 2 a group whose second token has not arrived
   produces no row; its first token's kv and score wait in a per-sequence tail
   state (essay §6.2; structure page §4.4 note on odd lengths).

Quantisation to the planes' formats is ``quantize``; this module returns
float64 rows.

Pins (tests/test_oracle_compressor.py): the pooling weights against scipy's
softmax; equal gate scores give the plain mean; a gate score far above the
other selects its token; adding a constant to a channel's scores changes
nothing; ratio 1 equals the RMSNorm of the projection; the RMSNorm output of a
unit weight has root-mean-square 1 (up to eps); the rotation preserves each
pair's norm and its inverse returns the pre-rotation rows (and the pre-rotation
dims are untouched); the index key is the normalised projection of the
pre-rotation latent, not of the rotated row; splitting one token sequence over
several calls through the tail state gives the rows of one call.
"""

import numpy as np

from . import rope


def rms_norm(v, weight, eps):
    """v [..., n] / sqrt(mean(v^2) + eps) * weight."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def project(x, w):
    """x [..., d_in] times w [d_out, d_in] transposed -> [..., d_out]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def pool(kvs, scores):
    """Per-channel softmax pooling over a group: kvs, scores [m, n] -> [n]."""
    kvs = np.asarray(kvs, dtype=np.float64)
    s = np.asarray(scores, dtype=np.float64)
    mx = np.max(s, axis=0, keepdims=True)
    e = np.exp(s - mx)
    return np.sum(e * kvs, axis=0) / np.sum(e, axis=0)


def finish_group(kvs, scores, j, ratio, norm_w, eps, wk, knorm_w, k_eps, freqs):
    """Rows written for group j: (main row [512], index key [128], pre-rotation latent [512])."""
    if ratio == 1:
        latent = np.asarray(kvs, dtype=np.float64)[0]
    else:
        latent = pool(kvs, scores)
    latent = rms_norm(latent, norm_w, eps)
    p = j * ratio
    main = rope.rotate_tail(latent, p, freqs)
    key = rms_norm(project(latent, wk), knorm_w, k_eps)
    key = rope.rotate_tail(key, p, freqs)
    return main, key, latent


def compress_call(x, pos, slot, ratio, wkv, wgate, norm_w, eps, wk, knorm_w, k_eps, freqs, tail_kv=None,
                  tail_score=None):
    """One call over token rows x [R, d_in] at positions pos [R] of sequences slot [R].

    Rows of one sequence are consecutive in the call with consecutive
    positions.  At ratio 2 a row at an odd position completes group pos // 2
    with the previous position: the previous row of the call when it belongs to
    the same sequence, else the sequence's tail state (tail_kv / tail_score
    [slots, 512]).  A row at an even position that ends its sequence's rows in
    the call leaves its kv and score in the tail state.

    Returns (rows, tail_kv, tail_score) where rows maps the emitting row index r
    to (j, main, key, latent) and the tail arrays are updated copies.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    slot = np.asarray(slot, dtype=np.int64)
    kv = project(x, wkv)
    sc = project(x, wgate) if ratio == 2 else None
    tail_kv = None if tail_kv is None else np.array(tail_kv, dtype=np.float64, copy=True)
    tail_score = None if tail_score is None else np.array(tail_score, dtype=np.float64, copy=True)
    rows = {}
    n = x.shape[0]
    for r in range(n):
        p = int(pos[r])
        if ratio == 1:
            rows[r] = (p,) + finish_group(kv[r:r + 1], None, p, 1, norm_w, eps, wk, knorm_w, k_eps, freqs)
            continue
        if p % 2 == 1:
            if r > 0 and slot[r - 1] == slot[r] and pos[r - 1] == p - 1:
                kv0, s0 = kv[r - 1], sc[r - 1]
            else:
                kv0, s0 = tail_kv[slot[r]], tail_score[slot[r]]
            j = p // 2
            rows[r] = (j,) + finish_group(np.stack([kv0, kv[r]]), np.stack([s0, sc[r]]), j, 2, norm_w, eps, wk,
                                          knorm_w, k_eps, freqs)
        else:
            last = r + 1 >= n or slot[r + 1] != slot[r]
            if last:
                tail_kv[slot[r]] = kv[r]
                tail_score[slot[r]] = sc[r]
    return rows, tail_kv, tail_score


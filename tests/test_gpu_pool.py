"""GPU parity of the candidate-pool builder (block scores and top-2048 blocks) against the oracle.

Block scores are maxima and clips of the scores, so they are compared bit for
bit with the oracle's block scores of the same GPU scores, and the kept blocks
bit for bit with the oracle's pool of those scores.  End to end (oracle scores
instead of GPU scores) the pool may differ only in blocks whose oracle block
score lies within the scores' rounding band of the last kept block.  The
pool's soundness property -- every row of the FULL top-k lies in a kept block,
so REINDEX over the pool selects what FULL selects -- is checked on the GPU's
own results.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs

from harness import (SCORE_TOL, gpu_scores, gpu_topk, oracle_score_bound, oracle_scores, oracle_topk,
                     topk_band_mismatches)

pytestmark = pytest.mark.gpu


def _pool(pos, ratio, n_cand, **kw):
    import sparse_latent_attention_amd as csa2
    cand = torch.empty(pos.shape[0], n_cand, dtype=torch.int32, device=pos.device)
    csa2.candidate_pool(pos, ratio, cand, **kw)
    return cand


def _valid_blocks(pos, ratio, width, B):
    nv = np.minimum((pos + 1) // ratio, width)
    return (nv + B - 1) // B


@pytest.mark.parametrize("rows,width,B,n_cand,ratio,kind", [
    (6, 3001, 8, 100, 1, "normal"),        # narrow select, ragged last block
    (4, 1 << 20, 8, 2048, 1, "normal"),    # the 1M-column decode shape (131072 blocks, wide select)
    (5, 200003, 8, 2048, 2, "special"),    # NaN / +-inf / ties, ratio 2, ragged width (scalar loads)
    (3, 50000, 4, 700, 1, "ties"),         # few distinct values: every block ties
    (3, 65536, 64, 2048, 1, "normal"),     # more kept blocks than blocks
    (4, 40000, 16, 16, 1, "short"),        # short histories, tiny pool
])
def test_pool_from_scores(rows, width, B, n_cand, ratio, kind):
    print(f"\n[pool] rows={rows} width={width} B={B} n_cand={n_cand} ratio={ratio} kind={kind}", flush=True)
    rng = np.random.default_rng(width + B)
    s = rng.standard_normal((rows, width)).astype(np.float32)
    pos = np.full(rows, ratio * width - 1, dtype=np.int64)
    if kind == "special":
        s[0, rng.random(width) < 0.2] = np.nan
        s[1, rng.random(width) < 0.001] = np.inf
        s[1, rng.random(width) < 0.001] = np.float32(3.4028235e38)
        s[2] = -np.inf
        s[3, :] = np.nan
        s[4, rng.random(width) < 0.5] = -0.0
        pos[2] = 2 * 777 + 1
    if kind == "ties":
        s = rng.integers(0, 3, (rows, width)).astype(np.float32)
    if kind == "short":
        pos[:] = [0, 5, 16 * 3, 1000]
    sc = torch.from_numpy(s).cuda()
    pt = torch.from_numpy(pos).cuda()
    got = _pool(pt, ratio, n_cand, scores=sc, block_rows=B).cpu().numpy()
    ref = oracle.candidates.candidate_pool(s.astype(np.float64), pos, ratio, B, n_cand)
    assert np.array_equal(got, ref)


FULL_CASES = {
    "lowp_small": CONFIGS["lowp_pool_decode_1m"].replace(batch=7, q_tokens=7, context=20003, ragged=True),
    "full_decode_small": CONFIGS["full_decode_64k"].replace(batch=6, q_tokens=6, context=30001, ragged=True,
                                                            pool_blocks=300),
    "prefill_small": CONFIGS["prefill_4096_at_128k"].replace(q_tokens=300, context=6000, reuse_layers=0,
                                                             pool_blocks=64),
    "tiny_full_fp32": CONFIGS["tiny_full_fp32"].replace(pool_blocks=8),
}


@pytest.mark.parametrize("name", list(FULL_CASES))
def test_indexer_block_max_and_pool(name):
    """Block scores written in the scoring pass == oracle block scores of the GPU scores; the pool from
    them == the pool computed from the scores == the oracle pool; soundness against FULL top-k."""
    cfg = FULL_CASES[name]
    B, n_cand = cfg.block_rows, cfg.pool_blocks
    print(f"\n[indexer block_max] {name} rows={cfg.q_tokens} width={cfg.width}", flush=True)
    x = make_inputs(cfg, 41, device="cuda")
    rows = cfg.q_tokens
    nb = -(-cfg.width // B)
    bm = torch.full((rows, nb), 12345.0, dtype=torch.float32, device="cuda")   # every element is written
    scores = gpu_scores(cfg, x, block_max=bm)
    plain = gpu_scores(cfg, x)
    assert torch.equal(scores, plain), "the block-max variant must not change the scores"
    s_np = scores.cpu().numpy().astype(np.float64)
    pos = x["pos"].cpu().numpy()
    nbv = _valid_blocks(pos, cfg.ratio, cfg.width, B)
    bm_np = bm.cpu().numpy().astype(np.float64)
    for r in range(rows):
        nv = min((int(pos[r]) + 1) // cfg.ratio, cfg.width)
        ref = oracle.candidates.block_maxima_row(s_np[r], nv, B)
        assert np.array_equal(bm_np[r, :nbv[r]], ref), f"row {r}"
        assert np.all(bm_np[r, nbv[r]:] == -np.inf)
    pos_t = x["pos"]
    p_fused = _pool(pos_t, cfg.ratio, n_cand, block_max=bm, width=cfg.width, block_rows=B).cpu().numpy()
    p_scores = _pool(pos_t, cfg.ratio, n_cand, scores=scores, block_rows=B).cpu().numpy()
    ref = oracle.candidates.candidate_pool(s_np, pos, cfg.ratio, B, n_cand)
    assert np.array_equal(p_fused, ref)
    assert np.array_equal(p_scores, ref)
    # soundness on the GPU's own results: each FULL top-k row lies in a kept block
    idx = gpu_topk(cfg, x, scores).cpu().numpy()
    if cfg.topk < n_cand:
        for r in range(rows):
            kept = set(int(b) for b in p_fused[r] if b >= 0)
            assert all(int(v) // B in kept for v in idx[r] if v >= 0), f"row {r}"


def test_reindex_over_gpu_pool_selects_full():
    """The pages' purpose of the pool, end to end: REINDEX over the GPU-built pool with the same indexer
    query selects the FULL layer's rows (differences only inside the scores' rounding band)."""
    cfg = FULL_CASES["lowp_small"]
    x = make_inputs(cfg, 43, device="cuda")
    rows = np.arange(cfg.q_tokens)
    nb = -(-cfg.width // cfg.block_rows)
    bm = torch.empty(cfg.q_tokens, nb, dtype=torch.float32, device="cuda")
    gpu_scores(cfg, x, block_max=bm)
    pool = _pool(x["pos"], cfg.ratio, cfg.pool_blocks, block_max=bm, width=cfg.width, block_rows=cfg.block_rows)
    rcfg = cfg.replace(index_mode="reindex", n_blocks=cfg.pool_blocks, pool_blocks=0)
    xr = dict(x)
    xr["cand"] = pool
    sel = gpu_topk(rcfg, xr, gpu_scores(rcfg, xr)).cpu().numpy()
    s_ref = oracle_scores(cfg, x, rows)
    bound = oracle_score_bound(cfg, x, rows)
    full_ref = oracle_topk(cfg, x, s_ref, rows)
    n_diff, n_bad = topk_band_mismatches(cfg, x, rows, sel, full_ref, s_ref, bound)
    print(f"[reindex over pool] index differences vs oracle FULL {n_diff}, outside the band {n_bad}")
    assert n_bad == 0


def test_pool_end_to_end_band():
    """GPU pool from GPU scores vs oracle pool from oracle scores: differences only near the cut."""
    cfg = FULL_CASES["full_decode_small"]
    x = make_inputs(cfg, 45, device="cuda")
    rows = np.arange(cfg.q_tokens)
    pool = _pool(x["pos"], cfg.ratio, cfg.pool_blocks, scores=gpu_scores(cfg, x), block_rows=cfg.block_rows)
    pool = pool.cpu().numpy()
    s_ref = oracle_scores(cfg, x, rows)
    bound = oracle_score_bound(cfg, x, rows)
    pos = x["pos"].cpu().numpy()
    ref = oracle.candidates.candidate_pool(s_ref, pos, cfg.ratio, cfg.block_rows, cfg.pool_blocks)
    n_diff = 0
    for r in rows:
        diff = set(int(b) for b in pool[r] if b >= 0) ^ set(int(b) for b in ref[r] if b >= 0)
        if not diff:
            continue
        n_diff += len(diff)
        nv = min((int(pos[r]) + 1) // cfg.ratio, cfg.width)
        m = oracle.candidates.block_maxima_row(s_ref[r], nv, cfg.block_rows)
        cut = np.sort(m)[::-1][min(cfg.pool_blocks, len(m)) - 1]
        band = 2 * SCORE_TOL * float(np.max(bound[r][np.isfinite(bound[r])]))
        assert all(abs(m[b] - cut) <= band for b in diff), f"row {r}"
    print(f"[pool end to end] block differences {n_diff}")


def _host_block_keys(s, n_vis, width):
    """Block keys by their definition: the largest key of each 8 valid columns, a NaN counting as
    0x007FFFFE (just below -inf), 0 for a block without valid columns."""
    u = s.astype(np.float32).view(np.uint32).copy()
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    u[u == 0x80000000] = 0
    key = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
    key[nan] = 0x007FFFFE
    key[:, :] = np.where(np.arange(width)[None, :] < n_vis[:, None], key, 0)
    pad = (-width) % 8
    return np.pad(key, ((0, 0), (0, pad))).reshape(s.shape[0], -1, 8).max(axis=2).astype(np.uint32)


@pytest.mark.parametrize("width,n_cand,kind", [(3001, 100, "special"), (1 << 20, 2048, "normal"),
                                               (200003, 2048, "special"), (50000, 700, "ties")])
def test_pool_from_block_keys(width, n_cand, kind):
    """Pool ranking from block keys (score-free route) == the oracle pool of the same scores, with NaN,
    +-inf, FLT_MAX and ties in the scores."""
    rows = 5
    rng = np.random.default_rng(width + n_cand)
    s = rng.standard_normal((rows, width)).astype(np.float32)
    pos = np.full(rows, width - 1, dtype=np.int64)
    if kind == "special":
        s[0, rng.random(width) < 0.3] = np.nan
        s[1, rng.random(width) < 0.002] = np.inf
        s[1, rng.random(width) < 0.002] = np.float32(3.4028235e38)
        s[2] = -np.inf
        s[2, ::3] = np.nan                       # blocks of NaN and -inf: NaN ranks below -inf
        s[3, :] = np.nan
        pos[4] = 777
    if kind == "ties":
        s = rng.integers(0, 3, (rows, width)).astype(np.float32)
    n_vis = np.minimum(pos + 1, width)
    bk = torch.from_numpy(_host_block_keys(s, n_vis, width).view(np.int32)).cuda()
    got = _pool(torch.from_numpy(pos).cuda(), 1, n_cand, block_keys=bk, width=width, block_rows=8).cpu().numpy()
    ref = oracle.candidates.candidate_pool(s.astype(np.float64), pos, 1, 8, n_cand)
    assert np.array_equal(got, ref)

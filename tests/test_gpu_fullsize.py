"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Every call goes through the same prepared C ABI calls bench.py uses (the
library picks chunking and splits from the shapes, so the launches are the
same).  The oracle checks sampled query rows one by one (scores over the whole
row, top-k, attention of every layer); properties that hold at any size are
checked on every row.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs

from harness import (BF16_ATOL, BF16_RTOL, F32_ATOL, F32_RTOL, SCORE_TOL, assert_close, oracle_attention,
                     oracle_score_bound, oracle_scores, oracle_topk, topk_band_mismatches)

pytestmark = pytest.mark.gpu

NAMES = ["tiny_full_fp32", "full_decode_64k", "prefill_4096_at_128k", "reindex_decode_1m", "lowp_full_decode_1m",
         "lowp_pool_decode_1m", "pages_fp4_decode_1m"]


def _run_path(cfg, x):
    """The path exactly as bench.py launches it.  When it keeps the scores on chip, the scores are
    also written by a separate call for the checks, and the score-free top-k must equal topk_select
    over them on every row."""
    from workloads.step import Step
    from harness import gpu_scores, gpu_topk
    step = Step(cfg, x)
    step()
    torch.cuda.synchronize()
    x["_pool"] = step.pool
    if step.score_free:
        scores = gpu_scores(cfg, x)
        ref = gpu_topk(cfg, x, scores)
        torch.cuda.synchronize()
        assert torch.equal(step.idx, ref), "score-free top-k differs from topk_select over the written scores"
        print(f"[{cfg.name}] score-free top-k == topk_select(written scores) on all {cfg.q_tokens} rows")
    else:
        scores = step.scores
    return scores, step.idx, step.outs


def _sample_rows(cfg):
    n = cfg.q_tokens
    if n <= 256:
        picks = [0, n // 2, n - 1] if n > 64 else [0, n - 1]
        if cfg.name == "tiny_full_fp32":
            return np.arange(n)
        return np.array(sorted(set(picks)))
    return np.array([0, 1, 1777, n - 2, n - 1])


@pytest.fixture(scope="module", params=NAMES)
def full(request):
    cfg = CONFIGS[request.param]
    print(f"\n[full] {cfg.name} seed=2 rows={cfg.q_tokens} width={cfg.width} layers={1 + cfg.reuse_layers}",
          flush=True)
    x = make_inputs(cfg, 2, device="cuda")
    torch.cuda.synchronize()
    scores, idx, outs = _run_path(cfg, x)
    yield cfg, x, scores, idx, outs
    del x, scores, idx, outs
    torch.cuda.empty_cache()


def test_every_row_selection_is_well_formed(full):
    cfg, x, scores, idx, _ = full
    ii = idx.cpu().numpy().astype(np.int64)
    pos = x["pos"].cpu().numpy()
    nv = (pos + 1) // cfg.ratio
    for r in range(ii.shape[0]):
        v = ii[r][ii[r] >= 0]
        assert np.all(ii[r][len(v):] == -1)
        assert np.all(np.diff(v) > 0)
        assert len(v) == min(cfg.topk, nv[r] if cfg.index_mode == "full" else len(v))
        assert len(v) == 0 or (v[0] >= 0 and v[-1] < nv[r])
        if cfg.index_mode == "reindex":
            blocks = set(int(b) for b in x["cand"][r].cpu().numpy() if b >= 0)
            assert set((v // cfg.block_rows).tolist()) <= blocks


def test_every_output_finite(full):
    cfg, x, scores, idx, outs = full
    for o in outs:
        assert torch.isfinite(o.float()).all()


def test_sampled_rows_scores_topk_attention(full):
    cfg, x, scores, idx, outs = full
    rows = _sample_rows(cfg)
    s_ref = oracle_scores(cfg, x, rows)
    bound = oracle_score_bound(cfg, x, rows)
    got = scores[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    inval = ~np.isfinite(bound)
    assert np.all(got[inval] == -np.inf) and np.all(s_ref[inval] == -np.inf)
    ratio = float((np.abs(got[~inval] - s_ref[~inval]) / bound[~inval]).max())
    print(f"[{cfg.name}] sampled rows {rows.tolist()[:6]}: score max |d|/A = {ratio:.3e}")
    assert ratio <= SCORE_TOL
    gi = idx[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(gi, oracle_topk(cfg, x, got, rows)), "top-k of the GPU scores is not bit-exact"
    n_diff, n_bad = topk_band_mismatches(cfg, x, rows, gi, oracle_topk(cfg, x, s_ref, rows), s_ref, bound)
    print(f"[{cfg.name}] end-to-end index differences {n_diff}, outside the band {n_bad}")
    assert n_bad == 0
    atol, rtol = (F32_ATOL, F32_RTOL) if cfg.out_dtype == "f32" else (BF16_ATOL, BF16_RTOL)
    for layer, o in enumerate(outs):
        ref = oracle_attention(cfg, x, gi, rows, layer=layer)
        e = assert_close(o[torch.from_numpy(rows).cuda()], ref, atol, rtol, f"{cfg.name} layer {layer}")
        print(f"[{cfg.name}] layer {layer} attention max_abs {e:.3e}")


def test_candidate_pool(full):
    """Every row: the pool is well formed, keeps the newest block and every FULL top-k row's block
    (soundness on the GPU's own scores); sampled rows: bit-exact with the oracle's pool of the GPU scores."""
    cfg, x, scores, idx, _ = full
    if not cfg.pool_blocks:
        pytest.skip("this workload builds no candidate pool")
    pool = x["_pool"].cpu().numpy()
    ii = idx.cpu().numpy()
    pos = x["pos"].cpu().numpy()
    B = cfg.block_rows
    for r in range(pool.shape[0]):
        nv = min((int(pos[r]) + 1) // cfg.ratio, cfg.width)
        v = pool[r][pool[r] >= 0]
        assert np.all(pool[r][len(v):] == -1) and np.all(np.diff(v) > 0)
        assert len(v) == min(cfg.pool_blocks, -(-nv // B))
        assert (nv - 1) // B in set(v.tolist())
        kept = set(v.tolist())
        assert all(int(c) // B in kept for c in ii[r] if c >= 0)
    rows = _sample_rows(cfg)
    s_gpu = scores[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    ref = oracle.candidates.candidate_pool(s_gpu, pos[rows], cfg.ratio, B, cfg.pool_blocks)
    assert np.array_equal(pool[rows], ref)

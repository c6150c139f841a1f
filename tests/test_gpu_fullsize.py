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


def _record(cfg, x, **fields):
    """With CSA2_RESULTS_DIR set, merges these measurements into the (workload, seed) record there
    (<workload>_s<seed>[_ragged].json); otherwise does nothing."""
    import json
    import os
    d = os.environ.get("CSA2_RESULTS_DIR")
    if not d:
        return
    os.makedirs(d, exist_ok=True)
    path = os.path.join(d, f"{cfg.name}_s{x['_seed']}{'_ragged' if cfg.ragged else ''}.json")
    rec = json.load(open(path)) if os.path.exists(path) else {"workload": cfg.name, "seed": x["_seed"],
                                                             "ragged": bool(cfg.ragged)}
    rec.update(fields)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)

# (workload, seed, ragged positions).  The two 1M decodes the measurements name run seeds 0, 1 and 2
# plus a ragged-position batch; the 64K decode runs a ragged batch as well; the 64K decode, the prefill
# chunk and the pages' formats run a second seed.
CASES = [("tiny_full_fp32", 2, False), ("full_decode_64k", 2, False), ("full_decode_64k", 0, False),
         ("full_decode_64k", 1, True),
         ("prefill_4096_at_128k", 2, False), ("prefill_4096_at_128k", 0, False),
         ("reindex_decode_1m", 0, False), ("reindex_decode_1m", 1, False), ("reindex_decode_1m", 2, False),
         ("reindex_decode_1m", 3, True), ("reindex_fp8_decode_1m", 2, False), ("reindex_pages_decode_1m", 2, False),
         ("lowp_full_decode_1m", 0, False), ("lowp_full_decode_1m", 1, False), ("lowp_full_decode_1m", 2, False),
         ("lowp_full_decode_1m", 3, True),
         ("lowp_pool_decode_1m", 2, False), ("pages_fp4_decode_1m", 2, False), ("pages_fp4_decode_1m", 0, False),
         ("lowp_owner_decode_1m", 2, False),
         ("prefill_owner_4096_at_128k", 2, False)]


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
        _record(cfg, x, score_free_topk_equals_written_scores_rows=int(cfg.q_tokens))
    else:
        scores = step.scores
    return scores, step.idx, step.outs


def _sample_rows(cfg, seed):
    """Rows the oracle checks one by one: every row of the tiny workload and of the 32-sequence decodes;
    8 rows (first, last and 6 seeded others) of the 64-sequence decodes; 8 rows of a prefill chunk."""
    n = cfg.q_tokens
    if n <= 32 or cfg.name == "tiny_full_fp32":
        return np.arange(n)
    rng = np.random.default_rng(1000 + seed)
    inner = rng.choice(np.arange(2, n - 2), size=4 if n > 256 else 6, replace=False)
    picks = {0, n - 1} | set(int(v) for v in inner)
    if n > 256:
        picks |= {1, 1777, n - 2}
    return np.array(sorted(picks))


@pytest.fixture(scope="module", params=CASES, ids=[f"{n}-s{s}{'-ragged' if r else ''}" for n, s, r in CASES])
def full(request):
    name, seed, ragged = request.param
    cfg = CONFIGS[name].replace(ragged=ragged)
    print(f"\n[full] {cfg.name} seed={seed} ragged={ragged} rows={cfg.q_tokens} width={cfg.width} "
          f"layers={1 + cfg.reuse_layers}", flush=True)
    x = make_inputs(cfg, seed, device="cuda")
    x["_seed"] = seed
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
    rows = _sample_rows(cfg, x["_seed"])
    s_ref = oracle_scores(cfg, x, rows)
    bound = oracle_score_bound(cfg, x, rows)
    got = scores[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    inval = ~np.isfinite(bound)
    assert np.all(got[inval] == -np.inf) and np.all(s_ref[inval] == -np.inf)
    ratio = float((np.abs(got[~inval] - s_ref[~inval]) / bound[~inval]).max())
    print(f"[{cfg.name}] sampled rows {rows.tolist()[:6]}: score max |d|/A = {ratio:.3e}")
    _record(cfg, x, rows_checked=[int(r) for r in rows], score_max_err_over_bound=ratio, score_tol=SCORE_TOL)
    assert ratio <= SCORE_TOL
    gi = idx[torch.from_numpy(rows).cuda()].cpu().numpy()
    exact = bool(np.array_equal(gi, oracle_topk(cfg, x, got, rows)))
    _record(cfg, x, topk_bit_exact_on_gpu_scores=exact)
    assert exact, "top-k of the GPU scores is not bit-exact"
    n_diff, n_bad = topk_band_mismatches(cfg, x, rows, gi, oracle_topk(cfg, x, s_ref, rows), s_ref, bound)
    print(f"[{cfg.name}] end-to-end index differences {n_diff}, outside the band {n_bad}")
    _record(cfg, x, topk_index_differences_vs_oracle_scores=int(n_diff), topk_differences_outside_band=int(n_bad))
    assert n_bad == 0
    atol, rtol = (F32_ATOL, F32_RTOL) if cfg.out_dtype == "f32" else (BF16_ATOL, BF16_RTOL)
    errs = []
    for layer, o in enumerate(outs):
        ref = oracle_attention(cfg, x, gi, rows, layer=layer)
        got_o = o[torch.from_numpy(rows).cuda()]
        e = assert_close(got_o, ref, atol, rtol, f"{cfg.name} layer {layer}")
        rel = float((np.abs(got_o.float().cpu().numpy().astype(np.float64) - ref) / np.maximum(np.abs(ref), atol)).max())
        errs.append({"layer": layer, "max_abs": float(e), "max_rel_over_max_abs_atol": rel})
        print(f"[{cfg.name}] layer {layer} attention max_abs {e:.3e}")
    _record(cfg, x, attention_errors=errs, attention_atol=atol, attention_rtol=rtol)


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
    rows = _sample_rows(cfg, x["_seed"])
    s_gpu = scores[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    ref = oracle.candidates.candidate_pool(s_gpu, pos[rows], cfg.ratio, B, cfg.pool_blocks)
    assert np.array_equal(pool[rows], ref)


def _row_error_bound(fmt, ref, scales):
    """Largest error the plane format's rounding allows per element of the float64 rows ``ref``
    (scales: the decoded per-element scale, for the block-scaled formats)."""
    if fmt == "bf16":
        return np.abs(ref) * 2.0 ** -8
    if fmt == "fp8":   # E4M3: half a step is <= 2^-4 relative for normals, 2^-10 * scale below
        return np.maximum(np.abs(ref) * 2.0 ** -4, scales * 2.0 ** -10)
    return scales * 1.0    # E2M1: steps of at most 2 (between 4 and 6) times the block scale


def test_owner_rows_written(full):
    """The write path of an owner layer: the compressed rows it appended for sampled query rows, decoded from
    the planes, equal the oracle's rows within the formats' rounding (plus the float32 tolerance)."""
    cfg, x, *_ = full
    if not cfg.d_model:
        pytest.skip("this workload appends no rows")
    from harness import to_numpy_f64
    c = x["compress"]
    rows = _sample_rows(cfg, x["_seed"])
    if cfg.ratio == 2:
        rows = np.array(sorted({int(r) | 1 for r in rows if (int(r) | 1) < cfg.q_tokens}))  # rows that emit
    f64 = lambda t: None if t is None else t.detach().cpu().double().numpy()
    freqs = oracle.rope.inv_freq(cfg.rope_dim, cfg.rope_theta, cfg.yarn_factor, cfg.yarn_orig)
    pos = c["pos"].cpu().numpy()
    for r in rows:
        sub = [r - 1, r] if cfg.ratio == 2 else [r]
        tk = None if c["tail_kv"] is None else f64(c["tail_kv"])
        ts = None if c["tail_score"] is None else f64(c["tail_score"])
        got_rows, _, _ = oracle.compressor.compress_call(
            f64(c["x"][sub]), pos[sub], np.zeros(len(sub), dtype=np.int64), cfg.ratio, f64(c["wkv"]), f64(c["wgate"]),
            f64(c["norm_w"]), 1e-6, f64(c["wk"]), f64(c["knorm_w"]), 1e-6, freqs, tk, ts)
        j, m_ref, k_ref, _ = got_rows[len(sub) - 1]
        n = int(c["row_base"][r]) + j
        main = x["main"].reshape(-1, x["main"].shape[-1])[n:n + 1]
        ms = None if x["main_scale"] is None else x["main_scale"].reshape(-1, x["main_scale"].shape[-1])[n:n + 1]
        kI = x["kI"].reshape(-1, x["kI"].shape[-1])[n:n + 1]
        ks = None if x["kI_scale"] is None else (x["kI_scale"].reshape(-1)[n:n + 1] if cfg.idx_dtype == "fp8"
                                                 else x["kI_scale"].reshape(-1, x["kI_scale"].shape[-1])[n:n + 1])
        m_got = to_numpy_f64(main, cfg.main_dtype, ms)[0]
        k_got = to_numpy_f64(kI, cfg.idx_dtype, ks)[0]
        # per-element scales of the block formats, from the stored scale bytes
        if cfg.main_dtype == "fp4":
            m_sc = np.repeat(oracle.formats.e8m0_to_f64(ms.cpu().numpy()[0]), 32)
        elif cfg.main_dtype == "nvfp4":
            m_sc = np.repeat(oracle.formats.decode_fp8_values(main.cpu().numpy()[0, 256:]), 16)
        else:
            m_sc = None
        k_sc = (np.full(128, float(ks.cpu()[0])) if cfg.idx_dtype == "fp8" else
                np.repeat(oracle.formats.e8m0_to_f64(ks.cpu().numpy()[0]), 32) if cfg.idx_dtype == "fp4" else None)
        slack_m = 1e-5 * (1 + np.abs(m_ref))
        slack_k = 1e-5 * (1 + np.abs(k_ref))
        assert np.all(np.abs(m_got - m_ref) <= _row_error_bound(cfg.main_dtype, m_ref, m_sc) + slack_m), f"row {r}"
        assert np.all(np.abs(k_got - k_ref) <= _row_error_bound(cfg.idx_dtype, k_ref, k_sc) + slack_k), f"row {r}"
    print(f"[{cfg.name}] appended rows of {len(rows)} sampled query rows within the formats' rounding")

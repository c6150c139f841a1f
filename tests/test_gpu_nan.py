"""GPU parity with NaN codes in the stored formats, element by element against the oracle.

E4M3 codes 0x7F / 0xFF and an E8M0 scale byte of 255 are legal bytes of the
planes the path reads and all decode to NaN.  The rules both sides follow:
a NaN dot stays NaN through the indexer's per-head ReLU, so its score is NaN
and ranks as -inf in the top-k; a NaN entry row in attention makes every
output element of its query row NaN (one softmax over all entries); NaN bytes
in rows that are not entries (not selected, outside the window) change
nothing.  The comparisons accept NaN only where the oracle has NaN too.
"""
import numpy as np
import pytest
import torch

from workloads import CONFIGS, make_inputs

from harness import (BF16_ATOL, BF16_RTOL, SCORE_TOL, assert_close, gpu_attention, gpu_scores, gpu_topk, index_scale,
                     oracle_attention, oracle_score_bound, oracle_scores, oracle_topk, topk_band_mismatches)
from workloads.step import index_plane_args

pytestmark = pytest.mark.gpu

LOWP = CONFIGS["lowp_full_decode_1m"].replace(batch=6, q_tokens=6, context=5003, ragged=True)
PAGES = CONFIGS["pages_fp4_decode_1m"].replace(batch=6, q_tokens=6, context=5003, ragged=True)


def _fix_positions(x):
    # every row sees at least 900 compressed rows, so the planted rows below are visible
    x["pos"][:] = torch.tensor([1000, 4000, 5002, 2500, 3333, 900], dtype=torch.int64, device=x["pos"].device)


def _plant_index_nans(cfg, x):
    """NaN in some key rows of each sequence and in one head of the query of row 3."""
    if cfg.idx_dtype == "fp8":
        kI = x["kI"]                      # [B, N, 128] E4M3 codes
        kI[:, 17, 5] = 0x7F
        kI[:, 300, 100] = 0xFF
        kI[:, 301, 0] = 0x7F
        x["qI"][3, 7, 11] = 0xFF          # head 7 of row 3: every dot of that head is NaN
    else:
        ks = x["kI_scale"]                # [B, N, 4] E8M0
        ks[:, 17, 0] = 255
        ks[:, 300, 3] = 255
        ks[:, 301, 1] = 255
        x["qI_scale"][3, 7, 2] = 255


def _check_scores(cfg, x, scores, rows):
    ref = oracle_scores(cfg, x, rows)
    bound = oracle_score_bound(cfg, x, rows)
    got = scores.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN scores differ in position"
    inval = np.isposinf(bound)            # invalid columns (a NaN key row makes its bound NaN, not +inf)
    assert np.all(got[inval] == -np.inf) and np.all(ref[inval] == -np.inf)
    fin = np.isfinite(ref) & ~inval
    assert np.all(np.isfinite(got[fin]))
    ratio = float((np.abs(got[fin] - ref[fin]) / bound[fin]).max())
    assert ratio <= SCORE_TOL, ratio
    n_nan = int(np.isnan(ref).sum())
    assert n_nan >= 3 * len(rows) and np.all(np.isnan(ref[3, :(int(x["pos"][3]) + 1) // cfg.ratio]))
    return ref, bound, got, n_nan


@pytest.mark.parametrize("cfg", [LOWP, PAGES], ids=["fp8_index", "mxfp4_index"])
def test_indexer_and_topk_with_nan_codes(cfg):
    x = make_inputs(cfg, 61, device="cuda")
    _fix_positions(x)
    _plant_index_nans(cfg, x)
    rows = np.arange(cfg.q_tokens)
    scores = gpu_scores(cfg, x)
    idx = gpu_topk(cfg, x, scores)
    torch.cuda.synchronize()
    ref, bound, got, n_nan = _check_scores(cfg, x, scores, rows)
    print(f"[nan {cfg.idx_dtype}] {n_nan} NaN scores, positions identical")
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, oracle_topk(cfg, x, got, rows)), "top-k of the GPU scores is not bit-exact"
    # the NaN key rows are never selected while finite candidates remain
    for r in rows:
        if r != 3:
            assert not ({17, 300, 301} & set(gi[r].tolist()))
    # row 3 scores all NaN: the lowest columns win every tie
    n3 = min(cfg.topk, (int(x["pos"][3]) + 1) // cfg.ratio)
    assert np.array_equal(gi[3, :n3], np.arange(n3))
    n_diff, n_bad = topk_band_mismatches(cfg, x, rows, gi, oracle_topk(cfg, x, ref, rows), ref, bound)
    assert n_bad == 0


@pytest.mark.parametrize("bk16", [False, True])
@pytest.mark.parametrize("base", ["lowp", "pages"])
def test_score_free_topk_with_nan_codes(base, bk16):
    """The score-free route (block keys, 32-bit or their top 16 bits, then re-scoring) returns what
    topk_select returns over the written NaN-bearing scores."""
    import sparse_latent_attention_amd as csa2
    cfg = (LOWP if base == "lowp" else PAGES).replace(context=30011)
    x = make_inputs(cfg, 62, device="cuda")
    _fix_positions(x)
    x["pos"][1] = 30010
    x["pos"][4] = 20000
    _plant_index_nans(cfg, x)
    rows = cfg.q_tokens
    assert csa2.topk_rescore_supported(rows, cfg.width, cfg.topk, fp8=cfg.idx_dtype == "fp8",
                                       fp4=cfg.idx_dtype == "fp4")
    kI, ikw = index_plane_args(cfg, x)
    bkeys = torch.empty(rows, -(-cfg.width // 8), dtype=torch.int16 if bk16 else torch.int32, device="cuda")
    csa2.indexer_score(x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, index_scale(cfg), None,
                       width=cfg.width, block_keys=bkeys, **ikw)
    out = torch.full((rows, cfg.topk), -7, dtype=torch.int32, device="cuda")
    ikw.pop("fp8", None)
    csa2.topk_rescore(x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, index_scale(cfg), out, bkeys,
                      cfg.width, **ikw)
    scores = gpu_scores(cfg, x)
    ref = gpu_topk(cfg, x, scores)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    assert np.isnan(s).sum() >= 3 * rows
    assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy())
    assert np.array_equal(out.cpu().numpy(), oracle_topk(cfg, x, s.astype(np.float64), np.arange(rows)))


def _plant_attention_nans(cfg, x, idx):
    """Row 1: a NaN in one of its selected main rows.  Row 2: a NaN in the ring slot of its own
    position (always in the window).  Row 4: a NaN in a main row it does not select and cannot
    see, and in a ring slot outside its window is impossible (full window), so its output must
    stay finite."""
    B = cfg.batch
    ii = idx.cpu().numpy()
    pos = x["pos"].cpu().numpy()
    W = cfg.window
    sel1 = int(ii[1, 5])
    nv4 = (int(pos[4]) + 1) // cfg.ratio
    hidden4 = nv4 + 3   # beyond row 4's visible prefix: never an entry even if it were selected
    slot2 = int(pos[2]) % W
    if cfg.main_dtype == "fp4":
        x["main_scale"][1, sel1, 7] = 255                 # E8M0 NaN: the whole 32-element block
        x["main_scale"][4, hidden4, 0] = 255
        x["swa"][2, slot2, 200] = 0x7F                    # E4M3 NaN code
    else:
        x["main"][1, sel1, 256 + 9] = 0x7F                # E4M3 scale of one 16-element block
        x["main"][4, hidden4, 256 + 0] = 0xFF
        x["swa"][2, slot2, 512 + 3] = 255                 # E8M0 scale of one 32-element block
        x["swa"][2, slot2, 40] = 0xFF                     # and an E4M3 NaN code in another block
    return sel1


@pytest.mark.parametrize("cfg", [LOWP, PAGES], ids=["fp4_main_fp8_swa", "pages_formats"])
def test_attention_with_nan_codes(cfg):
    x = make_inputs(cfg, 63, device="cuda")
    _fix_positions(x)
    idx = gpu_topk(cfg, x, gpu_scores(cfg, x))
    torch.cuda.synchronize()
    _plant_attention_nans(cfg, x, idx)
    out = gpu_attention(cfg, x, idx)
    torch.cuda.synchronize()
    rows = np.arange(cfg.q_tokens)
    ref = oracle_attention(cfg, x, idx.cpu().numpy(), rows)
    g = out.float().cpu().numpy()
    assert np.all(np.isnan(ref[1])) and np.all(np.isnan(ref[2]))
    assert np.all(np.isfinite(ref[[0, 3, 4, 5]]))
    assert np.array_equal(np.isnan(g), np.isnan(ref)), "NaN outputs differ in position"
    e = assert_close(out, ref, BF16_ATOL, BF16_RTOL, f"nan attention {cfg.main_dtype}")
    print(f"[nan attention {cfg.main_dtype}] rows 1, 2 NaN on both sides; others max_abs {e:.3e}")

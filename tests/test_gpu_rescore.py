"""GPU parity of the score-free FULL top-k (indexer_score with scores=None, then topk_rescore).

The score-free path must return exactly what topk_select returns over the
scores indexer_score writes, so every check here is bit-exact against that
materialised path on the same inputs, which in turn is checked against the
oracle (tests/test_gpu_parity.py, tests/test_gpu_fullsize.py):
  * (the select counts the block keys' bins itself; its threshold is checked
    through the top-k below);
  * each block key equals the largest order key of its 8 written scores (16-bit
    keys: its top 16 bits, all the select reads);
  * the top-k equals topk_select of the written scores, and the oracle's top-k
    of them.
Inputs include ragged histories (rows with fewer visible rows than k, a row
at position 0), duplicated key rows (exact score ties across blocks), and
the full 1M-row width, for FP8 and for MXFP4 index planes.
"""
import numpy as np
import pytest
import torch

from workloads import CONFIGS, make_inputs

from harness import gpu_scores, gpu_topk, index_scale, oracle_score_bound, oracle_topk
from workloads.step import index_plane_args

pytestmark = pytest.mark.gpu


def _order_keys(s):
    u = s.astype(np.float32).view(np.uint32).copy()
    u[(u & 0x7FFFFFFF) > 0x7F800000] = 0xFF800000
    u[u == 0x80000000] = 0
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def _score_free(cfg, x, k, bk16=False):
    import sparse_latent_attention_amd as csa2
    rows = x["pos"].shape[0]
    dev = x["pos"].device
    bkeys = torch.full((rows, -(-cfg.width // 8)), 12345, dtype=torch.int16 if bk16 else torch.int32, device=dev)
    kI, ikw = index_plane_args(cfg, x)
    csa2.indexer_score(x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, index_scale(cfg), None,
                       width=cfg.width, block_keys=bkeys, **ikw)
    out = torch.full((rows, k), -7, dtype=torch.int32, device=dev)
    ikw.pop("fp8", None)
    csa2.topk_rescore(x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, index_scale(cfg), out, bkeys,
                      cfg.width, **ikw)
    torch.cuda.synchronize()
    return bkeys, out


_MX = CONFIGS["pages_fp4_decode_1m"]
CASES = {
    "ragged_100k": (CONFIGS["lowp_full_decode_1m"].replace(batch=6, q_tokens=6, context=100003, ragged=True), 512),
    "short_rows": (CONFIGS["lowp_full_decode_1m"].replace(batch=5, q_tokens=5, context=30000, ragged=True), 512),
    "k2048": (CONFIGS["lowp_full_decode_1m"].replace(batch=3, q_tokens=3, context=50000), 2048),
    "ratio2": (CONFIGS["lowp_full_decode_1m"].replace(batch=4, q_tokens=4, context=80001, ratio=2, ragged=True), 512),
    "ties": (CONFIGS["lowp_full_decode_1m"].replace(batch=4, q_tokens=4, context=40000), 512),
    "full_1m": (CONFIGS["lowp_full_decode_1m"].replace(batch=3, q_tokens=3), 512),
    # every key row equal: every block queued (more blocks in a segment than the re-score's queue holds)
    "all_equal": (CONFIGS["lowp_full_decode_1m"].replace(batch=4, q_tokens=4, context=40000), 512),
    # 128 rows of 600000 columns: segments of 19456 columns, more block keys than one wave loads at once
    "wide_segments": (CONFIGS["lowp_full_decode_1m"].replace(batch=128, q_tokens=128, context=600000), 512),
    "k1_short_rows": (CONFIGS["lowp_full_decode_1m"].replace(batch=5, q_tokens=5, context=60000, ragged=True), 1),
    # MXFP4 index plane and query
    "mx_ragged_100k": (_MX.replace(batch=6, q_tokens=6, context=100003, ragged=True), 512),
    "mx_short_rows": (_MX.replace(batch=5, q_tokens=5, context=30000, ragged=True), 512),
    "mx_k2048_ratio2": (_MX.replace(batch=4, q_tokens=4, context=80001, ratio=2), 2048),
    "mx_ties": (_MX.replace(batch=4, q_tokens=4, context=40000), 512),
    "mx_full_1m": (_MX.replace(batch=3, q_tokens=3), 512),
    "mx_k1": (_MX.replace(batch=4, q_tokens=4, context=200001, ragged=True), 1),
}


BK16_CASES = ["ragged_100k", "short_rows", "k2048", "ties", "full_1m", "k1_short_rows", "all_equal", "wide_segments",
              "mx_short_rows", "mx_ties", "mx_full_1m"]


@pytest.mark.parametrize("name,bk16", [(n, False) for n in CASES] + [(n, True) for n in BK16_CASES])
def test_score_free_matches_written_scores(name, bk16):
    import sparse_latent_attention_amd as csa2
    cfg, k = CASES[name]
    print(f"\n[rescore] {name} rows={cfg.q_tokens} width={cfg.width} k={k} bk16={bk16}", flush=True)
    x = make_inputs(cfg, 51, device="cuda")
    rows = cfg.q_tokens
    if name.endswith("short_rows"):
        x["pos"][0] = 0
        x["pos"][1] = 300              # fewer visible rows than k
        x["pos"][2] = 8 * 64 + 2
    if name.endswith("ties"):
        # every 40th key row (and its scales) is a copy of row 17: equal scores across blocks
        kI = x["kI"].view(rows, -1, x["kI"].shape[-1])
        kI[:, ::40] = kI[:, 17:18]
        sc = x["kI_scale"].view(rows, -1, *x["kI_scale"].shape[2:])
        sc[:, ::40] = sc[:, 17:18]
    if name == "all_equal":
        kI = x["kI"].view(rows, -1, x["kI"].shape[-1])
        kI[:] = kI[:, 17:18]
        sc = x["kI_scale"].view(rows, -1, *x["kI_scale"].shape[2:])
        sc[:] = sc[:, 17:18]
    assert csa2.topk_rescore_supported(rows, cfg.width, k, fp8=cfg.idx_dtype == "fp8", fp4=cfg.idx_dtype == "fp4")
    bkeys, out = _score_free(cfg, x, k, bk16)

    scores = gpu_scores(cfg, x)
    ref_idx = gpu_topk(cfg, x, scores, k=k)
    s_np = scores.cpu().numpy()
    if rows <= 16:
        valid = np.isfinite(oracle_score_bound(cfg, x, np.arange(rows)))
    else:  # the columns each row sees (finite inputs: the same mask, without the float64 bound of every score)
        nv = (x["pos"].cpu().numpy().astype(np.int64) + 1) // cfg.ratio
        valid = np.arange(cfg.width)[None, :] < nv[:, None]
    keys = np.where(valid, _order_keys(s_np), 0).astype(np.uint32)
    pad = (-cfg.width) % 8
    want_bk = np.pad(keys, ((0, 0), (0, pad))).reshape(rows, -1, 8).max(axis=2)
    if bk16:
        assert np.array_equal(bkeys.cpu().numpy().view(np.uint16), (want_bk >> 16).astype(np.uint16))
    else:
        assert np.array_equal(bkeys.cpu().numpy().view(np.uint32), want_bk)
    got = out.cpu().numpy()
    assert np.array_equal(got, ref_idx.cpu().numpy()), "score-free top-k differs from topk_select of written scores"
    assert np.array_equal(got, oracle_topk(cfg, x, s_np.astype(np.float64), np.arange(rows), k=k))


def test_score_free_with_pool_block_scores():
    """The pool's block scores from a score-free pass equal those of the writing pass."""
    import sparse_latent_attention_amd as csa2
    cfg = CONFIGS["lowp_pool_decode_1m"].replace(batch=4, q_tokens=4, context=70001, ragged=True)
    x = make_inputs(cfg, 53, device="cuda")
    rows, nb = cfg.q_tokens, -(-cfg.width // 8)
    bm_a = torch.empty(rows, nb, dtype=torch.float32, device="cuda")
    bm_b = torch.empty(rows, nb, dtype=torch.float32, device="cuda")
    gpu_scores(cfg, x, block_max=bm_a)
    bkeys = torch.empty(rows, nb, dtype=torch.int32, device="cuda")
    kI = x["kI"].reshape(-1, cfg.idx_dim)
    csa2.indexer_score(x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, index_scale(cfg), None,
                       width=cfg.width, k_scale=x["kI_scale"].reshape(-1), fp8=True, block_keys=bkeys,
                       block_max=bm_b)
    torch.cuda.synchronize()
    assert torch.equal(bm_a, bm_b)


_PF = CONFIGS["prefill_4096_at_128k"]
DENSE_CASES = {
    # rows of one prefill chunk over a shared BF16 plane
    "bf16_chunk": (_PF.replace(q_tokens=300, context=30000, reuse_layers=0), 512),
    "bf16_ratio1": (_PF.replace(q_tokens=100, context=20000, ratio=1, reuse_layers=0), 512),
    "bf16_short_rows": (_PF.replace(q_tokens=200, context=700, reuse_layers=0), 512),   # 250..350 visible rows < k
    "bf16_k2048": (_PF.replace(q_tokens=64, context=40000, reuse_layers=0), 2048),
    "bf16_k1": (_PF.replace(q_tokens=33, context=9000, reuse_layers=0), 1),
    "bf16_few_rows": (_PF.replace(q_tokens=5, context=12000, reuse_layers=0), 512),      # fewer rows than a group
    "bf16_ties": (_PF.replace(q_tokens=70, context=26000, reuse_layers=0), 512),
}


@pytest.mark.parametrize("name", list(DENSE_CASES))
def test_score_free_bf16_chunk_matches_written_scores(name):
    """Prefill rows over one BF16 plane: the chunk kernel's block keys, then the best k blocks re-scored,
    give exactly topk_select over the written scores (and the oracle's top-k of them)."""
    import sparse_latent_attention_amd as csa2
    cfg, k = DENSE_CASES[name]
    print(f"\n[rescore bf16] {name} rows={cfg.q_tokens} width={cfg.width} k={k}", flush=True)
    x = make_inputs(cfg, 57, device="cuda")
    rows = cfg.q_tokens
    if name.endswith("ties"):
        kI = x["kI"]
        kI[::40] = kI[17:18]          # every 40th key row equals row 17: equal scores across blocks
        kI[5::40] = kI[17:18]
    if name == "all_equal":
        kI = x["kI"].view(rows, -1, x["kI"].shape[-1])
        kI[:] = kI[:, 17:18]
        sc = x["kI_scale"].view(rows, -1, *x["kI_scale"].shape[2:])
        sc[:] = sc[:, 17:18]
    assert csa2.topk_rescore_supported(rows, cfg.width, k, fp8=False, fp4=False, shared_plane=True)
    dev = x["pos"].device
    bkeys = torch.full((rows, -(-cfg.width // 8)), 12345, dtype=torch.int32, device=dev)
    kI, ikw = index_plane_args(cfg, x)
    csa2.indexer_score(x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, index_scale(cfg), None,
                       width=cfg.width, block_keys=bkeys, shared_plane=True)
    out = torch.full((rows, k), -7, dtype=torch.int32, device=dev)
    csa2.topk_rescore(x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, index_scale(cfg), out, bkeys,
                      cfg.width, dense=True, shared_plane=True)
    scores = gpu_scores(cfg, x)
    ref_idx = gpu_topk(cfg, x, scores, k=k)
    torch.cuda.synchronize()
    s_np = scores.cpu().numpy()
    if rows <= 16:
        valid = np.isfinite(oracle_score_bound(cfg, x, np.arange(rows)))
    else:  # the columns each row sees (finite inputs: the same mask, without the float64 bound of every score)
        nv = (x["pos"].cpu().numpy().astype(np.int64) + 1) // cfg.ratio
        valid = np.arange(cfg.width)[None, :] < nv[:, None]
    keys = np.where(valid, _order_keys(s_np), 0).astype(np.uint32)
    pad = (-cfg.width) % 8
    want_bk = np.pad(keys, ((0, 0), (0, pad))).reshape(rows, -1, 8).max(axis=2)
    assert np.array_equal(bkeys.cpu().numpy().view(np.uint32), want_bk), "block keys"
    got = out.cpu().numpy()
    assert np.array_equal(got, ref_idx.cpu().numpy()), "score-free top-k differs from topk_select of written scores"
    assert np.array_equal(got, oracle_topk(cfg, x, s_np.astype(np.float64), np.arange(rows), k=k))

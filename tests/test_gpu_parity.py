"""GPU parity of the HIP path against the oracle at sizes the oracle finishes in seconds.

Each config is a reduced copy of one of the five workloads (same dtypes and
head shapes) with ragged positions, widths that are not multiples of the tile
sizes, rows whose history is shorter than top-k, and rows at position 0.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs

from harness import (BF16_ATOL, BF16_RTOL, F32_ATOL, F32_RTOL, SCORE_TOL, assert_close, gpu_attention, gpu_scores,
                     gpu_topk, host_key_hist, oracle_attention, oracle_score_bound, oracle_scores, oracle_topk,
                     topk_band_mismatches)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_full_fp32": CONFIGS["tiny_full_fp32"],
    "tiny_dense_k128": CONFIGS["tiny_full_fp32"].replace(topk=128),
    "full_decode_small": CONFIGS["full_decode_64k"].replace(batch=7, q_tokens=7, context=3001, ragged=True),
    "full_decode_small_unit": CONFIGS["full_decode_64k"].replace(batch=4, q_tokens=4, context=2500, ragged=True,
                                                                 value_scale="unit"),
    "reindex_small": CONFIGS["reindex_decode_1m"].replace(batch=7, q_tokens=7, context=40001, n_blocks=200,
                                                          ragged=True),
    "reindex_fp8_small": CONFIGS["reindex_fp8_decode_1m"].replace(batch=7, q_tokens=7, context=40001, n_blocks=203,
                                                                  ragged=True),
    "reindex_pages_small": CONFIGS["reindex_pages_decode_1m"].replace(batch=7, q_tokens=7, context=40001,
                                                                      n_blocks=197, ragged=True),
    # blocks of 5 rows: the generic REINDEX kernel (the 8-row one serves block_rows == 8)
    "reindex_b5_small": CONFIGS["reindex_decode_1m"].replace(batch=5, q_tokens=5, context=20011, n_blocks=150,
                                                             block_rows=5, ragged=True),
    "lowp_small": CONFIGS["lowp_full_decode_1m"].replace(batch=7, q_tokens=7, context=5003, ragged=True),
    "pages_fp4_small": CONFIGS["pages_fp4_decode_1m"].replace(batch=7, q_tokens=7, context=5003, ragged=True),
    "prefill_small": CONFIGS["prefill_4096_at_128k"].replace(q_tokens=300, context=2000, reuse_layers=2),
}


def _tol(cfg):
    return (F32_ATOL, F32_RTOL) if cfg.out_dtype == "f32" else (BF16_ATOL, BF16_RTOL)


@pytest.fixture(scope="module", params=list(SMALL))
def case(request):
    cfg = SMALL[request.param]
    print(f"\n[case] {request.param} seed=11 rows={cfg.q_tokens} width={cfg.width}", flush=True)
    x = make_inputs(cfg, 11, device="cuda")
    scores = gpu_scores(cfg, x)
    idx = gpu_topk(cfg, x, scores)
    torch.cuda.synchronize()
    return request.param, cfg, x, scores, idx


def test_indexer_scores(case):
    name, cfg, x, scores, _ = case
    rows = np.arange(cfg.q_tokens)
    ref = oracle_scores(cfg, x, rows)
    bound = oracle_score_bound(cfg, x, rows)
    got = scores.cpu().numpy().astype(np.float64)
    inval = ~np.isfinite(bound)
    assert np.all(got[inval] == -np.inf) and np.all(ref[inval] == -np.inf)
    err = np.abs(got[~inval] - ref[~inval])
    ratio = float((err / bound[~inval]).max()) if err.size else 0.0
    print(f"[{name}] score max |d|/A = {ratio:.3e}")
    assert ratio <= SCORE_TOL


def test_topk_bit_exact_on_gpu_scores(case):
    name, cfg, x, scores, idx = case
    rows = np.arange(cfg.q_tokens)
    ref = oracle_topk(cfg, x, scores.cpu().numpy().astype(np.float64), rows)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_topk_end_to_end_band(case):
    name, cfg, x, scores, idx = case
    rows = np.arange(cfg.q_tokens)
    s_ref = oracle_scores(cfg, x, rows)
    ref = oracle_topk(cfg, x, s_ref, rows)
    bound = oracle_score_bound(cfg, x, rows)
    n_diff, n_bad = topk_band_mismatches(cfg, x, rows, idx.cpu().numpy(), ref, s_ref, bound)
    print(f"[{name}] end-to-end index differences: {n_diff} (outside the band: {n_bad})")
    assert n_bad == 0


def test_attention_all_layers(case):
    name, cfg, x, scores, idx = case
    rows = np.arange(cfg.q_tokens)
    atol, rtol = _tol(cfg)
    idx_np = idx.cpu().numpy()
    for layer in range(len(x["layers"])):
        out = gpu_attention(cfg, x, idx, layer=layer)
        ref = oracle_attention(cfg, x, idx_np, rows, layer=layer)
        e = assert_close(out, ref, atol, rtol, f"{name} layer {layer}")
        print(f"[{name}] layer {layer} attention max_abs {e:.3e}")


@pytest.mark.parametrize("rows", [1, 9, 300])
def test_decode_row_counts(rows):
    # 1 and 9 rows: the library's split choice; 300 rows: one workgroup per row, no merge pass
    cfg = SMALL["full_decode_small"].replace(batch=rows, q_tokens=rows)
    x = make_inputs(cfg, 5, device="cuda")
    idx = gpu_topk(cfg, x, gpu_scores(cfg, x))
    out = gpu_attention(cfg, x, idx)
    sample = np.unique(np.linspace(0, rows - 1, min(rows, 12)).astype(int))
    ref = oracle_attention(cfg, x, idx.cpu().numpy()[sample], sample)
    assert_close(out[torch.from_numpy(sample).cuda()], ref, BF16_ATOL, BF16_RTOL, f"decode rows={rows}")


@pytest.mark.parametrize("window,topk", [(16, 16), (48, 32), (16, 96), (128, 48), (1024, 2048)])
@pytest.mark.parametrize("base,rows", [("full_decode_small", 5), ("full_decode_small", 300), ("lowp_small", 7),
                                       ("prefill_small", None)])
def test_attention_ragged_tile_counts(base, rows, window, topk):
    """(window + topk) / 16 = 2, 5, 7, 11 tiles: the two-tile rounds then end with a half round (and decode
    splits with a short or empty last split); and the largest window and top-k the library
    takes (1024 + 2048: 192 tiles, the per-row index and validity buffers full)."""
    cfg = SMALL[base].replace(window=window, topk=topk)
    if rows is not None:
        cfg = cfg.replace(batch=rows, q_tokens=rows)
    else:
        cfg = cfg.replace(reuse_layers=0)
    print(f"\n[ragged tiles] {base} rows={cfg.q_tokens} window={window} topk={topk}", flush=True)
    x = make_inputs(cfg, 9, device="cuda")
    idx = gpu_topk(cfg, x, gpu_scores(cfg, x))
    out = gpu_attention(cfg, x, idx)
    sample = np.unique(np.linspace(0, cfg.q_tokens - 1, min(cfg.q_tokens, 10)).astype(int))
    ref = oracle_attention(cfg, x, idx.cpu().numpy()[sample], sample)
    assert_close(out[torch.from_numpy(sample).cuda()], ref, BF16_ATOL, BF16_RTOL, f"{base} W={window} k={topk}")


@pytest.mark.parametrize("rows,window,topk", [(517, 128, 512), (1000, 64, 128), (777, 16, 144)])
def test_prefill_row_stream(rows, window, topk):
    """Prefill rows streamed through one workgroup per CU (several consecutive rows each, the next
    row's tables built and its first tiles gathered during the row before): row counts that leave the
    last workgroup short, and rows of 20, 6 and 5 rounds.  Rows are sampled at every workgroup's
    first and last row over the first workgroups, and at the end."""
    cfg = SMALL["prefill_small"].replace(q_tokens=rows, context=2400, reuse_layers=0, window=window, topk=topk)
    print(f"\n[row stream] rows={rows} W={window} k={topk}", flush=True)
    x = make_inputs(cfg, 12, device="cuda")
    idx = gpu_topk(cfg, x, gpu_scores(cfg, x))
    out = gpu_attention(cfg, x, idx)
    per = -(-rows // 256)
    pick = sorted({r for b in range(0, 6) for r in (b * per, b * per + per - 1)} | {rows - 2, rows - 1})
    pick = np.array([r for r in pick if 0 <= r < rows])
    ref = oracle_attention(cfg, x, idx.cpu().numpy()[pick], pick)
    assert_close(out[torch.from_numpy(pick).cuda()], ref, BF16_ATOL, BF16_RTOL, f"row stream {rows}")


@pytest.mark.parametrize("window", [16, 48])
@pytest.mark.parametrize("base,rows", [("full_decode_small", 5), ("full_decode_small", 300), ("lowp_small", 7),
                                       ("prefill_small", None)])
def test_attention_window_only(base, rows, window):
    """No selected rows (top-k 0): 1 or 3 tiles, all from the window.  One tile leaves the rows kernel's
    first tile pair with only its zero-filled partner."""
    cfg = SMALL[base].replace(window=window, topk=0)
    if rows is not None:
        cfg = cfg.replace(batch=rows, q_tokens=rows)
    else:
        cfg = cfg.replace(reuse_layers=0)
    print(f"\n[window only] {base} rows={cfg.q_tokens} window={window}", flush=True)
    x = make_inputs(cfg, 10, device="cuda")
    idx = torch.empty(cfg.q_tokens, 0, dtype=torch.int32, device="cuda")
    out = gpu_attention(cfg, x, idx)
    sample = np.unique(np.linspace(0, cfg.q_tokens - 1, min(cfg.q_tokens, 10)).astype(int))
    ref = oracle_attention(cfg, x, idx.cpu().numpy()[sample], sample)
    assert_close(out[torch.from_numpy(sample).cuda()], ref, BF16_ATOL, BF16_RTOL, f"{base} W={window} k=0")


@pytest.mark.parametrize("splits", [1, 2, 3, 8])
@pytest.mark.parametrize("base", ["lowp_small", "full_decode_small", "pages_fp4_small"])
def test_decode_split_entries(base, splits):
    """Decode with each row's entries split over 1, 2, 3 or 8 workgroups (partial softmax states merged
    by a second kernel) against the oracle; uneven and empty splits included: 3 splits of 14, 14 and 12
    tiles, and 8 splits of 6 tiles cover the 40 tiles of a 128 + 512 row with the last split empty."""
    import sparse_latent_attention_amd as csa2
    from workloads.step import attn_storage_args
    cfg = SMALL[base]
    x = make_inputs(cfg, 12, device="cuda")
    idx = gpu_topk(cfg, x, gpu_scores(cfg, x))
    L = x["layers"][0]
    out = torch.empty_like(L["q"])
    kv, kw = attn_storage_args(cfg, x)
    csa2.sparse_attn_decode(L["q"], x["pos"], idx, kv, x["kv_row_base"], x["swa"], L["sink"],
                            csa2.rope_inv_freq(cfg.rope_dim, cfg.rope_theta, cfg.yarn_factor, cfg.yarn_orig).cuda(),
                            cfg.ratio, cfg.window, 1.0 / math.sqrt(cfg.dim), out, swa_scale=x["swa_scale"],
                            splits=splits, **kw)
    torch.cuda.synchronize()
    ref = oracle_attention(cfg, x, idx.cpu().numpy(), np.arange(cfg.q_tokens))
    e = assert_close(out, ref, BF16_ATOL, BF16_RTOL, f"{base} splits={splits}")
    print(f"[splits] {base} {splits}: max_abs {e:.3e}")


@pytest.mark.parametrize("base", ["lowp_small", "prefill_small"])
def test_injected_indices_and_masks(base):
    """-1 padding, duplicates, rows the group-causal mask hides, far out-of-range rows; for decode and
    for prefill (where the prefill kernel turns them into zero-row addresses and -inf score biases)."""
    cfg = SMALL[base]
    if cfg.phase == "prefill":
        cfg = cfg.replace(reuse_layers=0)
    x = make_inputs(cfg, 3, device="cuda")
    B, k = cfg.q_tokens, cfg.topk
    g = torch.Generator().manual_seed(0)
    idx = torch.randint(0, cfg.n_main_rows, (B, k), generator=g, dtype=torch.int32)
    idx[:, 0:16] = -1
    idx[:, 16:32] = idx[:, 32:48]                     # duplicates count twice
    idx[:, 48] = cfg.n_main_rows + 5                  # beyond the plane: masked (never read)
    idx[:, 49] = 2 ** 31 - 1
    idx[:, 50] = -7
    idx[1, :] = -1                                    # a row with no selected entry at all
    idx = idx.cuda()
    out = gpu_attention(cfg, x, idx)
    rows = np.unique(np.linspace(0, B - 1, min(B, 24)).astype(int))
    ref = oracle_attention(cfg, x, idx.cpu().numpy()[rows], rows)
    assert_close(out[torch.from_numpy(rows).cuda()], ref, BF16_ATOL, BF16_RTOL, f"injected indices {base}")


@pytest.mark.parametrize("base", ["full_decode_small_unit", "prefill_small"])
def test_sink_minus_inf(base):
    cfg = SMALL[base]
    if cfg.phase == "prefill":
        cfg = cfg.replace(reuse_layers=0)
    x = make_inputs(cfg, 4, device="cuda")
    x["layers"][0]["sink"] = torch.full_like(x["layers"][0]["sink"], -math.inf)
    idx = gpu_topk(cfg, x, gpu_scores(cfg, x))
    out = gpu_attention(cfg, x, idx)
    rows = np.unique(np.linspace(0, cfg.q_tokens - 1, min(cfg.q_tokens, 24)).astype(int))
    ref = oracle_attention(cfg, x, idx.cpu().numpy()[rows], rows)
    assert_close(out[torch.from_numpy(rows).cuda()], ref, BF16_ATOL, BF16_RTOL, f"sink=-inf {base}")


def test_topk_crafted_scores():
    # ties, NaN, -0, -inf and short rows, on the GPU kernel directly
    import sparse_latent_attention_amd as csa2
    rng = np.random.default_rng(1)
    rows, width, k = 9, 3000, 512
    s = rng.integers(-3, 4, (rows, width)).astype(np.float32) * 0.5
    s[0] = 1.0                                      # all equal: lowest columns win
    s[1, rng.random(width) < 0.3] = np.nan
    s[2, rng.random(width) < 0.5] = -0.0
    s[3] = -np.inf
    s[4, :] = np.arange(width, dtype=np.float32)    # distinct
    s[5] = rng.standard_normal(width).astype(np.float32)
    pos = np.array([2999, 2999, 2999, 2999, 2999, 2999, 100, 0, 511], dtype=np.int64)
    sc = torch.from_numpy(s).cuda()
    pt = torch.from_numpy(pos).cuda()
    out = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    csa2.topk_select(sc, pt, 1, out)
    ref = oracle.topk.topk_full(s.astype(np.float64), pos, 1, k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("rows,width,kind,k", [
    (3, 8000, "ties", 512),       # one workgroup per row; > 4096 keys at the threshold bin: read from memory
    (1100, 9000, "normal", 512),  # many rows: one workgroup per row, candidates in LDS
    (1030, 9000, "mixed", 512),   # many rows, some all-tied (fallback) and some short
    (1030, 9000, "mixed", 1),     # the smallest k
    (5, 3000, "ties", 1),
])
def test_topk_row_kernel(rows, width, kind, k):
    import sparse_latent_attention_amd as csa2
    print(f"\n[topk rows] rows={rows} width={width} kind={kind} k={k}", flush=True)
    rng = np.random.default_rng(rows + width)
    s = rng.standard_normal((rows, width)).astype(np.float32)
    pos = np.full(rows, width - 1, dtype=np.int64)
    if kind == "ties":
        s[:] = 2.5
        s[1, ::7] = 3.0
    if kind == "mixed":
        s[::5] = 1.0
        pos[1::7] = rng.integers(0, 600, len(pos[1::7]))
    sc = torch.from_numpy(s).cuda()
    pt = torch.from_numpy(pos).cuda()
    out = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    csa2.topk_select(sc, pt, 1, out)
    ref = oracle.topk.topk_full(s.astype(np.float64), pos, 1, k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("rows,width,kind,k,br", [
    (7, 16384, "normal", 512, 0),      # 16 columns per thread, keys held in registers
    (7, 32768, "normal", 512, 0),      # 32 per thread
    (5, 65536, "normal", 512, 0),      # 64 per thread, bins held, candidates' scores read again
    (6, 16384, "reindex", 512, 8),     # 8-row candidate blocks: -1 slots, blocks not yet visible
    (4, 32768, "reindex", 1, 8),
    (3, 65536, "reindex", 2048, 8),    # k > 1024: the floor from every key
    (4, 16000, "reindex", 512, 4),     # other block heights: one id per column
    (3, 48000, "reindex", 1024, 16),   # the largest k the threads' maxima bound
    (3, 65536, "skewed", 512, 0),      # the maxima's floor leaves too many keys: the floor from every key
    (4, 65536, "ties", 512, 0),        # heavy ties: the row from memory
    (5, 32768, "short", 1025, 0),      # fewer valid columns than threads or than k
    (9, 20000, "crafted", 512, 0),     # NaN, -0, -inf
    (3, 16386, "normal", 512, 0),      # width not a multiple of 4: the two-pass kernel
])
def test_topk_row_kernel_shapes(rows, width, kind, k, br):
    """Rows up to 65536 wide: one workgroup per row, bit-exact against the oracle's top-k."""
    import sparse_latent_attention_amd as csa2
    print(f"\n[topk row shapes] rows={rows} width={width} kind={kind} k={k} block_rows={br}", flush=True)
    rng = np.random.default_rng(rows * 7 + width + k)
    s = rng.standard_normal((rows, width)).astype(np.float32)
    pos = np.full(rows, width - 1, dtype=np.int64)
    cand = None
    if kind == "skewed":
        # most keys in one bin; the largest 2000 all in the first 4096 columns (64 threads' columns)
        s[:] = 1.01
        s[:, rng.choice(4096, 2000, replace=False)] = 2.0 + rng.random((rows, 2000)).astype(np.float32) * 6
    if kind == "ties":
        s = rng.integers(0, 3, (rows, width)).astype(np.float32)
        s[0] = 4.0
    if kind == "short":
        pos[0] = 300
        pos[1] = 5000
        pos[2] = 0
    if kind == "crafted":
        s[0, rng.random(width) < 0.3] = np.nan
        s[1, rng.random(width) < 0.5] = -0.0
        s[2] = -np.inf
        s[3, ::3] = np.nan
        s[3, 1::3] = -np.inf
        pos[4] = 700
        s[5] = np.round(s[5] * 4) / 4
    if kind == "reindex":
        nb = width // br
        pos[:] = 10 * width
        cand = np.stack([np.sort(rng.choice(10 * width // br, nb, replace=False)) for _ in range(rows)]).astype(np.int32)
        cand[1, -100:] = -1
        cand[0, ::37] = -1
        pos[2 % rows] = int(cand[2 % rows, nb // 2]) * br + br // 2   # half the blocks not visible, one in part
    sc = torch.from_numpy(s).cuda()
    pt = torch.from_numpy(pos).cuda()
    out = torch.full((rows, k), -9, dtype=torch.int32, device="cuda")
    assert csa2.topk_workspace_size(rows, width, k) == 0
    ct = None if cand is None else torch.from_numpy(cand).cuda()
    csa2.topk_select(sc, pt, 1, out, cand=ct, block_rows=br if br else 8)
    if cand is None:
        ref = oracle.topk.topk_full(s.astype(np.float64), pos, 1, k)
    else:
        ref = oracle.topk.topk_reindex(s.astype(np.float64), pos, 1, cand, br, k)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_deterministic():
    cfg = SMALL["reindex_small"]
    x = make_inputs(cfg, 8, device="cuda")
    a = gpu_scores(cfg, x)
    ia = gpu_topk(cfg, x, a)
    oa = gpu_attention(cfg, x, ia)
    b = gpu_scores(cfg, x)
    ib = gpu_topk(cfg, x, b)
    ob = gpu_attention(cfg, x, ib)
    assert torch.equal(a, b) and torch.equal(ia, ib) and torch.equal(oa, ob)


@pytest.mark.parametrize("rows,width,k,kind", [
    (5, 100003, 512, "normal"),      # wide path, ragged last chunk
    (3, 1 << 20, 512, "normal"),     # the 1M-column decode shape
    (4, 40000, 512, "ties"),         # few distinct values: chunks overflow, full-row fallback
    (6, 16384, 512, "reindex"),      # REINDEX mapping through 2048 candidate blocks
    (2, 20000, 2048, "normal"),      # largest k
    (3, 30000, 512, "short"),        # fewer valid columns than k in one row
    (3, 200000, 512, "quantized"),   # ~100 copies of each value: ties at the threshold inside the candidates
    (4, 100003, 1, "quantized"),     # the smallest k on the wide path
])
def test_topk_wide_rows(rows, width, k, kind):
    import sparse_latent_attention_amd as csa2
    print(f"\n[topk wide] rows={rows} width={width} k={k} kind={kind}", flush=True)
    rng = np.random.default_rng(width + rows)
    s = rng.standard_normal((rows, width)).astype(np.float32)
    cand = None
    pos = np.full(rows, width - 1, dtype=np.int64)
    if kind == "ties":
        s = rng.integers(0, 3, (rows, width)).astype(np.float32)
        s[0, :] = 7.0
    if kind == "quantized":
        s = np.round(s * 16) / 16
    if kind == "short":
        pos[1] = 300
    if kind == "reindex":
        nb = width // 8
        pos[:] = 10 * width
        cand = np.stack([np.sort(rng.choice(10 * width // 8, nb, replace=False)) for _ in range(rows)]).astype(np.int32)
        cand[1, -100:] = -1
        pos[2] = int(cand[2, nb // 2]) * 8 + 3          # half the candidates are not visible yet
    sc = torch.from_numpy(s).cuda()
    pt = torch.from_numpy(pos).cuda()
    out = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    ct = None if cand is None else torch.from_numpy(cand).cuda()
    csa2.topk_select(sc, pt, 1, out, cand=ct, block_rows=8)
    if cand is None:
        ref = oracle.topk.topk_full(s.astype(np.float64), pos, 1, k)
    else:
        ref = oracle.topk.topk_reindex(s.astype(np.float64), pos, 1, cand, 8, k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["reindex_decode_1m", "reindex_fp8_decode_1m", "reindex_pages_decode_1m"])
def test_reindex_equals_full_then_gather(name):
    """REINDEX over 8-row blocks computes each column with the FULL pass's arithmetic, so its scores are
    bit-identical to the FULL scores of the same plane rows (and -inf where the slot is -1 or the row is
    past the visible prefix): ragged positions, rows that see fewer blocks than the pool, -1 slots
    inside the id list's tail, a partially visible newest block, and a last step of fewer than 8 slots."""
    cfg = CONFIGS[name].replace(batch=6, q_tokens=6, context=60001, n_blocks=317, ragged=True)
    x = make_inputs(cfg, 23, device="cuda")
    x["pos"][2] = 9                                   # 10 visible rows: 2 blocks, the newest partial
    x["cand"][2] = -1
    x["cand"][2, :2] = torch.tensor([0, 1], dtype=torch.int32)
    full_cfg = cfg.replace(index_mode="full", n_blocks=0)
    re_s = gpu_scores(cfg, x).cpu().numpy()
    full_s = gpu_scores(full_cfg, {k: v for k, v in x.items() if k != "cand"}).cpu().numpy()
    cand = x["cand"].cpu().numpy().astype(np.int64)
    pos = x["pos"].cpu().numpy()
    for r in range(cfg.q_tokens):
        nv = (int(pos[r]) + 1) // cfg.ratio
        rows, valid = oracle.indexer.reindex_rows(cand[r], 8, nv)
        want = np.where(valid, full_s[r][np.where(valid, rows, 0)], -np.inf).astype(np.float32)
        assert np.array_equal(re_s[r].view(np.uint32), want.view(np.uint32)), f"row {r}"


@pytest.mark.parametrize("kw", [
    dict(batch=7, q_tokens=7, context=3001, ragged=True),      # ragged rows, width not a multiple of 64
    dict(batch=4, q_tokens=4, context=40003, ragged=True),
    dict(batch=3, q_tokens=3, context=150001),                 # more steps than one wave takes
])
def test_full_bf16_stream_equals_row_kernel(kw):
    """FULL rows of BF16 keys with scores only go through the staged block stream; asked for block
    scores as well, the call takes the per-row kernel.  Both write bit-identical scores, and the
    stream's key histogram equals a host recount."""
    cfg = CONFIGS["full_decode_64k"].replace(**kw)
    print(f"\n[full bf16 stream] {kw}", flush=True)
    x = make_inputs(cfg, 23, device="cuda")
    rows = cfg.q_tokens
    x["pos"][0] = 0                                   # one visible row
    h = torch.full((rows, 4096), 777, dtype=torch.int32, device="cuda")
    a = gpu_scores(cfg, x, key_hist=h)
    bm = torch.empty(rows, -(-cfg.width // 8), dtype=torch.float32, device="cuda")
    b = gpu_scores(cfg, x, block_max=bm)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    s_np = a.cpu().numpy()
    valid = np.isfinite(oracle_score_bound(cfg, x, np.arange(rows)))
    assert np.array_equal(h.cpu().numpy().astype(np.int64), host_key_hist(s_np, valid))
    assert np.all(np.isneginf(s_np[~valid]))


@pytest.mark.parametrize("name,kw", [
    ("lowp_full_decode_1m", dict(batch=6, q_tokens=6, context=100003, ragged=True)),
    ("full_decode_64k", dict(batch=5, q_tokens=5, context=40000, ragged=True)),
    ("full_decode_64k", dict(batch=4, q_tokens=4, context=200001, ragged=True)),
    ("reindex_decode_1m", dict(batch=5, q_tokens=5, context=300000, ragged=True, n_blocks=9000)),
    ("reindex_fp8_decode_1m", dict(batch=5, q_tokens=5, context=300000, ragged=True, n_blocks=8192)),
    ("reindex_pages_decode_1m", dict(batch=5, q_tokens=5, context=300000, ragged=True, n_blocks=9000)),
])
def test_key_hist_path(name, kw):
    """Indexer-built key histogram == host recount of the GPU scores; top-k through it is exact (rows
    wider than 65536 columns read it; narrower rows are selected one workgroup per row without it)."""
    import sparse_latent_attention_amd as csa2
    cfg = CONFIGS[name].replace(**kw)
    print(f"\n[key_hist] {name} {kw}", flush=True)
    x = make_inputs(cfg, 21, device="cuda")
    rows = cfg.q_tokens
    assert csa2.topk_uses_key_hist(rows, cfg.width, cfg.topk) == (cfg.width > 65536)
    h = torch.empty(rows, 4096, dtype=torch.int32, device="cuda")
    h.fill_(12345)                                   # the call must zero it
    scores = gpu_scores(cfg, x, key_hist=h)
    s_np = scores.cpu().numpy()
    valid = np.isfinite(oracle_score_bound(cfg, x, np.arange(rows)))
    assert np.array_equal(h.cpu().numpy().astype(np.int64), host_key_hist(s_np, valid))
    idx = gpu_topk(cfg, x, scores, key_hist=h)
    ref = oracle_topk(cfg, x, s_np.astype(np.float64), np.arange(rows))
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("name,kw", [
    ("full_decode_64k", dict(batch=6, q_tokens=6, context=3000, ragged=True, value_scale="unit")),
    ("full_decode_64k", dict(batch=300, q_tokens=300, context=1500, ragged=True, value_scale="unit")),
    ("prefill_4096_at_128k", dict(q_tokens=200, context=900, reuse_layers=0)),
])
def test_attention_large_logit_spread(name, kw):
    """Scores spread over many powers of two: the running max moves several times per row."""
    cfg = CONFIGS[name].replace(**kw)
    print(f"\n[spread] {name} {kw}", flush=True)
    x = make_inputs(cfg, 31, device="cuda")
    L = x["layers"][0]
    L["q"] = (L["q"].float() * 8.0).to(L["q"].dtype)
    idx = gpu_topk(cfg, x, gpu_scores(cfg, x))
    out = gpu_attention(cfg, x, idx)
    rows = np.unique(np.linspace(0, cfg.q_tokens - 1, min(cfg.q_tokens, 16)).astype(int))
    ref = oracle_attention(cfg, x, idx.cpu().numpy()[rows], rows)
    assert_close(out[torch.from_numpy(rows).cuda()], ref, BF16_ATOL, BF16_RTOL, f"spread {name}")


@pytest.mark.parametrize("rows,width,base,ratio", [(37, 9000, 100, 2), (8, 64, 0, 2), (300, 20000, 5, 2),
                                                   (13, 8300, 0, 2), (40, 9000, 7, 1)])
def test_shared_plane_scores_equal_per_row_path(rows, width, base, ratio):
    """Rows that share one plane (the staged-key-tile path for BF16 64 x 128): bit-identical scores to the
    per-row path, over ragged row groups (rows not a multiple of 8), ragged column ranges and stages
    (width not a multiple of 8192 or 64), rows that see nothing (position 0 at ratio 2) and rows that see
    every column."""
    import sparse_latent_attention_amd as csa2
    g = torch.Generator(device="cuda")
    g.manual_seed(rows * 7 + width)
    k = (torch.randn(base + width, 128, generator=g, device="cuda") * 0.1).to(torch.bfloat16)
    q = (torch.randn(rows, 64, 128, generator=g, device="cuda") * 0.1).to(torch.bfloat16)
    w = torch.randn(rows, 64, generator=g, device="cuda")
    pos = torch.randint(0, ratio * width + 10, (rows,), generator=g, device="cuda")
    pos[0] = 0
    pos[-1] = ratio * width + 5
    rb = torch.full((rows,), base, dtype=torch.int64, device="cuda")
    out = {}
    for shared in (True, False):
        s = torch.full((rows, width), float("nan"), dtype=torch.float32, device="cuda")
        csa2.indexer_score(q, w, k, rb, pos, ratio, 0.01, s, shared_plane=shared)
        out[shared] = s
    torch.cuda.synchronize()
    assert not torch.isnan(out[True]).any()
    assert torch.equal(out[True], out[False])
    nv = ((pos + 1) // ratio).clamp(max=width).cpu().numpy()
    got = out[True].cpu().numpy()
    for r in range(rows):
        assert np.all(got[r, nv[r]:] == -np.inf) and np.all(np.isfinite(got[r, :nv[r]]))
    # spot check against the oracle on a few rows
    tau = 0.01
    for r in sorted({0, rows // 2, rows - 1}):
        n = int(nv[r])
        if n == 0:
            continue
        kk = k[base:base + n].double().cpu().numpy()
        ref = oracle.indexer.scores_full(q[r:r + 1].double().cpu().numpy(), w[r:r + 1].double().cpu().numpy(),
                                         lambda i: kk, np.array([ratio * n - 1]), ratio, tau, n)[0]
        bound = oracle.indexer.score_abs_bound(q[r].double().cpu().numpy(), w[r].double().cpu().numpy(), kk, tau)
        assert np.all(np.abs(got[r, :n] - ref) <= SCORE_TOL * bound)


def test_empty_inputs():
    """Zero query rows through every entry point (device tensors with no elements), and zero-width rows in
    top-k (no valid column: all -1)."""
    import sparse_latent_attention_amd as csa2
    dev = "cuda"
    e64 = torch.empty(0, dtype=torch.int64, device=dev)
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device=dev)
    # indexer: no rows, and rows over an empty width
    csa2.indexer_score(bf(0, 64, 128), torch.zeros(0, 64, device=dev), bf(16, 128), e64, e64, 2, 0.01,
                       torch.empty(0, 100, device=dev))
    csa2.indexer_score(bf(3, 64, 128), torch.zeros(3, 64, device=dev), bf(16, 128),
                       torch.zeros(3, dtype=torch.int64, device=dev), torch.full((3,), 5, dtype=torch.int64, device=dev),
                       2, 0.01, torch.empty(3, 0, device=dev))
    # top-k: no rows; rows of width 0 give only -1
    csa2.topk_select(torch.empty(0, 50, device=dev), e64, 1, torch.empty(0, 16, dtype=torch.int32, device=dev))
    out = torch.zeros(4, 16, dtype=torch.int32, device=dev)
    csa2.topk_select(torch.empty(4, 0, device=dev), torch.full((4,), 9, dtype=torch.int64, device=dev), 1, out)
    torch.cuda.synchronize()
    assert bool((out == -1).all())
    # attention, decode and prefill: no rows
    freqs = csa2.rope_inv_freq(64, 160000.0, 16.0, 65536).to(dev)
    sink = torch.zeros(64, device=dev)
    csa2.sparse_attn_decode(bf(0, 64, 512), e64, torch.empty(0, 16, dtype=torch.int32, device=dev), bf(8, 512), e64,
                            bf(0, 128, 512), sink, freqs, 1, 128, 0.04, bf(0, 64, 512))
    csa2.sparse_attn_prefill(bf(0, 64, 512), e64, torch.empty(0, 16, dtype=torch.int32, device=dev), bf(8, 512),
                             bf(8, 512), 0, sink, freqs, 1, 128, 0.04, bf(0, 64, 512))
    # candidate pool and write path: no rows
    csa2.candidate_pool(e64, 1, torch.empty(0, 16, dtype=torch.int32, device=dev),
                        scores=torch.empty(0, 100, device=dev))
    csa2.compress(bf(0, 256), e64, torch.empty(0, dtype=torch.int32, device=dev), e64, bf(512, 256),
                  torch.ones(512, device=dev), bf(128, 512), torch.ones(128, device=dev), freqs,
                  torch.zeros(8, 512, device=dev), torch.zeros(8, 128, device=dev), ratio=1, main_format="f32",
                  idx_format="f32")
    torch.cuda.synchronize()

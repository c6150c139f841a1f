"""Shared helpers for the parity tests: run the HIP path, run the oracle, compare.

The GPU side goes only through the C ABI binding (sparse_latent_attention_amd);
the oracle side reads the same stored input tensors back to the host and
decodes them with oracle.formats.  Nothing computed by the GPU is fed to the
oracle except where a test states it (top-k of the GPU's own scores, and
attention over the GPU's selected rows, each compared separately).
"""

import math

import numpy as np
import torch

import oracle
from oracle import formats
from workloads.step import attn_storage_args, index_plane_args

# Tolerances.
# Indexer scores: |gpu - oracle| <= SCORE_TOL * A, A = tau_I sum_h |w_h| sum_d |q_hd k_d|.
# fp32 accumulation of D_I products plus H_I weighted terms gives an error of
# at most about (D_I + H_I + 2) u A with u = 2^-24, i.e. 1.16e-5 A for 64 x 128;
# the factor 4 covers the matrix core's own accumulation order.
SCORE_TOL = 4.6e-5
# bf16 outputs: the tolerance fixed for the path, read as |g - o| <= 2e-2 + 1e-2 |o|.
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
# f32 outputs (tiny config): scores in fp32 from fp32 inputs, probabilities and
# the weighted sum in fp32; relative error a few 1e-6, bounded here by 1e-4.
F32_ATOL, F32_RTOL = 1e-4, 1e-4


def to_numpy_f64(t, fmt, scale=None):
    """Decode a stored tensor (any device) to float64 numpy with the oracle's decoders."""
    t = t.detach().cpu()
    if fmt == "f32":
        return t.numpy().astype(np.float64)
    if fmt == "bf16":
        return formats.bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if fmt == "fp8":
        if scale is None:
            return formats.decode_fp8_values(t.numpy())
        return formats.decode_fp8_rows(t.numpy(), scale.detach().cpu().numpy())
    if fmt == "fp4":
        return formats.decode_fp4_rows(t.numpy(), scale.detach().cpu().numpy())
    if fmt == "nvfp4":
        return formats.decode_nvfp4_rows(t.numpy())
    if fmt == "fp8mx":
        return formats.decode_fp8_e8m0_rows(t.numpy())
    raise ValueError(fmt)


class LazyPlane:
    """Decodes rows of one stored plane on demand (plane[rows] / plane[:n])."""

    def __init__(self, data, fmt, scale=None):
        self.data, self.fmt, self.scale = data, fmt, scale
        self.shape = (data.shape[0],)

    def __getitem__(self, key):
        if isinstance(key, slice):
            idx = torch.arange(*key.indices(self.data.shape[0]))
        else:
            idx = torch.as_tensor(np.asarray(key), dtype=torch.int64)
        dev = self.data.device
        d = self.data.index_select(0, idx.to(dev))
        s = None if self.scale is None else self.scale.index_select(0, idx.to(self.scale.device))
        return to_numpy_f64(d, self.fmt, s)


def inv_freq_device(cfg, device="cuda"):
    import sparse_latent_attention_amd as csa2
    return csa2.rope_inv_freq(cfg.rope_dim, cfg.rope_theta, cfg.yarn_factor, cfg.yarn_orig).to(device)


def oracle_freqs(cfg):
    return oracle.rope.inv_freq(cfg.rope_dim, cfg.rope_theta, cfg.yarn_factor, cfg.yarn_orig)


def index_scale(cfg):
    return 1.0 / (math.sqrt(cfg.idx_dim) * math.sqrt(cfg.idx_heads))


def gpu_scores(cfg, x, key_hist=None, block_max=None):
    import sparse_latent_attention_amd as csa2
    rows = x["pos"].shape[0]
    scores = torch.empty(rows, cfg.width, dtype=torch.float32, device=x["pos"].device)
    kI, ikw = index_plane_args(cfg, x)
    # a prefill chunk's rows share one plane (row_base is 0 for every row)
    csa2.indexer_score(x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, index_scale(cfg), scores,
                       cand=x.get("cand"), block_rows=cfg.block_rows, key_hist=key_hist, block_max=block_max,
                       shared_plane=cfg.phase == "prefill", **ikw)
    return scores


def gpu_topk(cfg, x, scores, k=None, key_hist=None):
    import sparse_latent_attention_amd as csa2
    k = cfg.topk if k is None else k
    out = torch.empty(scores.shape[0], k, dtype=torch.int32, device=scores.device)
    csa2.topk_select(scores, x["pos"], cfg.ratio, out, cand=x.get("cand"), block_rows=cfg.block_rows,
                     key_hist=key_hist)
    return out


def host_key_hist(scores_np, valid):
    """Histogram of the top 12 bits of the score order key (the definition in include/csa2.h)."""
    u = scores_np.astype(np.float32).view(np.uint32).copy()
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    u[nan] = 0xFF800000
    u[u == 0x80000000] = 0
    key = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
    out = np.zeros((scores_np.shape[0], 4096), dtype=np.int64)
    for r in range(scores_np.shape[0]):
        np.add.at(out[r], (key[r][valid[r]] >> 20).astype(np.int64), 1)
    return out


def gpu_attention(cfg, x, idx, layer=0, out=None):
    import sparse_latent_attention_amd as csa2
    L = x["layers"][layer]
    q = L["q"]
    out = torch.empty_like(q) if out is None else out
    kv, kw = attn_storage_args(cfg, x)
    freqs = inv_freq_device(cfg, q.device)
    scale = 1.0 / math.sqrt(cfg.dim)
    if cfg.phase == "decode":
        swa = x["swa"]
        sws = x["swa_scale"]
        csa2.sparse_attn_decode(q, x["pos"], idx, kv, x["kv_row_base"], swa, L["sink"], freqs, cfg.ratio,
                                cfg.window, scale, out, swa_scale=sws, **kw)
    else:
        csa2.sparse_attn_prefill(q, x["pos"], idx, kv, L["swa"], x["swa_pos0"], L["sink"], freqs, cfg.ratio,
                                 cfg.window, scale, out, swa_scale=L["swa_scale"],
                                 kv_row_base=x["kv_row_base"], **kw)
    return out


# ---------------------------------------------------------------------------
# Oracle side (float64 on the host)

def oracle_planes(cfg, x):
    """Per-row accessors for the decoded index plane and main plane (lazy)."""
    if cfg.phase == "decode":
        B = cfg.batch
        kI = [LazyPlane(x["kI"][b], cfg.idx_dtype, None if x["kI_scale"] is None else x["kI_scale"][b]) for b in range(B)]
        main = [LazyPlane(x["main"][b], cfg.main_dtype, None if x["main_scale"] is None else x["main_scale"][b])
                for b in range(B)]
        return (lambda r: kI[r]), (lambda r: main[r])
    kI = LazyPlane(x["kI"], cfg.idx_dtype, x["kI_scale"])
    main = LazyPlane(x["main"], cfg.main_dtype, x["main_scale"])
    return (lambda r: kI), (lambda r: main)


def oracle_index_inputs(cfg, x, rows):
    qs = None if x.get("qI_scale") is None else x["qI_scale"][rows]
    q = to_numpy_f64(x["qI"][rows], cfg.idx_dtype, qs)
    w = x["w"][rows].detach().cpu().numpy().astype(np.float64)
    return q, w


def oracle_scores(cfg, x, rows):
    """Oracle indexer scores for the given query rows, [len(rows), width]."""
    q, w = oracle_index_inputs(cfg, x, rows)
    kI_of, _ = oracle_planes(cfg, x)
    pos = x["pos"][rows].cpu().numpy()
    tau = oracle.indexer.indexer_scale(cfg.idx_heads, cfg.idx_dim)
    pl = lambda i: kI_of(int(rows[i]))
    if cfg.index_mode == "reindex":
        cand = x["cand"][rows].cpu().numpy()
        return oracle.indexer.scores_reindex(q, w, pl, pos, cfg.ratio, cand, cfg.block_rows, tau)
    return oracle.indexer.scores_full(q, w, pl, pos, cfg.ratio, tau, cfg.width)


def oracle_score_bound(cfg, x, rows):
    """A per (row, column) for the score tolerance, +inf where the column is invalid."""
    q, w = oracle_index_inputs(cfg, x, rows)
    kI_of, _ = oracle_planes(cfg, x)
    tau = oracle.indexer.indexer_scale(cfg.idx_heads, cfg.idx_dim)
    out = np.full((len(rows), cfg.width), np.inf)
    for i, r in enumerate(rows):
        nv = (int(x["pos"][r]) + 1) // cfg.ratio
        if cfg.index_mode == "reindex":
            prow, valid = oracle.indexer.reindex_rows(x["cand"][r].cpu().numpy(), cfg.block_rows, nv)
            cols = np.nonzero(valid)[0]
            if len(cols):
                out[i, cols] = oracle.indexer.score_abs_bound(q[i], w[i], kI_of(int(r))[prow[cols]], tau)
        elif nv > 0:
            out[i, :nv] = oracle.indexer.score_abs_bound(q[i], w[i], kI_of(int(r))[:nv], tau)
    return out


def oracle_topk(cfg, x, scores_np, rows, k=None):
    k = cfg.topk if k is None else k
    pos = x["pos"][rows].cpu().numpy()
    if cfg.index_mode == "reindex":
        return oracle.topk.topk_reindex(scores_np, pos, cfg.ratio, x["cand"][rows].cpu().numpy(), cfg.block_rows, k)
    return oracle.topk.topk_full(scores_np, pos, cfg.ratio, k)


def oracle_attention(cfg, x, idx_np, rows, layer=0):
    """Oracle attention output for the given rows, with the given selected indices [len(rows), k]."""
    L = x["layers"][layer]
    q = to_numpy_f64(L["q"][rows], cfg.q_dtype)
    sink = L["sink"].cpu().numpy().astype(np.float64)
    freqs = oracle_freqs(cfg)
    tau = 1.0 / math.sqrt(cfg.dim)
    _, main_of = oracle_planes(cfg, x)
    out = np.empty(q.shape)
    pos = x["pos"][rows].cpu().numpy()
    for i, r in enumerate(rows):
        if cfg.phase == "decode":
            ring = to_numpy_f64(x["swa"][r], cfg.swa_dtype, None if x["swa_scale"] is None else x["swa_scale"][r])
            ents = oracle.attention.entries_decode(pos[i], idx_np[i], main_of(int(r)), ring, cfg.ratio)
        else:
            swa = LazyPlane(L["swa"], cfg.swa_dtype, L["swa_scale"])
            wpos = oracle.geometry.linear_window_positions(pos[i], cfg.window)
            t = wpos - x["swa_pos0"]
            t = t[(t >= 0) & (t < L["swa"].shape[0])]
            nv = (int(pos[i]) + 1) // cfg.ratio
            sel = np.asarray(idx_np[i], dtype=np.int64)
            sel = sel[(sel >= 0) & (sel < nv)]
            ents = np.concatenate([swa[t], main_of(int(r))[sel]], axis=0)
        out[i] = oracle.attention.attend(q[i], pos[i], ents, sink, tau, freqs)
    return out


def close_mask(g, ref, atol, rtol):
    """Elements that agree: both NaN, the same infinity, or finite with |g - o| <= atol + rtol |o|.
    Anything else fails, including a NaN or an infinity on one side only."""
    g = np.asarray(g, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_nan = np.isnan(g) & np.isnan(ref)
    same_inf = np.isinf(g) & np.isinf(ref) & (g == ref)
    fin = np.isfinite(g) & np.isfinite(ref)
    with np.errstate(invalid="ignore"):
        ok_fin = np.abs(g - ref) <= atol + rtol * np.abs(ref)
    return both_nan | same_inf | (fin & ok_fin)


def assert_close(gpu, ref, atol, rtol, what):
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} != {ref.shape}"
    ok = close_mask(g, ref, atol, rtol)
    fin = np.isfinite(g) & np.isfinite(ref)
    err = np.where(fin, np.abs(g - ref), 0.0)
    max_abs = float(err.max()) if err.size else 0.0
    big = fin & (np.abs(ref) > 1e-3)
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    info = f"{what}: max_abs={max_abs:.3e} max_rel(|o|>1e-3)={max_rel:.3e}"
    n_bad = int((~ok).sum())
    n_nf = int((~fin & ~ok).sum())
    assert n_bad == 0, info + f" ; {n_bad} elements outside {atol}+{rtol}|o| ({n_nf} of them non-finite on one side)"
    return max_abs


def topk_band_mismatches(cfg, x, rows, gpu_idx, oracle_idx, s_oracle, bound):
    """End-to-end index differences; each must lie within the score error band of the k-th score."""
    n_bad, n_diff = 0, 0
    for i in range(len(rows)):
        a = set(int(v) for v in gpu_idx[i] if v >= 0)
        b = set(int(v) for v in oracle_idx[i] if v >= 0)
        diff = a ^ b
        if not diff:
            continue
        n_diff += len(diff)
        # map rows back to columns to read their oracle scores
        if cfg.index_mode == "reindex":
            cand = x["cand"][rows[i]].cpu().numpy()
            nv = (int(x["pos"][rows[i]]) + 1) // cfg.ratio
            prow, valid = oracle.indexer.reindex_rows(cand, cfg.block_rows, nv)
            col_of = {int(p): c for c, p in enumerate(prow) if valid[c]}
        else:
            col_of = None
        s = s_oracle[i]
        finite = np.sort(s[np.isfinite(s)])[::-1]
        kth = finite[min(cfg.topk, len(finite)) - 1]
        band = 2 * SCORE_TOL * float(np.max(bound[i][np.isfinite(bound[i])]))
        for v in diff:
            c = col_of[v] if col_of is not None else v
            if abs(s[c] - kth) > band:
                n_bad += 1
    return n_diff, n_bad

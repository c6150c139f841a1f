"""Seeded synthetic inputs for a Csa2Config, in the stored formats the hot path reads.

Recipe (all draws from one torch.Generator seeded with ``seed`` on ``device``):

* q, main latent rows, SWA rows, indexer query and index-key rows: N(0,1),
  or N(0,1)/sqrt(dim) when ``value_scale == "inv_sqrt_d"`` (dim = the latent
  dim 512; the same factor is used for the 128-dim index vectors).  Stored
  rows are drawn directly in their post-RoPE form: an isotropic Gaussian pair
  is invariant under rotation, so no rotation is needed to get the right
  distribution.
* attn_sink and the indexer head weights w: N(0,1).
* decode positions: context-1 for every sequence, or (ragged) uniform in
  [0, context-1] with the first sequences pinned to 0, 1, window-1, window and
  context-1.
* REINDEX candidates: per query, min(n_blocks, visible blocks) distinct block
  ids drawn uniformly among the visible blocks, always containing the newest
  (partly filled) block, sorted ascending, -1 padded.
* FP8-E4M3 rows: per-row float32 scale amax/448, values cast with torch's
  float8_e4m3fn conversion.  FP8 indexer query: one float32 scale per (row,
  head), folded into w (w_eff = w * scale), as the anatomy page's indexer
  figure describes.
* FP4-E2M1 rows: one E8M0 scale per 32 elements, 2^ceil(log2(amax/6)); the
  scaled values are rounded to the nearest E2M1 magnitude (ties to the even
  code) and packed two per byte, element 2i in the low nibble.  The FP4 index
  plane and FP4 indexer query use this format (no scale folded into w).
* Packed FP4 main rows (288 B per 512): E2M1 as above with one E4M3 scale per
  16 elements, the scale being amax/6 rounded to E4M3 (at least 2^-9); values
  beyond 6 after scaling saturate.
* FP8 rows with E8M0 block scales (528 B per 512): one scale per 32 elements,
  2^ceil(log2(amax/448)); values cast with float8_e4m3fn.

Nothing here scores, selects, normalises or rotates.
"""

import math

import torch

from .configs import Csa2Config

_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _normal(g, shape, device, std, dtype=torch.float32):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def store_dense(x, dtype):
    if dtype == "f32":
        return x.to(torch.float32).contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def encode_fp8_rows(x):
    """x float32 [..., D] -> (codes uint8 [..., D], row scale float32 [...])."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (x / scale.unsqueeze(-1)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.to(torch.float32).contiguous()


def _e2m1_codes(y):
    """float32 -> E2M1 codes (nearest magnitude, ties to the even code, saturating at 6)."""
    mag = y.abs().clamp(max=6.0)
    grid = torch.tensor(_E2M1_MAG, device=y.device, dtype=torch.float32)
    mids = (grid[1:] + grid[:-1]) * 0.5
    code = torch.bucketize(mag, mids, right=False)            # ties go to the lower magnitude
    tie = mag == mids[code.clamp(max=6)]
    code = torch.where(tie & (code % 2 == 1), code + 1, code)  # ... unless that code is odd
    return code.to(torch.uint8) | ((y < 0).to(torch.uint8) << 3)


def encode_nvfp4_rows(x):
    """x float32 [..., D] -> rows uint8 [..., D/2 + D/16]: packed E2M1, then one E4M3 scale per 16."""
    shp = x.shape
    d = shp[-1]
    assert d % 16 == 0
    xb = x.reshape(*shp[:-1], d // 16, 16)
    amax = xb.abs().amax(dim=-1)
    sc = (amax / 6.0).clamp(min=2.0 ** -9, max=448.0).to(torch.float8_e4m3fn)
    y = xb / sc.to(torch.float32).unsqueeze(-1)
    code = _e2m1_codes(y).reshape(*shp[:-1], d)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return torch.cat([packed, sc.view(torch.uint8)], dim=-1).contiguous()


def encode_fp8_e8m0_rows(x):
    """x float32 [..., D] -> rows uint8 [..., D + D/32]: E4M3 codes, then one E8M0 scale per 32."""
    shp = x.shape
    d = shp[-1]
    assert d % 32 == 0
    xb = x.reshape(*shp[:-1], d // 32, 32)
    amax = xb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax / 448.0)), torch.full_like(amax, -127.0)).clamp_(-127.0, 127.0)
    codes = (xb / torch.exp2(e).unsqueeze(-1)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return torch.cat([codes.reshape(*shp[:-1], d), (e + 127.0).to(torch.uint8)], dim=-1).contiguous()


def encode_fp4_rows(x):
    """x float32 [..., D] -> (packed uint8 [..., D/2], E8M0 scales uint8 [..., D/32])."""
    shp = x.shape
    d = shp[-1]
    assert d % 32 == 0
    xb = x.reshape(*shp[:-1], d // 32, 32)
    amax = xb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax / 6.0)), torch.full_like(amax, -127.0))
    e = e.clamp_(-127.0, 127.0)
    y = xb / torch.exp2(e).unsqueeze(-1)
    code = _e2m1_codes(y).reshape(*shp[:-1], d)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).contiguous()
    scale = (e + 127.0).to(torch.uint8).reshape(*shp[:-1], d // 32).contiguous()
    return packed, scale


def _store_rows(g, shape, device, std, dtype, chunk_leading=False):
    """Draw rows of ``shape`` and store as ``dtype``; returns dict of tensors."""
    if dtype in ("f32", "bf16"):
        if chunk_leading and len(shape) == 3:
            out = torch.empty(shape, device=device, dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
            for b in range(shape[0]):
                out[b] = store_dense(_normal(g, shape[1:], device, std), dtype)
            return {"data": out}
        return {"data": store_dense(_normal(g, shape, device, std), dtype)}
    if dtype == "fp8":
        if chunk_leading and len(shape) == 3:
            codes = torch.empty(shape, device=device, dtype=torch.uint8)
            scale = torch.empty(shape[:-1], device=device, dtype=torch.float32)
            for b in range(shape[0]):
                codes[b], scale[b] = encode_fp8_rows(_normal(g, shape[1:], device, std))
            return {"data": codes, "scale": scale}
        codes, scale = encode_fp8_rows(_normal(g, shape, device, std))
        return {"data": codes, "scale": scale}
    if dtype == "fp4":
        if chunk_leading and len(shape) == 3:
            packed = torch.empty(shape[:-1] + (shape[-1] // 2,), device=device, dtype=torch.uint8)
            scale = torch.empty(shape[:-1] + (shape[-1] // 32,), device=device, dtype=torch.uint8)
            for b in range(shape[0]):
                packed[b], scale[b] = encode_fp4_rows(_normal(g, shape[1:], device, std))
            return {"data": packed, "scale": scale}
        packed, scale = encode_fp4_rows(_normal(g, shape, device, std))
        return {"data": packed, "scale": scale}
    if dtype in ("nvfp4", "fp8mx"):
        enc = encode_nvfp4_rows if dtype == "nvfp4" else encode_fp8_e8m0_rows
        row_bytes = shape[-1] // 2 + shape[-1] // 16 if dtype == "nvfp4" else shape[-1] + shape[-1] // 32
        if chunk_leading and len(shape) == 3:
            rows = torch.empty(shape[:-1] + (row_bytes,), device=device, dtype=torch.uint8)
            for b in range(shape[0]):
                rows[b] = enc(_normal(g, shape[1:], device, std))
            return {"data": rows}
        return {"data": enc(_normal(g, shape, device, std))}
    raise ValueError(dtype)


def decode_positions(cfg: Csa2Config, g, device):
    b = cfg.batch
    if not cfg.ragged:
        return torch.full((b,), cfg.context - 1, dtype=torch.int64, device=device)
    pos = torch.randint(0, cfg.context, (b,), generator=g, device=device, dtype=torch.int64)
    pins = [0, 1, cfg.window - 1, cfg.window, cfg.context - 1]
    for i, p in enumerate(pins[: b]):
        pos[i] = min(p, cfg.context - 1)
    return pos


def make_candidates(cfg: Csa2Config, pos, g, device):
    """Ascending, -1 padded candidate block ids per query row."""
    rows = pos.shape[0]
    nb, br = cfg.n_blocks, cfg.block_rows
    cand = torch.full((rows, nb), -1, dtype=torch.int32, device=device)
    for r in range(rows):
        nv = (int(pos[r]) + 1) // cfg.ratio
        vis_blocks = (nv + br - 1) // br
        if vis_blocks == 0:
            continue
        newest = vis_blocks - 1
        take = min(nb, vis_blocks)
        if take == vis_blocks:
            ids = torch.arange(vis_blocks, device=device)
        else:
            perm = torch.randperm(vis_blocks - 1, generator=g, device=device)[: take - 1]
            ids = torch.cat([perm, torch.tensor([newest], device=device)])
        cand[r, :take] = torch.sort(ids).values.to(torch.int32)
    return cand


def make_inputs(cfg: Csa2Config, seed: int, device="cpu"):
    """All inputs of one call of the hot path for ``cfg`` (dict of tensors and ints)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    std = 1.0 / math.sqrt(cfg.dim) if cfg.value_scale == "inv_sqrt_d" else 1.0
    H, D, HI, DI, W = cfg.heads, cfg.dim, cfg.idx_heads, cfg.idx_dim, cfg.window
    out = {"cfg": cfg, "seed": int(seed)}
    if cfg.phase == "decode":
        B = cfg.batch
        N = cfg.n_main_rows
        pos = decode_positions(cfg, g, device)
        out["pos"] = pos
        out["kv_row_base"] = torch.arange(B, dtype=torch.int64, device=device) * N
        m = _store_rows(g, (B, N, D), device, std, cfg.main_dtype, chunk_leading=True)
        out["main"], out["main_scale"] = m["data"], m.get("scale")
        s = _store_rows(g, (B, W, D), device, std, cfg.swa_dtype)
        out["swa"], out["swa_scale"] = s["data"], s.get("scale")
        k = _store_rows(g, (B, N, DI), device, std, cfg.idx_dtype, chunk_leading=True)
        out["kI"], out["kI_scale"] = k["data"], k.get("scale")
        rows = B
        out["layers"] = [{
            "q": store_dense(_normal(g, (B, H, D), device, std), cfg.q_dtype),
            "sink": _normal(g, (H,), device, 1.0),
        }]
    else:
        T = cfg.q_tokens
        p0 = cfg.context - T
        N = cfg.n_main_rows
        pos = torch.arange(p0, p0 + T, dtype=torch.int64, device=device)
        out["pos"] = pos
        out["kv_row_base"] = torch.zeros(T, dtype=torch.int64, device=device)
        m = _store_rows(g, (N, D), device, std, cfg.main_dtype)
        out["main"], out["main_scale"] = m["data"], m.get("scale")
        k = _store_rows(g, (N, DI), device, std, cfg.idx_dtype)
        out["kI"], out["kI_scale"] = k["data"], k.get("scale")
        swa_pos0 = max(0, p0 - W + 1)
        swa_rows = p0 + T - swa_pos0
        out["swa_pos0"] = swa_pos0
        layers = []
        for _ in range(1 + cfg.reuse_layers):
            s = _store_rows(g, (swa_rows, D), device, std, cfg.swa_dtype)
            layers.append({
                "q": store_dense(_normal(g, (T, H, D), device, std), cfg.q_dtype),
                "swa": s["data"], "swa_scale": s.get("scale"),
                "sink": _normal(g, (H,), device, 1.0),
            })
        out["layers"] = layers
        rows = T
    # indexer query and weights (the FULL / REINDEX layer's own)
    w = _normal(g, (rows, HI), device, 1.0)
    out["qI_scale"] = None
    if cfg.idx_dtype == "fp8":
        qraw = _normal(g, (rows, HI, DI), device, std)
        codes, qscale = encode_fp8_rows(qraw)
        out["qI"] = codes
        out["w"] = (w * qscale).contiguous()
    elif cfg.idx_dtype == "fp4":
        out["qI"], out["qI_scale"] = encode_fp4_rows(_normal(g, (rows, HI, DI), device, std))
        out["w"] = w.contiguous()
    else:
        out["qI"] = store_dense(_normal(g, (rows, HI, DI), device, std), cfg.idx_dtype)
        out["w"] = w.contiguous()
    if cfg.index_mode == "reindex":
        out["cand"] = make_candidates(cfg, pos, g, device)
    if cfg.d_model:
        # the write path's inputs: one hidden row per query token (its own sequence's newest token in
        # decode, the chunk's tokens in prefill), the owner layer's weights and the tail state
        c = make_compress_inputs(rows, cfg.d_model, cfg.ratio, int(seed) + 7919, device=device, seqs=1)
        slot = torch.arange(rows, dtype=torch.int32, device=device) if cfg.phase == "decode" else \
            torch.zeros(rows, dtype=torch.int32, device=device)
        n_slots = rows if cfg.phase == "decode" else 1
        c.update(pos=pos, slot=slot, row_base=out["kv_row_base"])
        if cfg.ratio == 2:
            c["tail_kv"] = _normal(g, (n_slots, 512), device, 1.0)
            c["tail_score"] = _normal(g, (n_slots, 512), device, 1.0)
        out["compress"] = c
    return out


def make_compress_inputs(rows, d_in, ratio, seed, device="cpu", seqs=None, pos0=0, slots=None, span=4096,
                         plane_rows=8192):
    """Inputs of the FULL layer's write path: bf16 hidden rows and bf16 weights, float32 norm weights and
    tail state, positions and sequence slots.

    ``seqs``: None gives one token per sequence (decode: row r is sequence r at a random position in
    [pos0, pos0 + span)); an int n splits the rows into n consecutive chunks, sequence s covering
    positions pos0 + 17 s ... (prefill chunks).  Weights are scaled so projections are O(1): wkv,
    wgate ~ N(0, 1/d_in), wk ~ N(0, 1/512), norm weights 1 + N(0, 0.01).  Sequence s's plane rows
    start at plane_rows * s (they must hold its rows pos // ratio).
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    bf = lambda shape, std: _normal(g, shape, device, std).to(torch.bfloat16)
    out = {"x": bf((rows, d_in), 1.0), "wkv": bf((512, d_in), d_in ** -0.5), "wk": bf((128, 512), 512 ** -0.5),
           "norm_w": 1.0 + _normal(g, (512,), device, 0.1), "knorm_w": 1.0 + _normal(g, (128,), device, 0.1)}
    out["wgate"] = bf((512, d_in), d_in ** -0.5) if ratio == 2 else None
    if seqs is None:
        slot = torch.arange(rows, dtype=torch.int32, device=device)
        pos = pos0 + torch.randint(0, span, (rows,), generator=g, device=device, dtype=torch.int64)
    else:
        bounds = torch.linspace(0, rows, seqs + 1).round().to(torch.int64).tolist()
        slot = torch.empty(rows, dtype=torch.int32, device=device)
        pos = torch.empty(rows, dtype=torch.int64, device=device)
        for s in range(seqs):
            a, b = bounds[s], bounds[s + 1]
            slot[a:b] = s
            pos[a:b] = pos0 + 17 * s + torch.arange(b - a, device=device)
    n_slots = int(slot.max()) + 1 if slots is None else slots
    out.update(pos=pos, slot=slot, row_base=slot.to(torch.int64) * plane_rows, plane_rows=plane_rows)
    if ratio == 2:
        out["tail_kv"] = _normal(g, (n_slots, 512), device, 1.0)
        out["tail_score"] = _normal(g, (n_slots, 512), device, 1.0)
    else:
        out["tail_kv"] = out["tail_score"] = None
    return out

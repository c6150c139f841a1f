"""One step of the hot path for a workload: output buffers plus the C ABI calls, marshalled once.

A step is the whole path over one batch (see bench.py): for a FULL owner layer
the write path that appends the step's compressed rows, the indexer scores,
the top-k, the candidate pool when the workload's FULL layer builds one, and
sparse attention for every layer that uses the selection.  Wide FULL rows with
an FP8 or MXFP4 index plane take the score-free route (indexer_score with scores=None,
then topk_rescore) whenever the library supports the shape; everything else
writes the scores and runs topk_select.  bench.py times these calls and the
full-size parity tests run exactly the same ones.
"""

import math

import torch


def index_plane_args(cfg, x):
    """(k, keyword arguments) of indexer_score / topk_rescore for the workload's index plane: the plane as
    [*, row elements or bytes] and its scale operands and format flags."""
    if cfg.idx_dtype == "fp4":
        kI = x["kI"].reshape(-1, cfg.idx_dim // 2)
        return kI, dict(fp4=True, k_scale=x["kI_scale"].reshape(-1, cfg.idx_dim // 32), q_scale=x["qI_scale"])
    kI = x["kI"].reshape(-1, cfg.idx_dim)
    kIs = None if x["kI_scale"] is None else x["kI_scale"].reshape(-1)
    return kI, dict(fp8=cfg.idx_dtype == "fp8", k_scale=kIs)


def attn_storage_args(cfg, x):
    """(kv, keyword arguments) of the sparse attention calls for the workload's main and SWA storage."""
    kv = x["main"].reshape(-1, x["main"].shape[-1])
    kvs = None if x["main_scale"] is None else x["main_scale"].reshape(-1, x["main_scale"].shape[-1])
    return kv, dict(rope_dim=cfg.rope_dim, kv_fp4=cfg.main_dtype == "fp4", swa_fp8=cfg.swa_dtype == "fp8",
                    kv_nvfp4=cfg.main_dtype == "nvfp4", swa_fp8mx=cfg.swa_dtype == "fp8mx", kv_scale=kvs)


_MAIN_FORMAT = {"f32": "f32", "bf16": "bf16", "fp4": "fp4", "nvfp4": "nvfp4"}
_IDX_FORMAT = {"f32": "f32", "bf16": "bf16", "fp8": "fp8", "fp4": "fp4"}


def compress_plane_args(cfg, x):
    """Keyword arguments of csa2.compress writing into the workload's main and index planes."""
    main = x["main"].reshape(-1, x["main"].shape[-1])
    idx = x["kI"].reshape(-1, x["kI"].shape[-1])
    ms = None if x["main_scale"] is None else x["main_scale"].reshape(-1, x["main_scale"].shape[-1])
    if x["kI_scale"] is None:
        isc = None
    elif cfg.idx_dtype == "fp8":
        isc = x["kI_scale"].reshape(-1)
    else:
        isc = x["kI_scale"].reshape(-1, x["kI_scale"].shape[-1])
    return main, idx, dict(main_format=_MAIN_FORMAT[cfg.main_dtype], idx_format=_IDX_FORMAT[cfg.idx_dtype],
                           main_scale=ms, idx_scale=isc)


class Step:
    """Buffers and prepared calls of one step, grouped by kernel: ``groups`` maps
    "compress" (owner layers) / "indexer_score" / "topk_select" / "candidate_pool" / "sparse_attn" to lists
    of calls, in launch order."""

    def __init__(self, cfg, x, score_free=None):
        import sparse_latent_attention_amd as csa2
        self.cfg = cfg
        dev = x["pos"].device
        rows = x["pos"].shape[0]
        self.rows = rows
        kI, ikw = index_plane_args(cfg, x)
        kv, akw = attn_storage_args(cfg, x)
        tau_i = 1.0 / math.sqrt(cfg.idx_dim * cfg.idx_heads)
        tau = 1.0 / math.sqrt(cfg.dim)
        quantised = cfg.idx_dtype in ("fp8", "fp4")
        # A prefill chunk's rows share one BF16 plane.  Its score-free route (block keys, the best blocks
        # re-scored) is exact but measured slower than writing the scores (8.40 against 7.40 ms for the
        # 4096-row chunk at 128K: the chunk kernel is bound by its matrix work, so the writes cost little,
        # while re-scoring 1/16 of the columns without shared key tiles costs more than the select
        # saves): it is taken only when asked for (score_free=True, bench.py --topk-route score-free).
        dense = cfg.idx_dtype == "bf16" and cfg.phase == "prefill"
        if score_free is None and dense:
            score_free = False
        if score_free is None:
            score_free = (cfg.index_mode == "full" and (quantised or dense) and
                          csa2.topk_rescore_supported(rows, cfg.width, cfg.topk, cfg.idx_heads, cfg.idx_dim,
                                                      fp8=cfg.idx_dtype == "fp8", fp4=cfg.idx_dtype == "fp4",
                                                      shared_plane=dense))
        self.score_free = score_free
        self.idx = torch.empty(rows, cfg.topk, dtype=torch.int32, device=dev)
        self.outs = [torch.empty_like(L["q"]) for L in x["layers"]]
        self.block_max = self.pool = None
        if cfg.pool_blocks:
            self.block_max = torch.empty(rows, -(-cfg.width // cfg.block_rows), dtype=torch.float32, device=dev)
            self.pool = torch.empty(rows, cfg.pool_blocks, dtype=torch.int32, device=dev)
        freqs = csa2.rope_inv_freq(cfg.rope_dim, cfg.rope_theta, cfg.yarn_factor, cfg.yarn_orig).to(dev)
        self.freqs = freqs

        idx_common = (x["qI"], x["w"], kI, x["kv_row_base"], x["pos"], cfg.ratio, tau_i)
        if score_free:
            self.scores = None
            self.key_hist = None
            # the select needs the block keys' top 16 bits only; the candidate pool and the BF16 route rank
            # blocks by the full keys
            bk_dtype = torch.int32 if (cfg.pool_blocks or dense) else torch.int16
            self.block_keys = torch.empty(rows, -(-cfg.width // 8), dtype=bk_dtype, device=dev)
            # the pool's block scores come from the block keys: no block_max pass
            self.block_max = None
            call_idx = csa2.prepare_indexer_score(*idx_common, None, width=cfg.width, block_keys=self.block_keys,
                                                  shared_plane=dense, **ikw)
            rkw = dict(ikw)
            rkw.pop("fp8", None)
            if dense:
                rkw.update(dense=True, shared_plane=True)
            call_topk = csa2.prepare_topk_rescore(*idx_common, self.idx, self.block_keys, cfg.width, **rkw)
        else:
            self.scores = torch.empty(rows, cfg.width, dtype=torch.float32, device=dev)
            # the indexer also builds the score-key histogram when top-k takes its wide-row path
            self.key_hist = (torch.empty(rows, 4096, dtype=torch.int32, device=dev)
                             if csa2.topk_uses_key_hist(rows, cfg.width, cfg.topk) else None)
            self.block_keys = None
            # a prefill chunk's rows all read the sequence's one plane
            call_idx = csa2.prepare_indexer_score(*idx_common, self.scores, cand=x.get("cand"),
                                                  block_rows=cfg.block_rows, key_hist=self.key_hist,
                                                  block_max=self.block_max, shared_plane=cfg.phase == "prefill",
                                                  **ikw)
            call_topk = csa2.prepare_topk_select(self.scores, x["pos"], cfg.ratio, self.idx, cand=x.get("cand"),
                                                 block_rows=cfg.block_rows, key_hist=self.key_hist)
        self.groups = {}
        if cfg.d_model:
            # the FULL owner layer first appends the step's compressed rows to its planes
            c = x["compress"]
            main, idx, pkw = compress_plane_args(cfg, x)
            self.groups["compress"] = [csa2.prepare_compress(
                c["x"], c["pos"], c["slot"], c["row_base"], c["wkv"], c["norm_w"], c["wk"], c["knorm_w"], freqs,
                main, idx, ratio=cfg.ratio, wgate=c["wgate"], tail_kv=c["tail_kv"], tail_score=c["tail_score"],
                **pkw)]
        self.groups["indexer_score"] = [call_idx]
        self.groups["topk_select"] = [call_topk]
        if cfg.pool_blocks:
            src = dict(block_keys=self.block_keys) if score_free else dict(block_max=self.block_max)
            self.groups["candidate_pool"] = [csa2.prepare_candidate_pool(
                x["pos"], cfg.ratio, self.pool, width=cfg.width, block_rows=cfg.block_rows, **src)]
        attn = []
        for li, L in enumerate(x["layers"]):
            if cfg.phase == "decode":
                attn.append(csa2.prepare_sparse_attn_decode(
                    L["q"], x["pos"], self.idx, kv, x["kv_row_base"], x["swa"], L["sink"], freqs, cfg.ratio,
                    cfg.window, tau, self.outs[li], swa_scale=x["swa_scale"], **akw))
            else:
                attn.append(csa2.prepare_sparse_attn_prefill(
                    L["q"], x["pos"], self.idx, kv, L["swa"], x["swa_pos0"], L["sink"], freqs, cfg.ratio,
                    cfg.window, tau, self.outs[li], swa_scale=L["swa_scale"], kv_row_base=x["kv_row_base"], **akw))
        self.groups["sparse_attn"] = attn

    def __call__(self, on_group=None):
        """Runs every call in order; ``on_group(name)`` is called before each group and once more at the end."""
        for name, calls in self.groups.items():
            if on_group is not None:
                on_group(name)
            for c in calls:
                c()
        if on_group is not None:
            on_group(None)

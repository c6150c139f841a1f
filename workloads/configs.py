"""The five CSA2 workloads, by shape.

Shapes follow the pages' model (DeepSeek-V4.1-Flash): 64 query heads over one
512-dim latent with a 64-dim rope tail, a 128-slot SWA ring, top-512, a 64 x
128 indexer, compression ratio 2 (encoder owners) or 1 (decoder owner), and a
2048 x 8 REINDEX candidate pool.
"""

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Csa2Config:
    name: str
    phase: str            # "decode" (one query per sequence, SWA ring) | "prefill" (one sequence, linear SWA)
    index_mode: str       # "full" | "reindex"
    batch: int            # decode: sequences (= query rows); prefill: 1
    q_tokens: int         # query rows per call
    context: int          # tokens of context up to and including the last query
    ratio: int            # compression ratio m
    heads: int
    dim: int
    rope_dim: int
    rope_theta: float
    yarn_factor: float
    yarn_orig: int
    window: int
    topk: int
    idx_heads: int
    idx_dim: int
    n_blocks: int = 0      # REINDEX candidate blocks per query
    block_rows: int = 8    # rows per candidate block
    reuse_layers: int = 0  # prefill: REUSE layers that attend with the FULL layer's indices
    main_dtype: str = "bf16"   # f32 | bf16 | fp4 (E8M0 / 32, planar) | nvfp4 (288 B rows: E4M3 / 16 inline)
    swa_dtype: str = "bf16"    # f32 | bf16 | fp8 (row scale) | fp8mx (528 B rows: E8M0 / 32 inline)
    idx_dtype: str = "bf16"    # f32 | bf16 | fp8 | fp4 (MXFP4) -- index plane and indexer query
    q_dtype: str = "bf16"      # f32 | bf16
    out_dtype: str = "bf16"    # f32 | bf16
    value_scale: str = "unit"  # "unit": N(0,1); "inv_sqrt_d": N(0,1)/sqrt(dim) for q, latent and index vectors
    ragged: bool = False       # decode: per-sequence positions drawn in [window, context-1]
    pool_blocks: int = 0       # FULL owner layer: candidate blocks it also builds for REINDEX layers (0: none)
    d_model: int = 0           # FULL owner layer: hidden width of the write path that first appends the step's
                               # compressed rows (compressor, main row, index key); 0: planes given as they are

    @property
    def n_main_rows(self):
        """Compressed rows per sequence plane (visible to the last query)."""
        return self.context // self.ratio

    @property
    def width(self):
        return self.n_blocks * self.block_rows if self.index_mode == "reindex" else self.n_main_rows

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


_COMMON = dict(heads=64, dim=512, rope_dim=64, rope_theta=160000.0, yarn_factor=16.0, yarn_orig=65536,
               window=128, topk=512, idx_heads=64, idx_dim=128)

CONFIGS = {
    # 256 causal queries at positions 0..255 of one sequence, fp32 throughout.
    "tiny_full_fp32": Csa2Config(
        name="tiny_full_fp32", phase="prefill", index_mode="full", batch=1, q_tokens=256, context=256, ratio=2,
        heads=4, dim=64, rope_dim=16, rope_theta=10000.0, yarn_factor=1.0, yarn_orig=0, window=16, topk=32,
        idx_heads=4, idx_dim=32, main_dtype="f32", swa_dtype="f32", idx_dtype="f32", q_dtype="f32",
        out_dtype="f32", value_scale="unit"),
    # 32 sequences, one query each at position 65535; 32768 compressed rows per sequence.
    "full_decode_64k": Csa2Config(
        name="full_decode_64k", phase="decode", index_mode="full", batch=32, q_tokens=32, context=65536, ratio=2,
        value_scale="inv_sqrt_d", **_COMMON),
    # 4096-token chunk ending at position 131071: one FULL layer selects, it and 5 REUSE layers attend.
    "prefill_4096_at_128k": Csa2Config(
        name="prefill_4096_at_128k", phase="prefill", index_mode="full", batch=1, q_tokens=4096, context=131072,
        ratio=2, reuse_layers=5, value_scale="unit", **_COMMON),
    # 32 sequences at position 1048575; REINDEX over 2048 candidate blocks x 8 rows of a 1M-row pool each.
    "reindex_decode_1m": Csa2Config(
        name="reindex_decode_1m", phase="decode", index_mode="reindex", batch=32, q_tokens=32, context=1 << 20,
        ratio=1, n_blocks=2048, block_rows=8, value_scale="inv_sqrt_d", **_COMMON),
    # The same REINDEX decode over quantised planes: FP8 index plane (128 B + float32 scale per row) with
    # an FP8 indexer query, FP4 main plane (E8M0 / 32), FP8 SWA ring.
    "reindex_fp8_decode_1m": Csa2Config(
        name="reindex_fp8_decode_1m", phase="decode", index_mode="reindex", batch=32, q_tokens=32,
        context=1 << 20, ratio=1, n_blocks=2048, block_rows=8, main_dtype="fp4", swa_dtype="fp8", idx_dtype="fp8",
        value_scale="inv_sqrt_d", **_COMMON),
    # ... and in the pages' 890 B/token formats: MXFP4 index plane (64 + 4 B per row) and query, packed FP4
    # main rows with E4M3 / 16 (288 B), FP8 SWA rows with E8M0 / 32 (528 B); unit-scale values.
    "reindex_pages_decode_1m": Csa2Config(
        name="reindex_pages_decode_1m", phase="decode", index_mode="reindex", batch=32, q_tokens=32,
        context=1 << 20, ratio=1, n_blocks=2048, block_rows=8, main_dtype="nvfp4", swa_dtype="fp8mx",
        idx_dtype="fp4", value_scale="unit", **_COMMON),
    # 64 sequences at position 1048575; FP4 main plane, FP8 SWA ring, FP8 index plane and indexer query.
    "lowp_full_decode_1m": Csa2Config(
        name="lowp_full_decode_1m", phase="decode", index_mode="full", batch=64, q_tokens=64, context=1 << 20,
        ratio=1, main_dtype="fp4", swa_dtype="fp8", idx_dtype="fp8", value_scale="inv_sqrt_d", **_COMMON),
    # The same decode step as the decoder's FULL owner layer runs it: besides its own top-512 it keeps
    # the 2048 best 8-row blocks as the candidate pool of the REINDEX layers.
    "lowp_pool_decode_1m": Csa2Config(
        name="lowp_pool_decode_1m", phase="decode", index_mode="full", batch=64, q_tokens=64, context=1 << 20,
        ratio=1, main_dtype="fp4", swa_dtype="fp8", idx_dtype="fp8", value_scale="inv_sqrt_d", pool_blocks=2048,
        **_COMMON),
    # The pages' own byte formats (the 890 B/token pool): packed FP4 main rows with an E4M3 scale per 16
    # (288 B), FP8 SWA rows with an E8M0 scale per 32 (528 B), an MXFP4 index plane (64 + 4 B per row) and
    # an MXFP4 indexer query; unit-scale values, like the post-RMSNorm latents the pages quantize.
    "pages_fp4_decode_1m": Csa2Config(
        name="pages_fp4_decode_1m", phase="decode", index_mode="full", batch=64, q_tokens=64, context=1 << 20,
        ratio=1, main_dtype="nvfp4", swa_dtype="fp8mx", idx_dtype="fp4", value_scale="unit", **_COMMON),
    # The decoder's FULL owner layer as one step: the write path (5120-wide hidden rows -> the new
    # compressed row of each sequence, m = 1), then the same scoring, selection and attention.
    "lowp_owner_decode_1m": Csa2Config(
        name="lowp_owner_decode_1m", phase="decode", index_mode="full", batch=64, q_tokens=64, context=1 << 20,
        ratio=1, main_dtype="fp4", swa_dtype="fp8", idx_dtype="fp8", value_scale="inv_sqrt_d", d_model=5120,
        **_COMMON),
    # An encoder FULL owner layer's prefill chunk: the write path pools the chunk's 4096 tokens into 2048
    # rows (m = 2) before the FULL layer scores them; then the 5 REUSE layers.
    "prefill_owner_4096_at_128k": Csa2Config(
        name="prefill_owner_4096_at_128k", phase="prefill", index_mode="full", batch=1, q_tokens=4096,
        context=131072, ratio=2, reuse_layers=5, value_scale="unit", d_model=5120, **_COMMON),
}

CONFIG_ORDER = ["tiny_full_fp32", "full_decode_64k", "prefill_4096_at_128k", "reindex_decode_1m",
                "reindex_fp8_decode_1m", "reindex_pages_decode_1m", "lowp_full_decode_1m", "lowp_pool_decode_1m", "pages_fp4_decode_1m", "lowp_owner_decode_1m",
                "prefill_owner_4096_at_128k"]


def get_config(name):
    return CONFIGS[name]

"""CPU oracle for the CSA2 sparse-attention hot path (test infrastructure).

This package is test infrastructure, not product code.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It is a plain, slow, float64 NumPy transcription of what the pages
define, and it shares no code with the HIP library under
``sparse_latent_attention_amd/``: no kernels, headers, tables or helpers.

Sources (cited by page title and section throughout):

* "DeepSeek-V4.1-Flash 架构解剖" (V4.1-Flash anatomy, ATOM engine view)
* "DeepSeek-V4.1-Flash 结构说明" (V4.1-Flash structure notes)
* "万字长文解析DeekSeekV4.1flash" (long essay, appendix A pseudo-code)
* "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash" (series overview)
* "DeepSeek-V4-Pro 架构解剖" (previous generation; its printed sink-softmax
  and indexer formulas state the mechanics CSA2 keeps)

Modules:

* ``formats``   -- bf16, OCP FP8-E4M3 (FN), FP4-E2M1 and E8M0 decoders
* ``geometry``  -- group-causal visibility, SWA ring / linear window mapping
* ``rope``      -- RoPE / YaRN inverse frequencies, rotation and its inverse
* ``indexer``   -- lightning-indexer scores, FULL and REINDEX
* ``topk``      -- per-row top-k with the ordering contract
* ``candidates`` -- the FULL layer's hierarchical candidate pool (8-row block maxima, top-2048)
* ``attention`` -- single-softmax sink attention over SWA + selected rows
* ``compressor`` -- the FULL layer's write path: pooled latent, main row, index key
* ``quantize``  -- float32 rows to the planes' FP8 / FP4 byte formats

Parity status of each function is stated in its module docstring.
"""

from . import formats, geometry, rope, indexer, topk, candidates, attention, compressor, quantize  # noqa: F401

"""Host-only checks of the C ABI library: it loads, exports what include/csa2.h declares,
the binding's struct layouts match the C compiler's, and argument validation rejects
bad calls before any launch (no GPU needed for any of these)."""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

csa2 = pytest.importorskip("sparse_latent_attention_amd")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(csa2.LIB_PATH)
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(csa2.EXPORTED)
    assert csa2.ABI_VERSION == 9


def test_struct_layouts_match_c_compiler():
    prog = r"""
#include <stdio.h>
#include <stddef.h>
#include "csa2.h"
#define F(T, f) printf(#T " " #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("csa2_index_args sizeof %zu\n", sizeof(csa2_index_args));
  printf("csa2_topk_args sizeof %zu\n", sizeof(csa2_topk_args));
  printf("csa2_attn_args sizeof %zu\n", sizeof(csa2_attn_args));
  printf("csa2_pool_args sizeof %zu\n", sizeof(csa2_pool_args));
  printf("csa2_compress_args sizeof %zu\n", sizeof(csa2_compress_args));
  F(csa2_compress_args, x) F(csa2_compress_args, rope_inv_freq) F(csa2_compress_args, eps) F(csa2_compress_args, k_eps) F(csa2_compress_args, tail_kv) F(csa2_compress_args, idx_scale_out)
  F(csa2_index_args, width) F(csa2_index_args, q) F(csa2_index_args, cand) F(csa2_index_args, scale) F(csa2_index_args, scores) F(csa2_index_args, key_hist) F(csa2_index_args, block_max) F(csa2_index_args, block_keys) F(csa2_index_args, q_scale_e8m0) F(csa2_index_args, k_scale_e8m0)
  F(csa2_pool_args, n_cand) F(csa2_pool_args, width) F(csa2_pool_args, scores) F(csa2_pool_args, block_max) F(csa2_pool_args, pos) F(csa2_pool_args, cand) F(csa2_pool_args, block_keys)
  F(csa2_topk_args, width) F(csa2_topk_args, scores) F(csa2_topk_args, out) F(csa2_topk_args, key_hist)
  F(csa2_attn_args, swa_rows) F(csa2_attn_args, q) F(csa2_attn_args, rope_inv_freq) F(csa2_attn_args, softmax_scale) F(csa2_attn_args, out)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    cls = {"csa2_index_args": csa2.IndexArgs, "csa2_topk_args": csa2.TopkArgs, "csa2_attn_args": csa2.AttnArgs,
           "csa2_pool_args": csa2.PoolArgs, "csa2_compress_args": csa2.CompressArgs}
    for line in out.strip().splitlines():
        t, f, v = line.split()
        if f == "sizeof":
            assert ctypes.sizeof(cls[t]) == int(v), line
        else:
            assert getattr(cls[t], f).offset == int(v), line


def _index_args(**kw):
    a = csa2.IndexArgs()
    a.struct_size = ctypes.sizeof(csa2.IndexArgs)
    a.mode, a.rows, a.heads, a.dim, a.ratio = 0, 4, 64, 128, 2
    a.q_dtype = a.k_dtype = csa2.BF16
    a.width = 100
    for p in ("q", "w", "k", "row_base", "pos", "scores"):
        setattr(a, p, ctypes.c_void_p(0x1000))
    a.scale = 0.01
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 8, csa2.ERR_INVALID_ARG),
    ("mode", 7, csa2.ERR_INVALID_ARG),
    ("ratio", 3, csa2.ERR_INVALID_ARG),
    ("heads", 32, csa2.ERR_UNSUPPORTED),
    ("k_dtype", csa2.F32, csa2.ERR_UNSUPPORTED),
    ("rows", -1, csa2.ERR_INVALID_ARG),
    ("q", None, csa2.ERR_INVALID_ARG),
    ("k_scale", ctypes.c_void_p(0x1000), csa2.ERR_INVALID_ARG),
    ("scale", float("nan"), csa2.ERR_INVALID_ARG),
    ("flags", 2, csa2.ERR_INVALID_ARG),      # 16-bit block keys: score-free mode only
    ("flags", 4, csa2.ERR_INVALID_ARG),
    ("flags", -1, csa2.ERR_INVALID_ARG),
])
def test_indexer_validation(field, value, status):
    a = _index_args(**{field: value})
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == status


def test_indexer_reindex_width_must_match_pool():
    a = _index_args(mode=csa2.MODE_REINDEX, cand=ctypes.c_void_p(0x1000), n_blocks=2048, block_rows=8, width=100)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    a = _index_args(mode=csa2.MODE_REINDEX, cand=None, n_blocks=2048, block_rows=8, width=16384)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG


def test_indexer_empty_calls_do_nothing():
    # no rows or no columns: OK even with a null score pointer (an empty tensor's), which otherwise selects
    # score-free mode
    for kw in (dict(rows=0), dict(width=0)):
        a = _index_args(scores=None, **kw)
        assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.OK, kw


def test_indexer_shared_plane_flag_rules():
    # FULL only; with rows == 0 a valid call returns OK before touching memory
    a = _index_args(flags=csa2.INDEX_SHARED_PLANE, rows=0)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.OK
    a = _index_args(flags=csa2.INDEX_SHARED_PLANE, mode=csa2.MODE_REINDEX, cand=ctypes.c_void_p(0x1000),
                    n_blocks=4, block_rows=8, width=32)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG


def test_indexer_block_max_rules():
    # REINDEX has no block scores; FULL block heights are powers of two in 4..64
    a = _index_args(mode=csa2.MODE_REINDEX, cand=ctypes.c_void_p(0x1000), n_blocks=4, block_rows=8, width=32,
                    block_max=ctypes.c_void_p(0x1000))
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    for b in (0, 2, 6, 128):
        a = _index_args(block_rows=b, block_max=ctypes.c_void_p(0x1000))
        assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG, b
    a = _index_args(block_rows=8, block_max=ctypes.c_void_p(0x1002))
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG


def test_score_free_mode_rules():
    ptr = ctypes.c_void_p(0x1000)
    fp8 = dict(q_dtype=csa2.FP8_E4M3, k_dtype=csa2.FP8_E4M3, k_scale=ptr, width=1 << 20)
    # score-free needs FULL and block_keys (and no key_hist: the select counts the block keys), and a
    # quantised 64 x 128 plane
    a = _index_args(scores=None, **fp8)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    a = _index_args(scores=None, key_hist=ptr, block_keys=ptr, **fp8)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    a = _index_args(scores=None, block_keys=ptr, rows=0, **fp8)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.OK
    a = _index_args(scores=None, block_keys=ptr, mode=csa2.MODE_REINDEX, cand=ptr, n_blocks=2048,
                    block_rows=8, **dict(fp8, width=16384))
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    a = _index_args(scores=None, block_keys=ptr, width=1 << 20)     # bf16
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_UNSUPPORTED
    a = _index_args(scores=None, block_keys=ptr, **dict(fp8, width=1 << 24))
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_UNSUPPORTED
    # block keys are only written in score-free mode
    a = _index_args(block_keys=ptr, key_hist=ptr, **fp8)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG


def test_mxfp4_indexer_rules():
    """MXFP4 q and k take both E8M0 planes (4-byte aligned for k) and no float scale; 64 x 128, FULL or
    REINDEX over 8-row blocks."""
    ptr = ctypes.c_void_p(0x1000)
    fp4 = dict(q_dtype=csa2.FP4_E2M1, k_dtype=csa2.FP4_E2M1, q_scale_e8m0=ptr, k_scale_e8m0=ptr, width=1 << 20)
    call = lambda **kw: csa2._lib.csa2_indexer_score(ctypes.byref(_index_args(**dict(fp4, **kw))), None)
    assert call(rows=0) == csa2.OK                                      # accepted shape, nothing to do
    assert call(q_scale_e8m0=None) == csa2.ERR_INVALID_ARG
    assert call(k_scale_e8m0=None) == csa2.ERR_INVALID_ARG
    assert call(k_scale_e8m0=ctypes.c_void_p(0x1002)) == csa2.ERR_INVALID_ARG
    assert call(k_scale=ptr) == csa2.ERR_INVALID_ARG
    assert call(heads=4, dim=32) == csa2.ERR_UNSUPPORTED
    # MXFP4 REINDEX: the 8-row candidate blocks of the pages' pool only
    assert call(mode=csa2.MODE_REINDEX, cand=ptr, n_blocks=2048, block_rows=16, width=32768) == csa2.ERR_UNSUPPORTED
    assert call(mode=csa2.MODE_REINDEX, cand=ptr, n_blocks=0, block_rows=8, width=0) == csa2.ERR_INVALID_ARG
    # the E8M0 planes belong to MXFP4 only
    a = _index_args(q_scale_e8m0=ptr, k_scale_e8m0=ptr)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    a = _index_args(q_dtype=csa2.FP8_E4M3, k_dtype=csa2.FP8_E4M3, k_scale=ptr, q_scale_e8m0=ptr)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    # score-free mode and the re-scoring select take MXFP4 like FP8
    a = _index_args(scores=None, block_keys=ptr, rows=0, **fp4)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.OK
    a = _index_args(scores=None, block_keys=ptr, **fp4)
    ws = csa2.topk_rescore_workspace_size(a.rows, a.width, 512)
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 512, ptr, ctypes.c_void_p(0x10000), ws - 1, None) == \
        csa2.ERR_WORKSPACE
    a = _index_args(scores=None, block_keys=ptr, **dict(fp4, k_scale_e8m0=None))
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 512, ptr, ctypes.c_void_p(0x10000), ws, None) == \
        csa2.ERR_INVALID_ARG


@pytest.mark.parametrize("kw,k,status", [
    (dict(), 0, csa2.ERR_INVALID_ARG), (dict(), 4096, csa2.ERR_INVALID_ARG),
    (dict(q_dtype=csa2.BF16, k_dtype=csa2.BF16), 512, csa2.ERR_UNSUPPORTED),
    (dict(width=4000), 512, csa2.ERR_UNSUPPORTED),          # narrow rows: no wide-row plan
    (dict(rows=2000), 512, csa2.ERR_UNSUPPORTED),           # many rows: one workgroup per row instead
    (dict(mode=csa2.MODE_REINDEX), 512, csa2.ERR_INVALID_ARG),
    (dict(key_hist=ctypes.c_void_p(0x1000)), 512, csa2.ERR_INVALID_ARG),
    (dict(block_keys=None), 512, csa2.ERR_INVALID_ARG),
])
def test_topk_rescore_validation(kw, k, status):
    ptr = ctypes.c_void_p(0x1000)
    base = dict(q_dtype=csa2.FP8_E4M3, k_dtype=csa2.FP8_E4M3, k_scale=ptr, width=1 << 20, scores=None,
                block_keys=ptr)
    base.update(kw)
    a = _index_args(**base)
    ws = csa2.topk_rescore_workspace_size(a.rows, a.width, 512)
    # every case is rejected on the host, before any launch
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), k, ptr, ctypes.c_void_p(0x10000), ws, None) == status


def test_topk_rescore_workspace_rules():
    ptr = ctypes.c_void_p(0x1000)
    a = _index_args(q_dtype=csa2.FP8_E4M3, k_dtype=csa2.FP8_E4M3, k_scale=ptr, width=1 << 20, scores=None,
                    block_keys=ptr)
    ws = csa2.topk_rescore_workspace_size(4, 1 << 20, 512)
    assert ws >= 2 * 4 * (1 << 20) * 4                      # full-capacity candidate lists
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 512, ptr, ctypes.c_void_p(0x10000), ws - 1, None) == \
        csa2.ERR_WORKSPACE
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 512, ptr, ctypes.c_void_p(0x10040), ws, None) == \
        csa2.ERR_INVALID_ARG
    # narrow rows: no quantised plan, but the BF16 shared-plane plan (the chosen blocks and their re-computed
    # scores) sizes the workspace
    assert csa2.topk_rescore_workspace_size(4, 4000, 512) >= 4 * 512 * 4 + 4 * 4096 * 4


def test_block_keys16_rules():
    """16-bit block keys: score-free FP8 / MXFP4 planes only (not the BF16 shared-plane route, which ranks
    full keys, nor REINDEX), and the re-scoring select takes them with the same flag."""
    ptr = ctypes.c_void_p(0x1000)
    fp8 = dict(q_dtype=csa2.FP8_E4M3, k_dtype=csa2.FP8_E4M3, k_scale=ptr, width=1 << 20, scores=None,
               block_keys=ptr, flags=csa2.INDEX_BLOCK_KEYS16)
    a = _index_args(rows=0, **fp8)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.OK
    a = _index_args(**dict(fp8, scores=ptr, block_keys=None))
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    a = _index_args(**dict(fp8, mode=csa2.MODE_REINDEX, cand=ptr, n_blocks=2048, block_rows=8, width=16384))
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    dense = dict(q_dtype=csa2.BF16, k_dtype=csa2.BF16, width=70000, scores=None, block_keys=ptr, rows=4096,
                 flags=csa2.INDEX_SHARED_PLANE | csa2.INDEX_BLOCK_KEYS16)
    a = _index_args(**dense)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_INVALID_ARG
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 512, ptr, ctypes.c_void_p(0x10000), 1 << 30, None) == \
        csa2.ERR_INVALID_ARG
    # accepted by the select: the workspace check is the next one it makes
    a = _index_args(**fp8)
    ws = csa2.topk_rescore_workspace_size(a.rows, a.width, 512)
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 512, ptr, ctypes.c_void_p(0x10000), ws - 1, None) == \
        csa2.ERR_WORKSPACE


def test_topk_rescore_bf16_shared_plane_rules():
    """BF16 score-free rows must state that they share one plane; then any width and row count is taken."""
    ptr = ctypes.c_void_p(0x1000)
    base = dict(q_dtype=csa2.BF16, k_dtype=csa2.BF16, width=70000, scores=None, block_keys=ptr, rows=4096)
    a = _index_args(**base)
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 512, ptr, ctypes.c_void_p(0x10000), 1 << 30, None) == \
        csa2.ERR_UNSUPPORTED
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.ERR_UNSUPPORTED
    a = _index_args(flags=csa2.INDEX_SHARED_PLANE, **base)
    ws = csa2.topk_rescore_workspace_size(4096, 70000, 512)
    assert ws >= 4096 * 512 * 4 + 4096 * 4096 * 4
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 512, ptr, ctypes.c_void_p(0x10000), ws - 1, None) == \
        csa2.ERR_WORKSPACE
    assert csa2._lib.csa2_topk_rescore(ctypes.byref(a), 0, ptr, ctypes.c_void_p(0x10000), ws, None) == \
        csa2.ERR_INVALID_ARG
    assert csa2.topk_rescore_supported(4096, 65536, 512, fp8=False, fp4=False, shared_plane=True)
    assert not csa2.topk_rescore_supported(4096, 65536, 512, fp8=False, fp4=False, shared_plane=False)
    assert not csa2.topk_rescore_supported(4096, 65536, 512, fp8=True)


def _pool_args(**kw):
    a = csa2.PoolArgs()
    a.struct_size = ctypes.sizeof(csa2.PoolArgs)
    a.rows, a.ratio, a.block_rows, a.n_cand, a.width = 4, 1, 8, 2048, 1 << 20
    a.scores = a.pos = a.cand = ctypes.c_void_p(0x1000)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 8, csa2.ERR_INVALID_ARG), ("n_cand", 0, csa2.ERR_INVALID_ARG),
    ("n_cand", 4096, csa2.ERR_INVALID_ARG), ("block_rows", 6, csa2.ERR_INVALID_ARG),
    ("block_rows", 2, csa2.ERR_INVALID_ARG), ("block_rows", 128, csa2.ERR_INVALID_ARG),
    ("ratio", 3, csa2.ERR_INVALID_ARG), ("width", 1 << 31, csa2.ERR_INVALID_ARG),
    ("scores", None, csa2.ERR_INVALID_ARG), ("cand", None, csa2.ERR_INVALID_ARG),
])
def test_candidate_pool_validation(field, value, status):
    a = _pool_args(**{field: value})
    ws = csa2.candidate_pool_workspace_size(4, 1 << 20, 8, 2048)
    # every case is rejected on the host, before any launch
    assert csa2._lib.csa2_candidate_pool(ctypes.byref(a), ctypes.c_void_p(0x10000), ws, None) == status


def test_candidate_pool_workspace_rules():
    ws = csa2.candidate_pool_workspace_size(4, 1 << 20, 8, 2048)
    assert ws >= 4 * (1 << 17) * 4                     # room for the block scores it may compute
    a = _pool_args()
    assert csa2._lib.csa2_candidate_pool(ctypes.byref(a), ctypes.c_void_p(0x10000), ws - 1, None) == \
        csa2.ERR_WORKSPACE
    assert csa2._lib.csa2_candidate_pool(ctypes.byref(a), ctypes.c_void_p(0x10010), ws, None) == \
        csa2.ERR_INVALID_ARG                            # workspace must be 256-byte aligned
    a = _pool_args(rows=0)
    assert csa2._lib.csa2_candidate_pool(ctypes.byref(a), None, 0, None) == csa2.OK


def test_empty_calls_launch_nothing():
    a = _index_args(rows=0)
    assert csa2._lib.csa2_indexer_score(ctypes.byref(a), None) == csa2.OK
    t = csa2.TopkArgs()
    t.struct_size, t.rows, t.k, t.ratio, t.width = ctypes.sizeof(csa2.TopkArgs), 0, 512, 1, 1000
    assert csa2._lib.csa2_topk_select(ctypes.byref(t), None, 0, None) == csa2.OK


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, csa2.ERR_INVALID_ARG), ("k", 4096, csa2.ERR_INVALID_ARG), ("ratio", 0, csa2.ERR_INVALID_ARG),
    ("width", 1 << 31, csa2.ERR_INVALID_ARG), ("n_blocks", 3, csa2.ERR_INVALID_ARG),
])
def test_topk_validation(field, value, status):
    t = csa2.TopkArgs()
    t.struct_size, t.rows, t.k, t.ratio, t.width = ctypes.sizeof(csa2.TopkArgs), 2, 512, 1, 1000
    t.scores = t.pos = t.out = ctypes.c_void_p(0x1000)
    setattr(t, field, value)
    assert csa2._lib.csa2_topk_select(ctypes.byref(t), None, 0, None) == status


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, csa2.ERR_INVALID_ARG), ("k", 4096, csa2.ERR_INVALID_ARG), ("ratio", 0, csa2.ERR_INVALID_ARG),
    ("width", 1 << 31, csa2.ERR_INVALID_ARG), ("n_blocks", 3, csa2.ERR_INVALID_ARG),
])
def test_topk_noalloc_validation(field, value, status):
    t = csa2.TopkArgs()
    t.struct_size, t.rows, t.k, t.ratio, t.width = ctypes.sizeof(csa2.TopkArgs), 2, 512, 1, 1000
    t.scores = t.pos = t.out = ctypes.c_void_p(0x1000)
    setattr(t, field, value)
    assert csa2._lib.csa2_topk_select_noalloc(ctypes.byref(t), None) == status


def test_topk_noalloc_rejects_sizes_beyond_its_scratch():
    """Shapes whose workspace is larger than the fixed scratch are refused before any HIP call; the
    decode shapes fit; empty calls do nothing."""
    cap = csa2.NOALLOC_SCRATCH_BYTES
    assert cap == 40 << 20
    t = csa2.TopkArgs()
    t.struct_size, t.k, t.ratio = ctypes.sizeof(csa2.TopkArgs), 512, 1
    t.scores = t.pos = t.out = ctypes.c_void_p(0x1000)
    t.rows, t.width = 1023, 131072
    assert csa2.topk_workspace_size(1023, 131072, 512) > cap
    assert csa2._lib.csa2_topk_select_noalloc(ctypes.byref(t), None) == csa2.ERR_WORKSPACE
    for rows, width in ((32, 65537), (64, 1 << 20), (256, 1 << 20)):
        assert 0 < csa2.topk_workspace_size(rows, width, 512) <= cap
    # rows up to 65536 wide take one workgroup per row: no workspace at any row count
    for rows, width in ((1, 65536), (32, 16384), (1023, 65536), (4096, 65536)):
        assert csa2.topk_workspace_size(rows, width, 512) == 0
    t.rows = 0
    assert csa2._lib.csa2_topk_select_noalloc(ctypes.byref(t), None) == csa2.OK


def _attn_args(**kw):
    a = csa2.AttnArgs()
    a.struct_size = ctypes.sizeof(csa2.AttnArgs)
    a.rows, a.heads, a.dim, a.rope_dim, a.topk, a.ratio, a.window = 4, 64, 512, 64, 512, 1, 128
    a.q_dtype = a.kv_dtype = a.swa_dtype = a.out_dtype = csa2.BF16
    for p in ("q", "pos", "idx", "kv", "kv_row_base", "swa", "sink", "rope_inv_freq", "out"):
        setattr(a, p, ctypes.c_void_p(0x1000))
    a.softmax_scale = 0.044
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("window", 100, csa2.ERR_INVALID_ARG), ("topk", 500, csa2.ERR_INVALID_ARG), ("ratio", 4, csa2.ERR_INVALID_ARG),
    ("window", 2048, csa2.ERR_INVALID_ARG), ("topk", 4096, csa2.ERR_INVALID_ARG),
    ("heads", 32, csa2.ERR_UNSUPPORTED), ("kv_dtype", csa2.FP8_E4M3, csa2.ERR_UNSUPPORTED),
    ("q_dtype", csa2.F32, csa2.ERR_UNSUPPORTED), ("kv_dtype", csa2.FP4_E2M1, csa2.ERR_INVALID_ARG),
    ("softmax_scale", 0.0, csa2.ERR_INVALID_ARG), ("sink", None, csa2.ERR_INVALID_ARG),
    ("q", ctypes.c_void_p(0x1004), csa2.ERR_INVALID_ARG),
])
def test_attention_validation(field, value, status):
    a = _attn_args(**{field: value})
    assert csa2._lib.csa2_sparse_attn_prefill(ctypes.byref(a), None) == status


def test_attention_inline_scale_rows():
    """E2M1 + E4M3/16 kv goes with FP8 + E8M0/32 swa and takes no separate scale arrays."""
    ptr = ctypes.c_void_p(0x1000)
    g = dict(kv_dtype=csa2.FP4_E2M1_E4M3G16, swa_dtype=csa2.FP8_E4M3_E8M0G32)
    run = lambda **kw: csa2._lib.csa2_sparse_attn_prefill(ctypes.byref(_attn_args(**kw)), None)
    assert run(rows=0, **g) == csa2.OK
    assert run(kv_scale=ptr, **g) == csa2.ERR_INVALID_ARG
    assert run(swa_scale=ptr, **g) == csa2.ERR_INVALID_ARG
    assert run(kv_dtype=csa2.FP4_E2M1_E4M3G16) == csa2.ERR_UNSUPPORTED            # with bf16 swa
    assert run(swa_dtype=csa2.FP8_E4M3_E8M0G32) == csa2.ERR_UNSUPPORTED           # with bf16 kv
    assert run(kv_dtype=csa2.FP4_E2M1, kv_scale=ptr, swa_dtype=csa2.FP8_E4M3_E8M0G32) == csa2.ERR_UNSUPPORTED


def test_decode_split_workspace_rules():
    """Decode rows split their entries over workgroups (256 / rows, at most 8, at most 4 from 32 rows on,
    at most one per pair of tiles) and need a workspace for the partial states; single splits need none."""
    per = 4 * 16 * (2 + 512) * 4                                   # 4 head groups x 16 heads x (max, sum, 512 values)
    assert csa2.attn_workspace_size(32, 64, 512, 128, 512, 0) == 32 * 4 * per    # 4 splits from 32 rows on
    assert csa2.attn_workspace_size(16, 64, 512, 128, 512, 0) == 16 * 8 * per    # 256 workgroups
    assert csa2.attn_workspace_size(32, 64, 512, 128, 512, 1) == 0
    assert csa2.attn_workspace_size(32, 64, 512, 128, 512, 3) == 32 * 3 * per
    assert csa2.attn_workspace_size(64, 64, 512, 128, 512, 0) == 64 * 4 * per    # 4 splits
    assert csa2.attn_workspace_size(300, 64, 512, 128, 512, 0) == 0            # one workgroup per row
    assert csa2.attn_workspace_size(1, 64, 512, 16, 16, 0) == 0                # one pair of tiles: no split
    assert csa2.attn_workspace_size(1, 64, 512, 128, 256, 0) == 1 * 8 * per    # 24 tiles: 8 splits
    assert csa2.attn_workspace_size(1, 64, 512, 64, 64, 0) == 1 * 4 * per      # 8 tiles: at most 4 splits
    a = _attn_args(rows=32, splits=0)
    need = csa2.attn_workspace_size(32, 64, 512, 128, 512, 0)
    assert csa2._lib.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == csa2.ERR_WORKSPACE
    assert csa2._lib.csa2_sparse_attn_decode(ctypes.byref(a), ctypes.c_void_p(0x10000), need - 1, None) == \
        csa2.ERR_WORKSPACE
    assert csa2._lib.csa2_sparse_attn_decode(ctypes.byref(a), ctypes.c_void_p(0x10040), need, None) == \
        csa2.ERR_INVALID_ARG                                        # not 256-byte aligned
    a = _attn_args(rows=8, splits=9)
    assert csa2._lib.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == csa2.ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert csa2.status_string(s)
    assert csa2.status_string(99) == "unknown status"


@pytest.mark.parametrize("dim,theta,factor,orig", [(64, 160000.0, 16.0, 65536), (16, 10000.0, 1.0, 0),
                                                   (64, 10000.0, 1.0, 0)])
def test_rope_table_matches_oracle(dim, theta, factor, orig):
    import oracle
    ours = csa2.rope_inv_freq(dim, theta, factor, orig).numpy()
    ref = oracle.rope.inv_freq(dim, theta, factor, orig)
    assert np.allclose(ours, ref, rtol=1e-14, atol=0)


def test_rope_table_rejects_bad_args():
    out = (ctypes.c_double * 8)()
    assert csa2._lib.csa2_rope_inv_freq(15, 1e4, 1.0, 0, out) == csa2.ERR_INVALID_ARG
    assert csa2._lib.csa2_rope_inv_freq(16, 0.5, 1.0, 0, out) == csa2.ERR_INVALID_ARG
    assert csa2._lib.csa2_rope_inv_freq(16, 1e4, 1.0, 0, None) == csa2.ERR_INVALID_ARG


def _compress_args(**kw):
    a = csa2.CompressArgs()
    a.struct_size = ctypes.sizeof(csa2.CompressArgs)
    a.rows, a.d_in, a.ratio, a.dim, a.idx_dim, a.rope_dim = 4, 5120, 2, 512, 128, 64
    a.main_dtype, a.idx_dtype = csa2.FP4_E2M1, csa2.FP8_E4M3
    for f in ("x", "pos", "slot", "row_base", "wkv", "wgate", "norm_w", "wk", "knorm_w", "rope_inv_freq", "tail_kv",
              "tail_score", "main_out", "main_scale_out", "idx_out", "idx_scale_out"):
        setattr(a, f, ctypes.c_void_p(0x1000))
    a.eps = a.k_eps = 1e-6
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), csa2.ERR_INVALID_ARG), (dict(ratio=3), csa2.ERR_INVALID_ARG),
    (dict(rows=-1), csa2.ERR_INVALID_ARG), (dict(dim=256), csa2.ERR_UNSUPPORTED),
    (dict(idx_dim=64), csa2.ERR_UNSUPPORTED), (dict(d_in=100), csa2.ERR_UNSUPPORTED),
    (dict(main_dtype=csa2.FP8_E4M3), csa2.ERR_UNSUPPORTED), (dict(idx_dtype=csa2.FP4_E2M1_E4M3G16), csa2.ERR_UNSUPPORTED),
    (dict(wgate=None), csa2.ERR_INVALID_ARG), (dict(tail_kv=None), csa2.ERR_INVALID_ARG),
    (dict(ratio=1), csa2.ERR_INVALID_ARG),                       # ratio 1 takes no gate and no tail state
    (dict(main_scale_out=None), csa2.ERR_INVALID_ARG), (dict(idx_scale_out=None), csa2.ERR_INVALID_ARG),
    (dict(main_dtype=csa2.BF16), csa2.ERR_INVALID_ARG),          # bf16 rows take no scale array
    (dict(eps=float("nan")), csa2.ERR_INVALID_ARG), (dict(k_eps=-1.0), csa2.ERR_INVALID_ARG),
    (dict(x=ctypes.c_void_p(0x1008)), csa2.ERR_INVALID_ARG), (dict(x=None), csa2.ERR_INVALID_ARG),
])
def test_compress_validation(kw, status):
    a = _compress_args(**kw)
    ws = max(csa2.compress_workspace_size(4, 5120, 2), 256)
    assert csa2._lib.csa2_compress(ctypes.byref(a), ctypes.c_void_p(0x10000), ws, None) == status


def test_compress_workspace_rules():
    # decode shapes split the 5120-wide reduction; the workspace holds every partial tile
    assert csa2.compress_workspace_size(64, 5120, 2) == 16 * 64 * 1024 * 4
    assert csa2.compress_workspace_size(4096, 5120, 2) == 4096 * 1024 * 4
    assert csa2.compress_workspace_size(64, 5120, 1) == 16 * 64 * 512 * 4
    assert csa2.compress_workspace_size(1024, 5120, 1) == 8 * 1024 * 512 * 4
    assert csa2.compress_workspace_size(0, 5120, 2) == 0 and csa2.compress_workspace_size(4, 100, 2) == 0
    a = _compress_args()
    need = csa2.compress_workspace_size(4, 5120, 2)
    assert csa2._lib.csa2_compress(ctypes.byref(a), ctypes.c_void_p(0x10000), need - 1, None) == csa2.ERR_WORKSPACE
    a = _compress_args(rows=0)
    assert csa2._lib.csa2_compress(ctypes.byref(a), None, 0, None) == csa2.OK

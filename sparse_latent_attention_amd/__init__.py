"""Python binding of libcsa2 (the CSA2 sparse-attention hot path for MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libcsa2.so``.  Torch tensors provide device memory and the current HIP
stream.  The library must have been built (``python
sparse_latent_attention_amd/build.py``); importing this package without it
raises ``ImportError`` -- there is no CPU fallback.

Entry points (same names as the C ABI in include/csa2.h):

* ``indexer_score``        lightning-indexer scores, FULL or REINDEX (or, with
                           ``scores=None``, only the block keys ``topk_rescore`` needs)
* ``topk_select``          per-row top-k of written scores
* ``topk_rescore``         top-k of FULL scores that were kept on chip
* ``candidate_pool``       the FULL owner layer's 2048 x 8 REINDEX candidate blocks
* ``sparse_attn_decode``   sink attention, SWA ring per query row
* ``sparse_attn_prefill``  sink attention, one linear SWA array
* ``compress``             the FULL owner layer's write path (compressor, main row, index key)
* ``rope_inv_freq``        float64 RoPE / YaRN frequency table (host)

``prepare_*`` variants marshal a call's arguments once and return a callable
that only crosses into the library (what bench.py times).
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa2.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_latent_attention_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

# Element types and modes (include/csa2.h).
F32, BF16, FP8_E4M3, FP4_E2M1, FP4_E2M1_E4M3G16, FP8_E4M3_E8M0G32 = 0, 1, 2, 3, 4, 5
MODE_FULL, MODE_REINDEX = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4

_vp = ctypes.c_void_p
_i32, _i64, _u32, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float


class IndexArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("mode", _i32), ("rows", _i32), ("heads", _i32), ("dim", _i32), ("ratio", _i32),
        ("q_dtype", _i32), ("k_dtype", _i32), ("n_blocks", _i32), ("block_rows", _i32), ("flags", _i32),
        ("width", _i64), ("q", _vp), ("w", _vp), ("k", _vp), ("k_scale", _vp), ("row_base", _vp), ("pos", _vp),
        ("cand", _vp), ("scale", _f32), ("_pad1", _i32), ("scores", _vp), ("key_hist", _vp), ("block_max", _vp),
        ("block_keys", _vp), ("q_scale_e8m0", _vp), ("k_scale_e8m0", _vp),
    ]


class TopkArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("rows", _i32), ("k", _i32), ("ratio", _i32), ("n_blocks", _i32),
        ("block_rows", _i32), ("width", _i64), ("scores", _vp), ("pos", _vp), ("cand", _vp), ("out", _vp),
        ("key_hist", _vp),
    ]


class PoolArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("rows", _i32), ("ratio", _i32), ("block_rows", _i32), ("n_cand", _i32),
        ("_pad0", _i32), ("width", _i64), ("scores", _vp), ("block_max", _vp), ("pos", _vp), ("cand", _vp),
        ("block_keys", _vp),
    ]


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("rows", _i32), ("heads", _i32), ("dim", _i32), ("rope_dim", _i32), ("topk", _i32),
        ("ratio", _i32), ("window", _i32), ("q_dtype", _i32), ("kv_dtype", _i32), ("swa_dtype", _i32),
        ("out_dtype", _i32), ("splits", _i32), ("_pad0", _i32), ("swa_rows", _i64), ("swa_pos0", _i64),
        ("q", _vp), ("pos", _vp), ("idx", _vp), ("kv", _vp), ("kv_scale", _vp), ("kv_row_base", _vp),
        ("swa", _vp), ("swa_scale", _vp), ("sink", _vp), ("rope_inv_freq", _vp), ("softmax_scale", _f32),
        ("_pad1", _i32), ("out", _vp),
    ]


class CompressArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("rows", _i32), ("d_in", _i32), ("ratio", _i32), ("dim", _i32), ("idx_dim", _i32),
        ("rope_dim", _i32), ("main_dtype", _i32), ("idx_dtype", _i32), ("_pad0", _i32), ("x", _vp), ("pos", _vp),
        ("slot", _vp), ("row_base", _vp), ("wkv", _vp), ("wgate", _vp), ("norm_w", _vp), ("wk", _vp),
        ("knorm_w", _vp), ("rope_inv_freq", _vp), ("eps", _f32), ("k_eps", _f32), ("tail_kv", _vp),
        ("tail_score", _vp), ("main_out", _vp), ("main_scale_out", _vp), ("idx_out", _vp), ("idx_scale_out", _vp),
    ]


_lib.csa2_abi_version.restype = _i32
_lib.csa2_status_string.restype = ctypes.c_char_p
_lib.csa2_status_string.argtypes = [_i32]
_lib.csa2_indexer_score.restype = _i32
_lib.csa2_indexer_score.argtypes = [ctypes.POINTER(IndexArgs), _vp]
_lib.csa2_topk_workspace_size.restype = ctypes.c_size_t
_lib.csa2_topk_workspace_size.argtypes = [_i32, _i64, _i32]
_lib.csa2_topk_select.restype = _i32
_lib.csa2_topk_select.argtypes = [ctypes.POINTER(TopkArgs), _vp, ctypes.c_size_t, _vp]
_lib.csa2_topk_rescore_workspace_size.restype = ctypes.c_size_t
_lib.csa2_topk_rescore_workspace_size.argtypes = [_i32, _i64, _i32]
_lib.csa2_topk_rescore.restype = _i32
_lib.csa2_topk_rescore.argtypes = [ctypes.POINTER(IndexArgs), _i32, _vp, _vp, ctypes.c_size_t, _vp]
_lib.csa2_candidate_pool_workspace_size.restype = ctypes.c_size_t
_lib.csa2_candidate_pool_workspace_size.argtypes = [_i32, _i64, _i32, _i32]
_lib.csa2_candidate_pool.restype = _i32
_lib.csa2_candidate_pool.argtypes = [ctypes.POINTER(PoolArgs), _vp, ctypes.c_size_t, _vp]
_lib.csa2_attn_workspace_size.restype = ctypes.c_size_t
_lib.csa2_attn_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
_lib.csa2_sparse_attn_decode.restype = _i32
_lib.csa2_sparse_attn_decode.argtypes = [ctypes.POINTER(AttnArgs), _vp, ctypes.c_size_t, _vp]
_lib.csa2_sparse_attn_prefill.restype = _i32
_lib.csa2_sparse_attn_prefill.argtypes = [ctypes.POINTER(AttnArgs), _vp]
_lib.csa2_compress_workspace_size.restype = ctypes.c_size_t
_lib.csa2_compress_workspace_size.argtypes = [_i32, _i32, _i32]
_lib.csa2_compress.restype = _i32
_lib.csa2_compress.argtypes = [ctypes.POINTER(CompressArgs), _vp, ctypes.c_size_t, _vp]
_lib.csa2_topk_noalloc_scratch_bytes.restype = ctypes.c_size_t
_lib.csa2_topk_noalloc_scratch_bytes.argtypes = []
_lib.csa2_topk_select_noalloc.restype = _i32
_lib.csa2_topk_select_noalloc.argtypes = [ctypes.POINTER(TopkArgs), _vp]
_lib.csa2_rope_inv_freq.restype = _i32
_lib.csa2_rope_inv_freq.argtypes = [_i32, ctypes.c_double, ctypes.c_double, _i64, ctypes.POINTER(ctypes.c_double)]

ABI_VERSION = _lib.csa2_abi_version()
EXPORTED = ("csa2_abi_version", "csa2_status_string", "csa2_indexer_score", "csa2_topk_workspace_size",
            "csa2_topk_select", "csa2_topk_rescore_workspace_size", "csa2_topk_rescore",
            "csa2_candidate_pool_workspace_size", "csa2_candidate_pool", "csa2_attn_workspace_size", "csa2_sparse_attn_decode", "csa2_sparse_attn_prefill",
            "csa2_compress_workspace_size", "csa2_compress", "csa2_rope_inv_freq", "csa2_topk_noalloc_scratch_bytes",
            "csa2_topk_select_noalloc")


class Csa2Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def status_string(status):
    return _lib.csa2_status_string(int(status)).decode()


def _check(fn, status):
    if status != OK:
        raise Csa2Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("csa2: all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("csa2: all tensors must be contiguous")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dense_code(t, name):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"csa2: {name} must be float32 or bfloat16, got {t.dtype}")


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise ValueError(f"csa2: {name} must be {dtype}, got {t.dtype}")


def _scratch(nbytes, device, stream):
    """A workspace the call allocates itself.  It is allocated on torch's current stream; when the
    call runs on another stream, the caching allocator is told so (record_stream), so the block is
    not handed out again before that stream's kernels are done with it."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(ws.device):
        ws.record_stream(stream)
    return ws


def rope_inv_freq(rope_dim, theta, yarn_factor=1.0, yarn_orig_len=0):
    """float64 frequency table computed by the library on the host (CPU tensor)."""
    out = (ctypes.c_double * (rope_dim // 2))()
    _check("csa2_rope_inv_freq", _lib.csa2_rope_inv_freq(int(rope_dim), float(theta), float(yarn_factor),
                                                          int(yarn_orig_len), out))
    return torch.tensor(list(out), dtype=torch.float64)


def _index_args(q, w, k, row_base, pos, ratio, scale, scores, width, k_scale, cand, block_rows, fp8, key_hist,
                block_max, block_keys, fp4=False, q_scale=None):
    _dev(q, w, k, row_base, pos, scores, k_scale, cand, key_hist, block_max, block_keys, q_scale)
    if key_hist is not None and (key_hist.dtype != torch.int32 or tuple(key_hist.shape) != (q.shape[0], 4096)):
        raise ValueError("csa2.indexer_score: key_hist must be int32 [rows, 4096]")
    rows, heads, dim = q.shape
    if fp8 and fp4:
        raise ValueError("csa2.indexer_score: fp8 and fp4 exclude each other")
    if fp4:
        # packed E2M1: q [rows, heads, dim / 2], k [*, dim / 2]; E8M0 scales per 32 elements
        _need(q, torch.uint8, "q")
        _need(k, torch.uint8, "k")
        _need(q_scale, torch.uint8, "q_scale")
        _need(k_scale, torch.uint8, "k_scale")
        code = FP4_E2M1
        if tuple(q_scale.shape) != (rows, heads, dim // 16) or k_scale.shape[-1] != dim // 16:
            raise ValueError("csa2.indexer_score: fp4 scales must be [rows, heads, dim / 32] and [*, dim / 32]")
    elif q_scale is not None:
        raise ValueError("csa2.indexer_score: q_scale is for fp4 only")
    elif fp8:
        _need(q, torch.uint8, "q")
        _need(k, torch.uint8, "k")
        code = FP8_E4M3
    else:
        code = _dense_code(q, "q")
        if k.dtype != q.dtype:
            raise ValueError("csa2: q and k must share a dtype")
    _need(w, torch.float32, "w")
    _need(row_base, torch.int64, "row_base")
    _need(pos, torch.int64, "pos")
    if scores is not None:
        _need(scores, torch.float32, "scores")
        if scores.shape[0] != rows:
            raise ValueError("csa2.indexer_score: scores rows")
        width = scores.shape[1]
    if w.shape != (rows, heads) or k.shape[-1] != dim or row_base.shape != (rows,) or pos.shape != (rows,):
        raise ValueError("csa2.indexer_score: inconsistent shapes")
    a = IndexArgs()
    a.struct_size = ctypes.sizeof(IndexArgs)
    a.mode = MODE_REINDEX if cand is not None else MODE_FULL
    a.rows, a.heads, a.dim, a.ratio = rows, heads, 2 * dim if fp4 else dim, int(ratio)
    a.q_dtype = a.k_dtype = code
    a.width = int(width)
    if cand is not None:
        _need(cand, torch.int32, "cand")
        if cand.shape[0] != rows:
            raise ValueError("csa2.indexer_score: cand rows")
        a.n_blocks, a.block_rows = cand.shape[1], int(block_rows)
    if block_max is not None:
        _need(block_max, torch.float32, "block_max")
        nb = -(-a.width // int(block_rows))
        if tuple(block_max.shape) != (rows, nb):
            raise ValueError(f"csa2.indexer_score: block_max must be [rows, {nb}]")
        a.block_rows = int(block_rows)
    if block_keys is not None:
        # int32: the full 32-bit block keys; int16: their top 16 bits (INDEX_BLOCK_KEYS16)
        if block_keys.dtype not in (torch.int32, torch.int16):
            raise ValueError("csa2: block_keys must be int32 or int16")
        if tuple(block_keys.shape) != (rows, -(-a.width // 8)):
            raise ValueError("csa2.indexer_score: block_keys must be [rows, ceil(width / 8)]")
        if block_keys.dtype == torch.int16:
            a.flags |= INDEX_BLOCK_KEYS16
    a.block_max, a.block_keys = _ptr(block_max), _ptr(block_keys)
    if fp4:
        a.q_scale_e8m0, a.k_scale_e8m0 = _ptr(q_scale), _ptr(k_scale)
        a.q, a.w, a.k = _ptr(q), _ptr(w), _ptr(k)
    else:
        a.q, a.w, a.k, a.k_scale = _ptr(q), _ptr(w), _ptr(k), _ptr(k_scale)
    a.row_base, a.pos, a.cand, a.scores = _ptr(row_base), _ptr(pos), _ptr(cand), _ptr(scores)
    a.key_hist = _ptr(key_hist)
    a.scale = float(scale)
    return a


INDEX_SHARED_PLANE = 1
INDEX_BLOCK_KEYS16 = 2


def indexer_score(q, w, k, row_base, pos, ratio, scale, scores, *, k_scale=None, cand=None, block_rows=8,
                  fp8=False, fp4=False, q_scale=None, key_hist=None, block_max=None, block_keys=None, width=None,
                  shared_plane=False, stream=None):
    """Fills ``scores`` [rows, width] (float32).  REINDEX when ``cand`` is given.

    q [rows, H_I, D_I] and k [*, D_I] are float32/bfloat16, or uint8 FP8-E4M3
    codes with ``fp8=True`` (then ``k_scale`` [*] float32 is required and the
    query scales are already folded into w), or MXFP4 with ``fp4=True``: packed
    E2M1 q [rows, H_I, D_I / 2] and k [*, D_I / 2] with E8M0 block scales
    ``q_scale`` [rows, H_I, D_I / 32] and ``k_scale`` [*, D_I / 32] (uint8;
    FULL only).  ``key_hist`` (int32 [rows, 4096])
    optionally receives the score-key histogram topk_select can reuse.
    ``block_max`` (FULL only, float32 [rows, ceil(width / block_rows)])
    optionally receives the candidate pool's block scores.  ``scores=None``
    (with ``width`` and ``block_keys`` [rows, ceil(width / 8)], no ``key_hist``)
    selects the score-free mode whose top-k ``topk_rescore`` takes; int32 block
    keys are the full keys, int16 ones their top 16 bits (FP8 / MXFP4 planes: half
    the bytes, and all the select needs; the candidate pool needs int32).
    ``shared_plane=True`` (FULL only) states that every row reads the plane rows of
    ``row_base[0]`` (a prefill chunk of one sequence); the library may then stage
    key tiles once for several rows (same results).
    """
    a = _index_args(q, w, k, row_base, pos, ratio, scale, scores, width, k_scale, cand, block_rows, fp8, key_hist,
                    block_max, block_keys, fp4, q_scale)
    a.flags |= INDEX_SHARED_PLANE if shared_plane else 0
    _check("csa2_indexer_score", _lib.csa2_indexer_score(ctypes.byref(a), _stream(stream)))
    return scores


def topk_rescore_workspace_size(rows, width, k):
    return int(_lib.csa2_topk_rescore_workspace_size(int(rows), int(width), int(k)))


def topk_rescore_supported(rows, width, k, heads=64, dim=128, fp8=True, fp4=False, shared_plane=False):
    """Whether the score-free FULL path (indexer_score(scores=None) + topk_rescore) takes these sizes:
    FP8-E4M3 or MXFP4 index planes (wide rows), or a BF16 plane whose rows share it (``shared_plane``,
    a prefill chunk; ``fp8`` and ``fp4`` False)."""
    if heads != 64 or dim != 128 or not 1 <= k <= 2048 or rows < 1:
        return False
    if not (fp8 or fp4):
        return bool(shared_plane) and width < (1 << 31)
    return topk_rescore_workspace_size(rows, width, k) > 0 and _quant_rescore_plan(rows, width)


def _quant_rescore_plan(rows, width):
    # the wide-row plan the quantised planes' select uses: fewer than 1024 rows, 8192 <= width < 2^24
    return rows < 1024 and 8192 <= width < (1 << 24)


def topk_rescore(q, w, k, row_base, pos, ratio, scale, out, block_keys, width, *, k_scale=None,
                 fp4=False, q_scale=None, dense=False, shared_plane=False, workspace=None, stream=None):
    """Top-k ``out`` [rows, k] int32 of the scores a score-free indexer_score call with these arguments kept on
    chip (its ``block_keys``); bit-identical to topk_select over the written scores.  FP8 index planes by
    default, MXFP4 ones with ``fp4=True`` (and ``q_scale``, as for indexer_score), BF16 ones with
    ``dense=True`` and ``shared_plane=True`` (rows of one prefill chunk)."""
    _dev(out)
    _need(out, torch.int32, "out")
    a = _index_args(q, w, k, row_base, pos, ratio, scale, None, width, k_scale, None, 8, not (fp4 or dense), None,
                    None, block_keys, fp4, q_scale)
    a.flags |= INDEX_SHARED_PLANE if shared_plane else 0
    if out.shape[0] != a.rows:
        raise ValueError("csa2.topk_rescore: out rows")
    need = topk_rescore_workspace_size(a.rows, a.width, out.shape[1])
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _scratch(need, out.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("csa2_topk_rescore", _lib.csa2_topk_rescore(ctypes.byref(a), out.shape[1], _ptr(out), _ptr(workspace),
                                                       ws_bytes, _stream(stream)))
    return out


def topk_workspace_size(rows, width, k):
    return int(_lib.csa2_topk_workspace_size(int(rows), int(width), int(k)))


def topk_uses_key_hist(rows, width, k=512):
    """Whether topk_select takes its wide-row path for this shape (the one that reads ``key_hist``)."""
    return topk_workspace_size(rows, width, k) > 0


def topk_select(scores, pos, ratio, out, *, cand=None, block_rows=8, key_hist=None, workspace=None, stream=None):
    """Fills ``out`` [rows, k] int32 with the selected plane rows (ascending, -1 padded).

    ``key_hist`` is the histogram indexer_score wrote for these scores, if any.
    """
    _dev(workspace)
    a = _topk_args(scores, pos, ratio, out, cand, block_rows, key_hist)
    rows, width = a.rows, a.width
    need = topk_workspace_size(rows, width, a.k)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _scratch(need, scores.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("csa2_topk_select", _lib.csa2_topk_select(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def _topk_args(scores, pos, ratio, out, cand, block_rows, key_hist):
    _dev(scores, pos, out, cand, key_hist)
    _need(scores, torch.float32, "scores")
    _need(pos, torch.int64, "pos")
    _need(out, torch.int32, "out")
    rows, width = scores.shape
    if out.shape[0] != rows or pos.shape != (rows,):
        raise ValueError("csa2.topk_select: inconsistent shapes")
    a = TopkArgs()
    a.struct_size = ctypes.sizeof(TopkArgs)
    a.rows, a.k, a.ratio, a.width = rows, out.shape[1], int(ratio), width
    if cand is not None:
        _need(cand, torch.int32, "cand")
        a.n_blocks, a.block_rows = cand.shape[1], int(block_rows)
    a.scores, a.pos, a.cand, a.out = _ptr(scores), _ptr(pos), _ptr(cand), _ptr(out)
    a.key_hist = _ptr(key_hist)
    return a


NOALLOC_SCRATCH_BYTES = int(_lib.csa2_topk_noalloc_scratch_bytes())


def topk_select_noalloc(scores, pos, ratio, out, *, cand=None, block_rows=8, key_hist=None, stream=None):
    """topk_select without any allocation: the library's fixed per-GPU scratch array is the workspace
    (for callers that cannot allocate).  Calls that overlap on one GPU race on that array."""
    a = _topk_args(scores, pos, ratio, out, cand, block_rows, key_hist)
    _check("csa2_topk_select_noalloc", _lib.csa2_topk_select_noalloc(ctypes.byref(a), _stream(stream)))
    return out


def candidate_pool_workspace_size(rows, width, block_rows=8, n_cand=2048):
    return int(_lib.csa2_candidate_pool_workspace_size(int(rows), int(width), int(block_rows), int(n_cand)))


def candidate_pool(pos, ratio, cand, *, scores=None, block_max=None, block_keys=None, width=None, block_rows=8,
                   workspace=None, stream=None):
    """Fills ``cand`` [rows, n_cand] int32 with the FULL layer's candidate blocks (ascending, -1 padded).

    Block scores come from ``block_keys`` (int32 [rows, ceil(width / 8)] from a
    score-free indexer_score) or ``block_max`` (written by indexer_score) when
    given, else from ``scores`` [rows, width].  ``width`` is the FULL score
    width (taken from ``scores`` when omitted).
    """
    _dev(pos, cand, scores, block_max, block_keys, workspace)
    _need(pos, torch.int64, "pos")
    _need(cand, torch.int32, "cand")
    rows = cand.shape[0]
    if width is None:
        if scores is None:
            raise ValueError("csa2.candidate_pool: width is needed when scores is not given")
        width = scores.shape[1]
    if scores is not None:
        _need(scores, torch.float32, "scores")
        if tuple(scores.shape) != (rows, width):
            raise ValueError("csa2.candidate_pool: scores must be [rows, width]")
    if block_max is not None:
        _need(block_max, torch.float32, "block_max")
        if tuple(block_max.shape) != (rows, -(-int(width) // int(block_rows))):
            raise ValueError("csa2.candidate_pool: block_max must be [rows, ceil(width / block_rows)]")
    if block_keys is not None:
        _need(block_keys, torch.int32, "block_keys")
        if tuple(block_keys.shape) != (rows, -(-int(width) // 8)):
            raise ValueError("csa2.candidate_pool: block_keys must be [rows, ceil(width / 8)]")
    if pos.shape != (rows,):
        raise ValueError("csa2.candidate_pool: pos must be [rows]")
    a = PoolArgs()
    a.struct_size = ctypes.sizeof(PoolArgs)
    a.rows, a.ratio, a.block_rows, a.n_cand, a.width = rows, int(ratio), int(block_rows), cand.shape[1], int(width)
    a.scores, a.block_max, a.pos, a.cand = _ptr(scores), _ptr(block_max), _ptr(pos), _ptr(cand)
    a.block_keys = _ptr(block_keys)
    need = candidate_pool_workspace_size(rows, width, block_rows, a.n_cand)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _scratch(need, pos.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("csa2_candidate_pool", _lib.csa2_candidate_pool(ctypes.byref(a), _ptr(workspace), ws_bytes,
                                                           _stream(stream)))
    return cand


def _attn_args(q, pos, idx, kv, kv_scale, kv_row_base, swa, swa_scale, sink, inv_freq, ratio, window,
               softmax_scale, out, rope_dim, kv_fp4, swa_fp8, kv_nvfp4=False, swa_fp8mx=False):
    _dev(q, pos, idx, kv, kv_scale, kv_row_base, swa, swa_scale, sink, inv_freq, out)
    rows, heads, dim = q.shape
    _need(pos, torch.int64, "pos")
    _need(idx, torch.int32, "idx")
    _need(sink, torch.float32, "sink")
    _need(inv_freq, torch.float64, "rope_inv_freq")
    _need(kv_row_base, torch.int64, "kv_row_base")
    if kv_fp4:
        _need(kv, torch.uint8, "kv")
        _need(kv_scale, torch.uint8, "kv_scale")
    if swa_fp8:
        _need(swa, torch.uint8, "swa")
        _need(swa_scale, torch.float32, "swa_scale")
    if kv_nvfp4 or swa_fp8mx:
        # rows with inline scales: E2M1 + E4M3 per 16 (dim/2 + dim/16 bytes) and
        # FP8 + E8M0 per 32 (dim + dim/32 bytes); the two go together
        if not (kv_nvfp4 and swa_fp8mx) or kv_fp4 or swa_fp8 or kv_scale is not None or swa_scale is not None:
            raise ValueError("csa2.sparse_attn: kv_nvfp4 goes with swa_fp8mx, without separate scales")
        _need(kv, torch.uint8, "kv")
        _need(swa, torch.uint8, "swa")
        if kv.shape[-1] != dim // 2 + dim // 16:
            raise ValueError(f"csa2.sparse_attn: kv rows must be {dim // 2 + dim // 16} bytes")
    if out.shape != q.shape or idx.shape[0] != rows or pos.shape != (rows,) or sink.shape != (heads,) \
            or inv_freq.shape != (rope_dim // 2,) or kv_row_base.shape != (rows,):
        raise ValueError("csa2.sparse_attn: inconsistent shapes")
    a = AttnArgs()
    a.struct_size = ctypes.sizeof(AttnArgs)
    a.rows, a.heads, a.dim, a.rope_dim, a.topk = rows, heads, dim, int(rope_dim), idx.shape[1]
    a.ratio, a.window = int(ratio), int(window)
    a.q_dtype, a.out_dtype = _dense_code(q, "q"), _dense_code(out, "out")
    a.kv_dtype = FP4_E2M1 if kv_fp4 else FP4_E2M1_E4M3G16 if kv_nvfp4 else _dense_code(kv, "kv")
    a.swa_dtype = FP8_E4M3 if swa_fp8 else FP8_E4M3_E8M0G32 if swa_fp8mx else _dense_code(swa, "swa")
    a.q, a.pos, a.idx, a.kv, a.kv_scale = _ptr(q), _ptr(pos), _ptr(idx), _ptr(kv), _ptr(kv_scale)
    a.kv_row_base, a.swa, a.swa_scale, a.sink = _ptr(kv_row_base), _ptr(swa), _ptr(swa_scale), _ptr(sink)
    a.rope_inv_freq, a.softmax_scale, a.out = _ptr(inv_freq), float(softmax_scale), _ptr(out)
    return a


def attn_workspace_size(rows, heads, dim, window, topk, splits=0):
    return int(_lib.csa2_attn_workspace_size(int(rows), int(heads), int(dim), int(window), int(topk), int(splits)))


def _swa_row_len(dim, swa_fp8mx):
    return dim + dim // 32 if swa_fp8mx else dim


def sparse_attn_decode(q, pos, idx, kv, kv_row_base, swa, sink, inv_freq, ratio, window, softmax_scale, out, *,
                       rope_dim=64, kv_scale=None, swa_scale=None, kv_fp4=False, swa_fp8=False, kv_nvfp4=False,
                       swa_fp8mx=False, splits=0, workspace=None, stream=None):
    """Decode attention: ``swa`` is one ring [rows, window, D] per query row.

    ``kv_nvfp4`` with ``swa_fp8mx`` selects rows with inline scales: kv
    [*, D/2 + D/16] bytes (E2M1, then one E4M3 per 16) and swa
    [rows, window, D + D/32] bytes (FP8-E4M3, then one E8M0 per 32).
    ``splits`` (0 = the library's choice) splits few rows' entries over workgroups; the
    workspace for their partial states is allocated here unless given."""
    _dev(workspace)
    a = _attn_args(q, pos, idx, kv, kv_scale, kv_row_base, swa, swa_scale, sink, inv_freq, ratio, window,
                   softmax_scale, out, rope_dim, kv_fp4, swa_fp8, kv_nvfp4, swa_fp8mx)
    if tuple(swa.shape) != (a.rows, a.window, _swa_row_len(a.dim, swa_fp8mx)):
        raise ValueError("csa2.sparse_attn_decode: swa must be [rows, window, dim]")
    if swa_fp8 and tuple(swa_scale.shape) != (a.rows, a.window):
        raise ValueError("csa2.sparse_attn_decode: swa_scale must be [rows, window]")
    a.splits = int(splits)
    need = attn_workspace_size(a.rows, a.heads, a.dim, a.window, a.topk, a.splits)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("csa2_sparse_attn_decode", _lib.csa2_sparse_attn_decode(ctypes.byref(a), _ptr(workspace), ws_bytes,
                                                                   _stream(stream)))
    return out


def sparse_attn_prefill(q, pos, idx, kv, swa, swa_pos0, sink, inv_freq, ratio, window, softmax_scale, out, *,
                        rope_dim=64, kv_row_base=None, kv_scale=None, swa_scale=None, kv_fp4=False, swa_fp8=False,
                        kv_nvfp4=False, swa_fp8mx=False, stream=None):
    """Prefill attention: ``swa`` is one linear array [swa_rows, D]; row t holds position swa_pos0 + t.
    Storage flags as for sparse_attn_decode."""
    if kv_row_base is None:
        kv_row_base = torch.zeros(q.shape[0], dtype=torch.int64, device=q.device)
    a = _attn_args(q, pos, idx, kv, kv_scale, kv_row_base, swa, swa_scale, sink, inv_freq, ratio, window,
                   softmax_scale, out, rope_dim, kv_fp4, swa_fp8, kv_nvfp4, swa_fp8mx)
    if swa.dim() != 2 or swa.shape[1] != _swa_row_len(a.dim, swa_fp8mx) or \
            (swa_fp8 and tuple(swa_scale.shape) != (swa.shape[0],)):
        raise ValueError("csa2.sparse_attn_prefill: swa must be [swa_rows, dim] (and swa_scale [swa_rows])")
    a.swa_rows, a.swa_pos0 = swa.shape[0], int(swa_pos0)
    _check("csa2_sparse_attn_prefill", _lib.csa2_sparse_attn_prefill(ctypes.byref(a), _stream(stream)))
    return out


# Plane formats of csa2_compress, by name: main rows and index keys.
_MAIN_FORMATS = {"f32": F32, "bf16": BF16, "fp4": FP4_E2M1, "nvfp4": FP4_E2M1_E4M3G16}
_IDX_FORMATS = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp4": FP4_E2M1}


def compress_workspace_size(rows, d_in, ratio):
    return int(_lib.csa2_compress_workspace_size(int(rows), int(d_in), int(ratio)))


def compress(x, pos, slot, row_base, wkv, norm_w, wk, knorm_w, inv_freq, main_out, idx_out, *, ratio, wgate=None,
             eps=1e-6, k_eps=1e-6, tail_kv=None, tail_score=None, main_format="bf16", idx_format="fp8",
             main_scale=None, idx_scale=None, workspace=None, stream=None):
    """The FULL layer's write path (csa2_compress): pools the token rows x [R, d_in] (bf16) into latent
    rows, writes the rotated main rows into ``main_out`` and the index keys into ``idx_out`` at plane row
    row_base[r] + pos[r] // ratio for each row r that completes a group.

    Weights: wkv / wgate [512, d_in] bf16, wk [128, 512] bf16, norm_w [512] and knorm_w [128] float32;
    inv_freq: the float64 rope table on the device.  Ratio 2 needs wgate and the tail state
    tail_kv / tail_score [slots, 512] float32 (rows of sequence s use slot[r] = s).
    main_format: "f32" | "bf16" | "fp4" (with main_scale, E8M0 [*, 16]) | "nvfp4" (288-byte rows);
    idx_format: "f32" | "bf16" | "fp8" (with idx_scale, float32 [*]) | "fp4" (with idx_scale, E8M0 [*, 4]).
    """
    _dev(x, pos, slot, row_base, wkv, wgate, norm_w, wk, knorm_w, inv_freq, main_out, idx_out, tail_kv, tail_score,
         main_scale, idx_scale, workspace)
    _need(x, torch.bfloat16, "x")
    _need(wkv, torch.bfloat16, "wkv")
    _need(wk, torch.bfloat16, "wk")
    _need(norm_w, torch.float32, "norm_w")
    _need(knorm_w, torch.float32, "knorm_w")
    _need(inv_freq, torch.float64, "rope_inv_freq")
    _need(pos, torch.int64, "pos")
    _need(slot, torch.int32, "slot")
    _need(row_base, torch.int64, "row_base")
    if wgate is not None:
        _need(wgate, torch.bfloat16, "wgate")
    for t, n in ((tail_kv, "tail_kv"), (tail_score, "tail_score")):
        if t is not None:
            _need(t, torch.float32, n)
            if t.dim() != 2 or t.shape[1] != 512:
                raise ValueError(f"csa2.compress: {n} must be [slots, 512]")
    rows, d_in = x.shape
    if pos.shape != (rows,) or slot.shape != (rows,) or row_base.shape != (rows,) or wkv.shape != (512, d_in) \
            or (wgate is not None and wgate.shape != (512, d_in)) or wk.shape != (128, 512):
        raise ValueError("csa2.compress: inconsistent shapes")
    if main_format not in _MAIN_FORMATS or idx_format not in _IDX_FORMATS:
        raise ValueError("csa2.compress: unknown plane format")
    a = CompressArgs()
    a.struct_size = ctypes.sizeof(CompressArgs)
    a.rows, a.d_in, a.ratio, a.dim, a.idx_dim, a.rope_dim = rows, d_in, int(ratio), 512, 128, 64
    a.main_dtype, a.idx_dtype = _MAIN_FORMATS[main_format], _IDX_FORMATS[idx_format]
    a.x, a.pos, a.slot, a.row_base = _ptr(x), _ptr(pos), _ptr(slot), _ptr(row_base)
    a.wkv, a.wgate, a.norm_w, a.wk, a.knorm_w = _ptr(wkv), _ptr(wgate), _ptr(norm_w), _ptr(wk), _ptr(knorm_w)
    a.rope_inv_freq, a.eps, a.k_eps = _ptr(inv_freq), float(eps), float(k_eps)
    a.tail_kv, a.tail_score = _ptr(tail_kv), _ptr(tail_score)
    a.main_out, a.main_scale_out, a.idx_out, a.idx_scale_out = _ptr(main_out), _ptr(main_scale), _ptr(idx_out), \
        _ptr(idx_scale)
    need = compress_workspace_size(rows, d_in, ratio)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _scratch(need, x.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("csa2_compress", _lib.csa2_compress(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream)))


class Prepared:
    """A C ABI call with its arguments marshalled once: ``call()`` only crosses into the library.

    The tensors used to build it must stay alive and unchanged in shape while it is used.
    """

    def __init__(self, fn_name, fn, args, stream):
        self.fn_name, self._fn, self._args, self._stream = fn_name, fn, args, stream

    def __call__(self):
        _check(self.fn_name, self._fn(*self._args, self._stream))


def _prepare(fn_name, call, stream):
    """Runs ``call`` once with a recording stub to capture the marshalled arguments."""
    captured = {}
    real = getattr(_lib, fn_name)

    def stub(*a):
        captured["args"] = a[:-1]
        return OK

    setattr(_lib, fn_name, stub)
    try:
        call()
    finally:
        setattr(_lib, fn_name, real)
    return Prepared(fn_name, real, captured["args"], _stream(stream))


def prepare_indexer_score(*args, stream=None, **kw):
    return _prepare("csa2_indexer_score", lambda: indexer_score(*args, stream=stream, **kw), stream)


def prepare_topk_select(*args, stream=None, **kw):
    if "workspace" not in kw or kw["workspace"] is None:
        scores, out = args[0], args[3]
        need = topk_workspace_size(scores.shape[0], scores.shape[1], out.shape[1])
        kw["workspace"] = torch.empty(max(need, 1), dtype=torch.uint8, device=scores.device)
    p = _prepare("csa2_topk_select", lambda: topk_select(*args, stream=stream, **kw), stream)
    p.workspace = kw["workspace"]
    return p


def prepare_sparse_attn_decode(*args, stream=None, **kw):
    if kw.get("workspace") is None:
        q, idx, swa = args[0], args[2], args[5]
        need = attn_workspace_size(q.shape[0], q.shape[1], q.shape[2], args[9], idx.shape[1], kw.get("splits", 0))
        kw["workspace"] = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    p = _prepare("csa2_sparse_attn_decode", lambda: sparse_attn_decode(*args, stream=stream, **kw), stream)
    p.workspace = kw["workspace"]
    return p


def prepare_sparse_attn_prefill(*args, stream=None, **kw):
    return _prepare("csa2_sparse_attn_prefill", lambda: sparse_attn_prefill(*args, stream=stream, **kw), stream)


def prepare_candidate_pool(*args, stream=None, **kw):
    if kw.get("workspace") is None:
        pos, cand = args[0], args[2]
        width = kw["scores"].shape[1] if kw.get("scores") is not None else kw["width"]
        need = candidate_pool_workspace_size(cand.shape[0], width, kw.get("block_rows", 8), cand.shape[1])
        kw["workspace"] = torch.empty(max(need, 1), dtype=torch.uint8, device=pos.device)
    p = _prepare("csa2_candidate_pool", lambda: candidate_pool(*args, stream=stream, **kw), stream)
    p.workspace = kw["workspace"]
    return p


def prepare_compress(x, *args, stream=None, **kw):
    if kw.get("workspace") is None:
        need = compress_workspace_size(x.shape[0], x.shape[1], kw["ratio"])
        kw["workspace"] = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    p = _prepare("csa2_compress", lambda: compress(x, *args, stream=stream, **kw), stream)
    p.workspace = kw["workspace"]
    return p


def prepare_topk_rescore(*args, stream=None, **kw):
    if kw.get("workspace") is None:
        out, width = args[7], args[9]
        need = topk_rescore_workspace_size(out.shape[0], width, out.shape[1])
        kw["workspace"] = torch.empty(max(need, 1), dtype=torch.uint8, device=out.device)
    p = _prepare("csa2_topk_rescore", lambda: topk_rescore(*args, stream=stream, **kw), stream)
    p.workspace = kw["workspace"]
    return p

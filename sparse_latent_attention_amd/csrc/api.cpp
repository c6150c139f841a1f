// C ABI entry points: host-side validation, launch-shape choice and dispatch.
// Every check runs before any HIP call; a rejected call launches nothing.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/csa2.h"
#include "kernels.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Rows per pooled block of the candidate pool: a power of two in 4..64.
bool pool_block_ok(int32_t b) { return b >= 4 && b <= 64 && (b & (b - 1)) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t elem_bytes(int dtype) {
    switch (dtype) {
        case CSA2_F32: return 4;
        case CSA2_BF16: return 2;
        case CSA2_FP8_E4M3: return 1;
        case CSA2_FP4_E2M1: return 1;  // two elements per byte; rows are dim / 2 bytes
        default: return 0;
    }
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

// Scale operands match the element type: FP8 takes k_scale, MXFP4 takes both
// E8M0 planes, the other types take none.
bool index_scales_ok(const csa2_index_args* a) {
    const bool fp8 = a->k_dtype == CSA2_FP8_E4M3, fp4 = a->k_dtype == CSA2_FP4_E2M1;
    return fp8 == (a->k_scale != nullptr) && fp4 == (a->q_scale_e8m0 != nullptr) &&
           fp4 == (a->k_scale_e8m0 != nullptr) && aligned(a->k_scale_e8m0, 4);
}


// Score-free mode over a BF16 plane: rows that share one plane (a prefill chunk), 64 x 128.
bool dense_score_free(const csa2_index_args* a) {
    return a->k_dtype == CSA2_BF16 && a->q_dtype == CSA2_BF16 && a->heads == 64 && a->dim == 128 &&
           (a->flags & CSA2_INDEX_SHARED_PLANE) != 0 && a->width < (1LL << 31);
}

// Workspace of the BF16 score-free select: the chosen blocks [rows, k], their re-computed scores
// [rows, 8 k], and the larger of the two selects' own workspaces.
size_t dense_rescore_bytes(int32_t rows, int64_t width, int32_t k) {
    if (rows <= 0 || width <= 0 || width >= (1LL << 31) || k < 1 || k > 2048) return 0;
    const int64_t nbk = (width + 7) / 8;
    const size_t t1 = csa2::topk_workspace_bytes(rows, nbk), t2 = csa2::topk_workspace_bytes(rows, 8 * (int64_t)k);
    return align256((size_t)rows * k * 4) + align256((size_t)rows * 8 * k * 4) + align256(t1 > t2 ? t1 : t2);
}

}  // namespace

extern "C" {

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char* csa2_status_string(int32_t status) {
    switch (status) {
        case CSA2_OK: return "ok";
        case CSA2_ERR_INVALID_ARG: return "invalid argument";
        case CSA2_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
        case CSA2_ERR_WORKSPACE: return "workspace too small";
        case CSA2_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int32_t csa2_rope_inv_freq(int32_t rope_dim, double theta, double yarn_factor, int64_t yarn_orig_len, double* out) {
    if (out == nullptr || rope_dim <= 0 || (rope_dim % 2) != 0 || !(theta > 1.0) || !(yarn_factor >= 1.0))
        return CSA2_ERR_INVALID_ARG;
    const double two_pi = 6.283185307179586476925286766559;
    for (int32_t i = 0; i < rope_dim / 2; ++i) {
        const double f = pow(theta, -2.0 * (double)i / (double)rope_dim);
        double fi = f;
        if (yarn_factor > 1.0 && yarn_orig_len > 0) {
            // turns this frequency makes within the original context length
            const double turns = (double)yarn_orig_len * f / two_pi;
            double gamma = (turns - 1.0) / (32.0 - 1.0);
            gamma = gamma < 0.0 ? 0.0 : (gamma > 1.0 ? 1.0 : gamma);
            fi = (1.0 - gamma) * f / yarn_factor + gamma * f;
        }
        out[i] = fi;
    }
    return CSA2_OK;
}

int32_t csa2_indexer_score(const csa2_index_args* a, csa2_stream_t stream) {
    if (a == nullptr || a->struct_size < sizeof(csa2_index_args)) return CSA2_ERR_INVALID_ARG;
    if (a->mode != CSA2_MODE_FULL && a->mode != CSA2_MODE_REINDEX) return CSA2_ERR_INVALID_ARG;
    if (a->rows < 0 || a->rows > 65535 || a->width < 0 || (a->ratio != 1 && a->ratio != 2)) return CSA2_ERR_INVALID_ARG;
    if (a->q_dtype != a->k_dtype || elem_bytes(a->k_dtype) == 0) return CSA2_ERR_UNSUPPORTED;
    if (!csa2::indexer_supported(a->heads, a->dim, a->k_dtype)) return CSA2_ERR_UNSUPPORTED;
    const bool reindex = a->mode == CSA2_MODE_REINDEX;
    if ((a->flags & ~(CSA2_INDEX_SHARED_PLANE | CSA2_INDEX_BLOCK_KEYS16)) != 0 || (reindex && a->flags != 0))
        return CSA2_ERR_INVALID_ARG;
    const bool bk16 = (a->flags & CSA2_INDEX_BLOCK_KEYS16) != 0;
    if (a->k_dtype == CSA2_FP4_E2M1 && reindex && a->block_rows != 8) return CSA2_ERR_UNSUPPORTED;
    if (reindex) {
        if (a->cand == nullptr || a->n_blocks <= 0 || a->block_rows <= 0 || a->block_rows > 64) return CSA2_ERR_INVALID_ARG;
        if (a->width != (int64_t)a->n_blocks * a->block_rows) return CSA2_ERR_INVALID_ARG;
        if (a->block_max != nullptr) return CSA2_ERR_INVALID_ARG;
    } else if (a->block_max != nullptr && !pool_block_ok(a->block_rows)) {
        return CSA2_ERR_INVALID_ARG;
    }
    // Nothing to compute (an empty output may come with a null pointer, which would
    // otherwise read as score-free mode).
    if (a->rows == 0 || a->width == 0) return CSA2_OK;
    // Score-free mode: FULL rows of a quantised plane keep their scores on chip and
    // leave the block keys for csa2_topk_rescore.
    const bool score_free = a->scores == nullptr;
    if (a->block_keys != nullptr && !score_free) return CSA2_ERR_INVALID_ARG;
    if (score_free) {
        if (reindex || a->key_hist != nullptr || a->block_keys == nullptr) return CSA2_ERR_INVALID_ARG;
        if (!csa2::indexer_rescore_supported(a->heads, a->dim, a->k_dtype) && !dense_score_free(a))
            return CSA2_ERR_UNSUPPORTED;
        if (a->width >= (1LL << 24) && !dense_score_free(a)) return CSA2_ERR_UNSUPPORTED;
        if (!aligned(a->block_keys, 4)) return CSA2_ERR_INVALID_ARG;
        if (bk16 && dense_score_free(a)) return CSA2_ERR_INVALID_ARG;  // that route ranks full keys
    } else if (bk16) {
        return CSA2_ERR_INVALID_ARG;  // 16-bit block keys exist in score-free mode only
    }
    if (a->q == nullptr || a->w == nullptr || a->k == nullptr || a->row_base == nullptr || a->pos == nullptr)
        return CSA2_ERR_INVALID_ARG;
    if (!index_scales_ok(a)) return CSA2_ERR_INVALID_ARG;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->scores, 4) || !aligned(a->w, 4) ||
        !aligned(a->block_max, 4))
        return CSA2_ERR_INVALID_ARG;
    if (!isfinite(a->scale)) return CSA2_ERR_INVALID_ARG;

    csa2::IndexParams p;
    p.q = a->q; p.w = a->w; p.k = a->k; p.k_scale = a->k_scale; p.row_base = a->row_base; p.pos = a->pos;
    p.q_e8 = a->q_scale_e8m0; p.k_e8 = a->k_scale_e8m0;
    p.cand = reindex ? a->cand : nullptr; p.scores = a->scores; p.key_hist = a->key_hist; p.width = a->width;
    p.n_blocks = reindex ? a->n_blocks : 0; p.block_rows = reindex ? a->block_rows : 1; p.ratio = a->ratio;
    p.scale = a->scale;
    p.shared_plane = (a->flags & CSA2_INDEX_SHARED_PLANE) != 0;
    p.bk16 = bk16;
    p.block_max = reindex ? nullptr : a->block_max;
    p.block_keys = score_free ? a->block_keys : nullptr;
    p.bm_rows = p.block_max != nullptr ? a->block_rows : 4;
    p.bm_blocks = (a->width + p.bm_rows - 1) / p.bm_rows;
    // Columns per workgroup: multiples of 256 (4 waves x 64), aiming at ~4096 workgroups.
    const int64_t work = a->width * (int64_t)a->rows;
    int64_t per = (work + 256LL * 4096 - 1) / (256LL * 4096);
    if (per < 4) per = 4;
    if (per > 16) per = 16;
    // FULL FP8 planes (132-byte key rows incl. scale): 2048 columns per workgroup, about the bytes a
    // 4096-column MXFP4 workgroup reads; at 1M x 64 this shortened the grid's last partial round
    // (1.296 -> 1.288 ms), while MXFP4 planes were fastest at 4096.
    if (!reindex && a->k_dtype == CSA2_FP8_E4M3 && per > 8) per = 8;
    const int64_t need = (a->width + 255) / 256;
    if (per > need) per = need;
    p.cols_per_wg = 256 * per;
    return hip_status(csa2::launch_indexer_score(p, a->rows, a->heads, a->dim, a->k_dtype, reindex,
                                                 reinterpret_cast<hipStream_t>(stream)));
}

// Wide-row plan of the score-free select, or nseg == 0 if these sizes have none.
static void rescore_plan(int32_t rows, int64_t width, int& chunk, int& nseg) {
    chunk = nseg = 0;
    if (rows <= 0 || width <= 0 || width >= (1LL << 24)) return;
    csa2::topk_plan(rows, width, chunk, nseg, 4096);
}

// Workspace of the quantised-plane score-free select (0: these sizes have no plan).
static size_t quant_rescore_bytes(int32_t rows, int64_t width) {
    int chunk, nseg;
    rescore_plan(rows, width, chunk, nseg);
    if (nseg == 0) return 0;
    const size_t lists = (size_t)rows * nseg * chunk;
    const size_t parts = (size_t)csa2::block_key_hist_parts((width + 7) / 8);
    return align256((size_t)rows * 4) + align256((size_t)rows * nseg * 4) + 2 * align256(lists * 4) +
           align256((size_t)rows * parts * 4096 * 4);
}

size_t csa2_topk_rescore_workspace_size(int32_t rows, int64_t width, int32_t k) {
    const size_t a = quant_rescore_bytes(rows, width), b = dense_rescore_bytes(rows, width, k);
    return a > b ? a : b;
}

// BF16 plane: the k best 8-column blocks by block key (ties to the lower block), re-scored with the FULL
// pass's arithmetic through the REINDEX kernel, then the exact select over their columns.  The top-k of
// the row lies in those blocks: a column with one of the k largest scores has a score >= T, the k-th
// largest block key, so its block's key is >= T; every block with a key > T is chosen, and if the k-th
// largest score equals T, the lowest-numbered columns with score T lie in the lowest-numbered blocks with
// key T (each such block holds at least one), of which the k - #(keys > T) lowest are chosen.
static int32_t dense_rescore(const csa2_index_args* a, int32_t k, int32_t* out, void* workspace, hipStream_t st) {
    const int rows = a->rows;
    const int64_t nbk = (a->width + 7) / 8;
    char* w = static_cast<char*>(workspace);
    int32_t* cand = reinterpret_cast<int32_t*>(w);
    w += align256((size_t)rows * k * 4);
    float* sc = reinterpret_cast<float*>(w);
    w += align256((size_t)rows * 8 * k * 4);
    void* tws = w;

    csa2::TopkParams bp;  // best k blocks
    bp.scores = nullptr; bp.pos = a->pos; bp.cand = nullptr; bp.out = cand; bp.key_hist = nullptr;
    bp.width = nbk; bp.k = k; bp.ratio = a->ratio; bp.n_blocks = 0; bp.block_rows = 1; bp.col_group = 8;
    bp.pool_keys = a->block_keys; bp.plain_keys = true;
    hipError_t e = csa2::launch_topk_select(bp, rows, tws, st);

    csa2::IndexParams ip;  // their columns, re-scored
    ip.q = a->q; ip.w = a->w; ip.k = a->k; ip.k_scale = nullptr; ip.row_base = a->row_base; ip.pos = a->pos;
    ip.q_e8 = nullptr; ip.k_e8 = nullptr; ip.cand = cand; ip.scores = sc; ip.key_hist = nullptr;
    ip.block_max = nullptr; ip.block_keys = nullptr; ip.width = 8 * (int64_t)k; ip.cols_per_wg = 0;
    ip.bm_blocks = 0; ip.n_blocks = k; ip.block_rows = 8; ip.bm_rows = 4; ip.ratio = a->ratio; ip.scale = a->scale;
    ip.shared_plane = false; ip.bk16 = false;
    if (e == hipSuccess) e = csa2::launch_indexer_score(ip, rows, 64, 128, CSA2_BF16, true, st);

    csa2::TopkParams fp;  // the exact select over them
    fp.scores = sc; fp.pos = a->pos; fp.cand = cand; fp.out = out; fp.key_hist = nullptr;
    fp.width = 8 * (int64_t)k; fp.k = k; fp.ratio = a->ratio; fp.n_blocks = k; fp.block_rows = 8; fp.col_group = 1;
    fp.pool_keys = nullptr; fp.plain_keys = false;
    if (e == hipSuccess) e = csa2::launch_topk_select(fp, rows, tws, st);
    return hip_status(e);
}

int32_t csa2_topk_rescore(const csa2_index_args* a, int32_t k, int32_t* out, void* workspace, size_t workspace_bytes,
                          csa2_stream_t stream) {
    if (a == nullptr || a->struct_size < sizeof(csa2_index_args)) return CSA2_ERR_INVALID_ARG;
    if (a->mode != CSA2_MODE_FULL || a->rows < 0 || a->width < 0 || (a->ratio != 1 && a->ratio != 2))
        return CSA2_ERR_INVALID_ARG;
    if (k < 1 || k > 2048 || (a->flags & ~(CSA2_INDEX_SHARED_PLANE | CSA2_INDEX_BLOCK_KEYS16)) != 0)
        return CSA2_ERR_INVALID_ARG;
    const bool dense = a->q_dtype == a->k_dtype && dense_score_free(a);
    const bool bk16 = (a->flags & CSA2_INDEX_BLOCK_KEYS16) != 0;
    if (bk16 && dense) return CSA2_ERR_INVALID_ARG;
    if (!dense && (a->q_dtype != a->k_dtype || !csa2::indexer_rescore_supported(a->heads, a->dim, a->k_dtype)))
        return CSA2_ERR_UNSUPPORTED;
    if (a->rows == 0) return CSA2_OK;
    int chunk = 0, nseg = 0;
    if (!dense) {
        rescore_plan(a->rows, a->width, chunk, nseg);
        if (nseg == 0) return CSA2_ERR_UNSUPPORTED;  // narrow rows: score, then csa2_topk_select
    }
    const size_t need = csa2_topk_rescore_workspace_size(a->rows, a->width, k);
    if (workspace_bytes < need) return CSA2_ERR_WORKSPACE;
    if (workspace == nullptr || !aligned(workspace, 256)) return CSA2_ERR_INVALID_ARG;
    if (a->q == nullptr || a->w == nullptr || a->k == nullptr || a->row_base == nullptr || a->pos == nullptr ||
        a->key_hist != nullptr || a->block_keys == nullptr || out == nullptr || !index_scales_ok(a))
        return CSA2_ERR_INVALID_ARG;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->w, 4) || !isfinite(a->scale))
        return CSA2_ERR_INVALID_ARG;
    if (dense) return dense_rescore(a, k, out, workspace, reinterpret_cast<hipStream_t>(stream));

    csa2::IndexParams ip;
    ip.q = a->q; ip.w = a->w; ip.k = a->k; ip.k_scale = a->k_scale; ip.row_base = a->row_base; ip.pos = a->pos;
    ip.q_e8 = a->q_scale_e8m0; ip.k_e8 = a->k_scale_e8m0;
    ip.cand = nullptr; ip.scores = nullptr; ip.key_hist = nullptr; ip.block_max = nullptr;
    ip.block_keys = a->block_keys; ip.width = a->width; ip.cols_per_wg = 0; ip.bm_blocks = 0; ip.n_blocks = 0;
    ip.block_rows = 1; ip.bm_rows = 4; ip.ratio = a->ratio; ip.scale = a->scale; ip.shared_plane = false;
    ip.bk16 = bk16;
    csa2::TopkParams tp;
    tp.scores = nullptr; tp.pos = a->pos; tp.cand = nullptr; tp.out = out; tp.key_hist = nullptr;
    tp.width = a->width; tp.k = k; tp.ratio = a->ratio; tp.n_blocks = 0; tp.block_rows = 1; tp.col_group = 1;
    tp.pool_keys = nullptr; tp.plain_keys = false;

    char* w = static_cast<char*>(workspace);
    uint32_t* b1 = reinterpret_cast<uint32_t*>(w);
    w += align256((size_t)a->rows * 4);
    uint32_t* seg_count = reinterpret_cast<uint32_t*>(w);
    w += align256((size_t)a->rows * nseg * 4);
    uint32_t* keys = reinterpret_cast<uint32_t*>(w);
    w += align256((size_t)a->rows * nseg * chunk * 4);
    int32_t* cols = reinterpret_cast<int32_t*>(w);
    w += align256((size_t)a->rows * nseg * chunk * 4);
    uint32_t* hist = reinterpret_cast<uint32_t*>(w);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = csa2::launch_block_key_hist(a->block_keys, bk16, (a->width + 7) / 8, a->rows, hist, st);
    if (e == hipSuccess)
        e = csa2::launch_topk_threshold(tp, a->rows, hist, csa2::block_key_hist_parts((a->width + 7) / 8), b1, st);
    if (e == hipSuccess)
        e = csa2::launch_indexer_rescore(ip, a->rows, a->k_dtype, b1, chunk, nseg, keys, cols, seg_count, st);
    if (e == hipSuccess) e = csa2::launch_topk_final(tp, a->rows, keys, cols, seg_count, nseg, chunk, st);
    return hip_status(e);
}

// Split of the projections' K range when rows are few (decode): enough
// workgroups to stream the weights, up to 16 splits (each adds a rows x nproj
// float32 partial tile that the finish kernel reads back), d_in / ksplit a
// multiple of 64.
static int compress_ksplit(int32_t rows, int32_t d_in, int32_t ratio) {
    const int64_t tiles = (int64_t)((rows + 63) / 64) * (ratio == 2 ? 16 : 8);
    int ks = 1;
    while (tiles * ks < 1024 && ks < 16 && (d_in / 64) % (2 * ks) == 0) ks *= 2;
    return ks;
}

size_t csa2_compress_workspace_size(int32_t rows, int32_t d_in, int32_t ratio) {
    if (rows <= 0 || d_in <= 0 || d_in % 64 != 0 || (ratio != 1 && ratio != 2)) return 0;
    return align256((size_t)compress_ksplit(rows, d_in, ratio) * rows * (ratio == 2 ? 1024 : 512) * 4);
}

int32_t csa2_compress(const csa2_compress_args* a, void* workspace, size_t workspace_bytes, csa2_stream_t stream) {
    if (a == nullptr || a->struct_size < sizeof(csa2_compress_args)) return CSA2_ERR_INVALID_ARG;
    if (a->rows < 0 || a->rows > (1 << 24) || a->d_in <= 0 || (a->ratio != 1 && a->ratio != 2))
        return CSA2_ERR_INVALID_ARG;
    if (a->dim != 512 || a->idx_dim != 128 || a->rope_dim != 64 || a->d_in % 64 != 0) return CSA2_ERR_UNSUPPORTED;
    if (!csa2::compress_supported(a->main_dtype, a->idx_dtype)) return CSA2_ERR_UNSUPPORTED;
    if (!(a->eps >= 0.f) || !(a->k_eps >= 0.f) || !isfinite(a->eps) || !isfinite(a->k_eps)) return CSA2_ERR_INVALID_ARG;
    const bool r2 = a->ratio == 2;
    if ((a->wgate != nullptr) != r2 || (a->tail_kv != nullptr) != r2 || (a->tail_score != nullptr) != r2)
        return CSA2_ERR_INVALID_ARG;
    const bool main_scale = a->main_dtype == CSA2_FP4_E2M1;
    const bool idx_scale = a->idx_dtype == CSA2_FP8_E4M3 || a->idx_dtype == CSA2_FP4_E2M1;
    if ((a->main_scale_out != nullptr) != main_scale || (a->idx_scale_out != nullptr) != idx_scale)
        return CSA2_ERR_INVALID_ARG;
    if (a->rows == 0) return CSA2_OK;
    const size_t need = csa2_compress_workspace_size(a->rows, a->d_in, a->ratio);
    if (workspace_bytes < need) return CSA2_ERR_WORKSPACE;
    if (workspace == nullptr || !aligned(workspace, 256)) return CSA2_ERR_INVALID_ARG;
    if (a->x == nullptr || a->pos == nullptr || a->slot == nullptr || a->row_base == nullptr || a->wkv == nullptr ||
        a->norm_w == nullptr || a->wk == nullptr || a->knorm_w == nullptr || a->rope_inv_freq == nullptr ||
        a->main_out == nullptr || a->idx_out == nullptr)
        return CSA2_ERR_INVALID_ARG;
    if (!aligned(a->x, 16) || !aligned(a->wkv, 16) || !aligned(a->wgate, 16) || !aligned(a->wk, 16) ||
        !aligned(a->main_out, 8) || !aligned(a->idx_out, 8) || !aligned(a->idx_scale_out, 4) ||
        !aligned(a->tail_kv, 8) || !aligned(a->tail_score, 8))
        return CSA2_ERR_INVALID_ARG;
    csa2::CompressParams p;
    p.x = static_cast<const uint16_t*>(a->x); p.pos = a->pos; p.slot = a->slot; p.row_base = a->row_base;
    p.wkv = static_cast<const uint16_t*>(a->wkv); p.wgate = static_cast<const uint16_t*>(a->wgate);
    p.norm_w = a->norm_w; p.wk = static_cast<const uint16_t*>(a->wk); p.knorm_w = a->knorm_w;
    p.inv_freq = a->rope_inv_freq; p.tail_kv = a->tail_kv; p.tail_score = a->tail_score;
    p.main_out = a->main_out; p.main_scale_out = a->main_scale_out; p.idx_out = a->idx_out;
    p.idx_scale_out = a->idx_scale_out; p.partial = static_cast<float*>(workspace);
    p.eps = a->eps; p.k_eps = a->k_eps; p.rows = a->rows; p.d_in = a->d_in; p.nproj = r2 ? 1024 : 512;
    p.ksplit = compress_ksplit(a->rows, a->d_in, a->ratio);
    return hip_status(csa2::launch_compress(p, a->ratio, a->main_dtype, a->idx_dtype,
                                            reinterpret_cast<hipStream_t>(stream)));
}

size_t csa2_topk_workspace_size(int32_t rows, int64_t width, int32_t k) {
    (void)k;
    if (rows <= 0 || width <= 0 || width >= (1LL << 31)) return 0;
    return csa2::topk_workspace_bytes(rows, width);
}

// Host-side checks of csa2_topk_select's arguments that do not involve the workspace.
static int32_t validate_topk(const csa2_topk_args* a) {
    if (a == nullptr || a->struct_size < sizeof(csa2_topk_args)) return CSA2_ERR_INVALID_ARG;
    if (a->rows < 0 || a->k < 1 || a->k > 2048 || a->width < 0 || a->width >= (1LL << 31)) return CSA2_ERR_INVALID_ARG;
    if (a->ratio != 1 && a->ratio != 2) return CSA2_ERR_INVALID_ARG;
    if (a->n_blocks < 0) return CSA2_ERR_INVALID_ARG;
    if (a->n_blocks > 0) {
        if (a->cand == nullptr || a->block_rows <= 0 || a->block_rows > 64) return CSA2_ERR_INVALID_ARG;
        if (a->width != (int64_t)a->n_blocks * a->block_rows) return CSA2_ERR_INVALID_ARG;
    }
    return CSA2_OK;
}

int32_t csa2_topk_select(const csa2_topk_args* a, void* workspace, size_t workspace_bytes, csa2_stream_t stream) {
    const int32_t st = validate_topk(a);
    if (st != CSA2_OK) return st;
    const size_t need = csa2_topk_workspace_size(a->rows, a->width, a->k);
    if (workspace_bytes < need) return CSA2_ERR_WORKSPACE;
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 256))) return CSA2_ERR_INVALID_ARG;
    if (a->rows == 0) return CSA2_OK;
    if (a->pos == nullptr || a->out == nullptr || (a->scores == nullptr && a->width > 0)) return CSA2_ERR_INVALID_ARG;
    csa2::TopkParams p;
    p.scores = a->scores; p.pos = a->pos; p.cand = a->n_blocks > 0 ? a->cand : nullptr; p.out = a->out;
    p.key_hist = a->key_hist;
    p.width = a->width; p.k = a->k; p.ratio = a->ratio; p.n_blocks = a->n_blocks;
    p.block_rows = a->n_blocks > 0 ? a->block_rows : 1;
    p.col_group = 1;
    p.pool_keys = nullptr; p.plain_keys = false;
    return hip_status(csa2::launch_topk_select(p, a->rows, workspace, reinterpret_cast<hipStream_t>(stream)));
}

size_t csa2_candidate_pool_workspace_size(int32_t rows, int64_t width, int32_t block_rows, int32_t n_cand) {
    (void)n_cand;
    if (rows <= 0 || width <= 0 || width >= (1LL << 31) || !pool_block_ok(block_rows)) return 0;
    const int64_t nb = (width + block_rows - 1) / block_rows;
    return align256((size_t)rows * (size_t)nb * sizeof(float)) + csa2::topk_workspace_bytes(rows, nb);
}

int32_t csa2_candidate_pool(const csa2_pool_args* a, void* workspace, size_t workspace_bytes, csa2_stream_t stream) {
    if (a == nullptr || a->struct_size < sizeof(csa2_pool_args)) return CSA2_ERR_INVALID_ARG;
    if (a->rows < 0 || a->n_cand < 1 || a->n_cand > 2048 || a->width < 0 || a->width >= (1LL << 31))
        return CSA2_ERR_INVALID_ARG;
    if ((a->ratio != 1 && a->ratio != 2) || !pool_block_ok(a->block_rows)) return CSA2_ERR_INVALID_ARG;
    const size_t need = csa2_candidate_pool_workspace_size(a->rows, a->width, a->block_rows, a->n_cand);
    if (workspace_bytes < need) return CSA2_ERR_WORKSPACE;
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 256))) return CSA2_ERR_INVALID_ARG;
    if (a->rows == 0) return CSA2_OK;
    if (a->pos == nullptr || a->cand == nullptr) return CSA2_ERR_INVALID_ARG;
    if (a->width > 0 && a->scores == nullptr && a->block_max == nullptr && a->block_keys == nullptr)
        return CSA2_ERR_INVALID_ARG;
    if (a->block_keys != nullptr && a->block_rows != 8) return CSA2_ERR_INVALID_ARG;
    if (!aligned(a->scores, 4) || !aligned(a->block_max, 4) || !aligned(a->block_keys, 4)) return CSA2_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t nb = (a->width + a->block_rows - 1) / a->block_rows;
    const float* bmax = a->block_max;
    char* ws = static_cast<char*>(workspace);
    if (a->block_keys == nullptr && bmax == nullptr && nb > 0) {
        float* buf = reinterpret_cast<float*>(ws);
        const hipError_t e = csa2::launch_block_max(a->scores, a->pos, a->ratio, a->width, a->block_rows, a->rows,
                                                    buf, st);
        if (e != hipSuccess) return CSA2_ERR_HIP;
        bmax = buf;
    }
    csa2::TopkParams p;
    p.scores = bmax; p.pos = a->pos; p.cand = nullptr; p.out = a->cand; p.key_hist = nullptr;
    p.width = nb; p.k = a->n_cand; p.ratio = a->ratio; p.n_blocks = 0; p.block_rows = 1;
    p.col_group = a->block_rows;
    p.pool_keys = a->block_keys; p.plain_keys = false;
    if (a->block_keys != nullptr) p.scores = nullptr;
    void* tws = need > 0 ? ws + align256((size_t)a->rows * (size_t)nb * sizeof(float)) : nullptr;
    return hip_status(csa2::launch_topk_select(p, a->rows, tws, st));
}

static int32_t validate_attn(const csa2_attn_args* a, bool decode) {
    if (a == nullptr || a->struct_size < sizeof(csa2_attn_args)) return CSA2_ERR_INVALID_ARG;
    if (a->rows < 0 || a->topk < 0 || a->topk > 2048 || a->window < 16 || a->window > 1024 || (a->window % 16) != 0 ||
        (a->topk % 16) != 0 || a->splits < 0 || a->splits > 8)
        return CSA2_ERR_INVALID_ARG;
    if (a->ratio != 1 && a->ratio != 2) return CSA2_ERR_INVALID_ARG;
    if (!(a->softmax_scale > 0.f) || !isfinite(a->softmax_scale)) return CSA2_ERR_INVALID_ARG;
    csa2::AttnShape s{a->heads, a->dim, a->rope_dim, a->q_dtype, a->kv_dtype, a->swa_dtype, a->out_dtype};
    if (!csa2::attn_supported(s)) return CSA2_ERR_UNSUPPORTED;
    if (a->rows == 0) return CSA2_OK;
    if (a->q == nullptr || a->pos == nullptr || a->kv == nullptr || a->kv_row_base == nullptr || a->swa == nullptr ||
        a->sink == nullptr || a->rope_inv_freq == nullptr || a->out == nullptr)
        return CSA2_ERR_INVALID_ARG;
    if (a->topk > 0 && a->idx == nullptr) return CSA2_ERR_INVALID_ARG;
    if ((a->kv_dtype == CSA2_FP4_E2M1) != (a->kv_scale != nullptr)) return CSA2_ERR_INVALID_ARG;
    if ((a->swa_dtype == CSA2_FP8_E4M3) != (a->swa_scale != nullptr)) return CSA2_ERR_INVALID_ARG;
    if (!aligned(a->q, 16) || !aligned(a->kv, 16) || !aligned(a->swa, 16) || !aligned(a->out, 16))
        return CSA2_ERR_INVALID_ARG;
    if (!decode && (a->swa_rows < 0 || a->swa_pos0 < 0)) return CSA2_ERR_INVALID_ARG;
    return CSA2_OK;
}

static csa2::AttnParams attn_params(const csa2_attn_args* a) {
    csa2::AttnParams p;
    p.q = a->q; p.pos = a->pos; p.idx = a->idx; p.kv = a->kv; p.kv_scale = a->kv_scale; p.kv_row_base = a->kv_row_base;
    p.swa = a->swa; p.swa_scale = a->swa_scale; p.sink = a->sink; p.inv_freq = a->rope_inv_freq; p.out = a->out;
    p.swa_rows = a->swa_rows; p.swa_pos0 = a->swa_pos0; p.rows = a->rows;
    p.topk = a->topk; p.ratio = a->ratio; p.window = a->window;
    p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
    p.splits = 1;
    p.part = nullptr;
    return p;
}

size_t csa2_attn_workspace_size(int32_t rows, int32_t heads, int32_t dim, int32_t window, int32_t topk,
                                int32_t splits) {
    if (rows <= 0 || heads <= 0 || dim <= 0 || window < 0 || topk < 0 || splits < 0 || splits > 8) return 0;
    return csa2::attn_decode_workspace(rows, heads, dim, csa2::attn_decode_splits(rows, heads, dim, window, topk, splits));
}

int32_t csa2_sparse_attn_decode(const csa2_attn_args* a, void* workspace, size_t workspace_bytes,
                                csa2_stream_t stream) {
    int32_t st = validate_attn(a, true);
    if (st != CSA2_OK || a->rows == 0) return st;
    csa2::AttnParams p = attn_params(a);
    p.splits = csa2::attn_decode_splits(a->rows, a->heads, a->dim, a->window, a->topk, a->splits);
    const size_t need = csa2::attn_decode_workspace(a->rows, a->heads, a->dim, p.splits);
    if (workspace_bytes < need) return CSA2_ERR_WORKSPACE;
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 256))) return CSA2_ERR_INVALID_ARG;
    p.part = static_cast<float*>(workspace);
    csa2::AttnShape s{a->heads, a->dim, a->rope_dim, a->q_dtype, a->kv_dtype, a->swa_dtype, a->out_dtype};
    return hip_status(csa2::launch_sparse_attn(p, s, true, reinterpret_cast<hipStream_t>(stream)));
}

int32_t csa2_sparse_attn_prefill(const csa2_attn_args* a, csa2_stream_t stream) {
    int32_t st = validate_attn(a, false);
    if (st != CSA2_OK || a->rows == 0) return st;
    csa2::AttnParams p = attn_params(a);
    csa2::AttnShape s{a->heads, a->dim, a->rope_dim, a->q_dtype, a->kv_dtype, a->swa_dtype, a->out_dtype};
    return hip_status(csa2::launch_sparse_attn(p, s, false, reinterpret_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// csa2_topk_select_noalloc: csa2_topk_select with its workspace in a fixed device array.
//
// The array lives in this library's code object on every GPU it runs on, for the life of the
// process.  Host code never uses its name as an address (it is a host-side stand-in there):
// the device address comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that pointer is passed to kernels.
static __device__ __align__(256) uint8_t csa2_topk_scratch[CSA2_TOPK_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array, or nullptr on a HIP error.
static void* topk_scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(csa2_topk_scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

size_t csa2_topk_noalloc_scratch_bytes(void) { return CSA2_TOPK_NOALLOC_SCRATCH_BYTES; }

int32_t csa2_topk_select_noalloc(const csa2_topk_args* a, csa2_stream_t stream) {
    const int32_t st = validate_topk(a);
    if (st != CSA2_OK) return st;
    const size_t need = csa2_topk_workspace_size(a->rows, a->width, a->k);
    if (need > (size_t)CSA2_TOPK_NOALLOC_SCRATCH_BYTES) return CSA2_ERR_WORKSPACE;
    if (a->rows == 0) return CSA2_OK;
    void* ws = nullptr;
    if (need > 0) {
        ws = topk_scratch_for_current_device();
        if (ws == nullptr) return CSA2_ERR_HIP;
    }
    return csa2_topk_select(a, ws, need, stream);
}

}  // extern "C"

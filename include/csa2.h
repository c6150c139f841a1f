/*
 * csa2.h -- C ABI of the CSA2 sparse-attention hot path for AMD Instinct MI355X (gfx950).
 *
 * The path, as the pages define it for DeepSeek-V4.1-Flash:
 *   1. the lightning indexer scores compressed KV rows
 *      ("DeepSeek-V4.1-Flash 架构解剖", special module "indexer", fig. 3b and
 *      its score formula; "万字长文解析DeekSeekV4.1flash", appendix A.15.2);
 *   2. top-k (k = 512) selects rows per query: FULL over every visible row,
 *      REINDEX over a 2048 x 8 candidate pool, REUSE takes another layer's
 *      selection unchanged (anatomy page, figs. 2b, 2c, 2d);
 *   3. one softmax over the layer's SWA rows plus the selected rows, 64 query
 *      heads over one shared 512-dim latent with K == V, a per-head sink in the
 *      denominator, then the inverse rotation of the output's rope tail
 *      (anatomy page, shared attention path and "出来之后"; "DeepSeek-V4-Pro
 *      架构解剖", attention merge fig. 2d formula).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE memory owned by the caller.  The library
 *     keeps no state between calls, never frees caller memory, and allocates
 *     nothing: scratch space comes in through an explicit workspace argument
 *     whose size the matching *_workspace_size() call reports.  (The one
 *     exception, csa2_topk_select_noalloc, uses a fixed array in the library's
 *     own device memory instead.)
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); the
 *     call returns after the launches, without synchronising.  Calls are
 *     re-entrant; two calls on different streams must not share a workspace.
 *   - Arrays are dense and row-major with the shapes stated below.
 *   - Every output element is written (invalid score columns get -inf,
 *     unfilled top-k slots get -1).
 *   - Arguments are validated on the host before any launch.  An invalid
 *     argument returns CSA2_ERR_INVALID_ARG, a shape/dtype combination with no
 *     compiled kernel returns CSA2_ERR_UNSUPPORTED (never a fallback), a
 *     workspace that is too small returns CSA2_ERR_WORKSPACE; nothing is
 *     launched in those cases.  A HIP launch error returns CSA2_ERR_HIP.
 *   - Caller contracts the library cannot check (it does not read device
 *     memory on the host): planes hold every row a query may touch
 *     (row_base[r] + n_visible(r) rows), candidate blocks are ascending,
 *     FP8/FP4 scales are non-negative.
 *
 * Geometry shared by all calls.  For a query at absolute position pos and
 * compression ratio m, compressed row j is visible iff j < (pos + 1) / m
 * (integer division; the group-causal mask: a row becomes visible once the
 * query has passed its group's last token, "DeepSeek-V4.1-Flash 结构说明",
 * section 4.1).  SWA entry e of a window of W covers position
 * pos - (W - 1) + e and is absent when that position is negative.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 9

/* Status codes. */
#define CSA2_OK 0
#define CSA2_ERR_INVALID_ARG 1
#define CSA2_ERR_UNSUPPORTED 2
#define CSA2_ERR_WORKSPACE 3
#define CSA2_ERR_HIP 4

/* Element types of stored tensors. */
#define CSA2_F32 0      /* IEEE binary32 */
#define CSA2_BF16 1     /* bfloat16 */
#define CSA2_FP8_E4M3 2 /* OCP FP8 E4M3 "FN" (bias 7, S.1111.111 = NaN), one byte per element */
#define CSA2_FP4_E2M1 3 /* OCP FP4 E2M1, two per byte (element 2i in the low nibble) */
/* Rows with their scales inline (the pages' 890 B/token pool, "DeepSeek-V4.1-Flash 架构解剖",
 * "换成 packed FP4 主池"):
 *   CSA2_FP4_E2M1_E4M3G16: D/2 bytes of packed E2M1, then D/16 E4M3 scales, one per 16
 *                          elements (288 B per 512-element row);
 *   CSA2_FP8_E4M3_E8M0G32: D bytes of FP8-E4M3, then D/32 E8M0 scales, one per 32
 *                          elements (528 B per 512-element row). */
#define CSA2_FP4_E2M1_E4M3G16 4
#define CSA2_FP8_E4M3_E8M0G32 5

/* Indexer modes. */
#define CSA2_MODE_FULL 0
#define CSA2_MODE_REINDEX 1

typedef struct ihipStream_t* csa2_stream_t; /* == hipStream_t */

/* ABI version of the loaded library (CSA2_ABI_VERSION it was built with). */
int32_t csa2_abi_version(void);

/* Static, human-readable text for a status code. */
const char* csa2_status_string(int32_t status);

/* ------------------------------------------------------------------------ */
/* Lightning-indexer scores.
 *
 *   score[r, c] = scale * sum_{h < heads} w[r, h] * ReLU(<q[r, h, :], k(row(r, c), :)>)
 *
 * ("DeepSeek-V4.1-Flash 架构解剖", special module "indexer", score formula:
 * a weighted sum over indexer heads of per-head dot products, w without an
 * activation, scale = dim^-1/2 * heads^-1/2; the per-head ReLU is the long
 * essay's appendix A.15.2 pseudo-code.)
 *
 * FULL:    row(r, c) = row_base[r] + c, valid iff c < (pos[r] + 1) / ratio.
 *          Only valid columns are read; columns [n_visible, width) get -inf.
 * REINDEX: column c = i * block_rows + t maps to plane row
 *          row_base[r] + cand[r, i] * block_rows + t, valid iff
 *          cand[r, i] >= 0 and cand[r, i] * block_rows + t < (pos[r] + 1) / ratio
 *          (anatomy page, fig. 2c REINDEX: re-score only the 2048 x 8
 *          candidate rows).  width must equal n_blocks * block_rows.
 *
 * FP8 (k_dtype == q_dtype == CSA2_FP8_E4M3): k is scaled by k_scale[row]; the
 * query's per-(row, head) scale is folded into w by the caller (anatomy page,
 * fig. 3b: the FP32 scale is folded into w, not passed separately).
 *
 * MXFP4 (k_dtype == q_dtype == CSA2_FP4_E2M1): q is [rows, heads, dim / 2]
 * packed E2M1 with E8M0 block scales q_scale_e8m0 [rows, heads, dim / 32], k is
 * [*, dim / 2] with k_scale_e8m0 [*, dim / 32] (one E8M0 byte per 32 elements,
 * a power of two; "DeepSeek-V4.1-Flash 结构说明" §5.3: the indexer keys and, at
 * inference, the indexer query are FP4 with one E8M0 scale per 32 channels;
 * "万字长文解析DeekSeekV4.1flash" §10.6: 64 + 4 bytes per key row).  Each
 * dot product is the sum over 32-element blocks of (q block . k block) times
 * both blocks' scales; k_scale is NULL.  (heads, dim) = (64, 128), FULL, or
 * REINDEX with block_rows 8.
 *
 * REINDEX with block_rows 8 (the pages' 2048 x 8 pool) and (heads, dim) =
 * (64, 128) gathers whole candidate blocks for BF16, FP8 and MXFP4 planes and
 * computes every column with the FULL pass's arithmetic, so its scores are
 * bit-identical to the FULL scores of the same plane rows.
 *
 * Supported: (heads, dim) in {(4, 32), (64, 128)}; q_dtype == k_dtype in
 * {F32, BF16, FP8_E4M3}, or FP4_E2M1 as above.  rows * width fits in int64.
 *
 * flags: CSA2_INDEX_SHARED_PLANE (FULL only) is the caller's statement that
 * row_base holds one value in every row (the query tokens of a prefill chunk
 * of one sequence all index that sequence's compressed rows).  The library
 * may then read row_base[0] only and stage each key tile once for several
 * query rows (BF16 planes of 64 x 128 without key_hist or block_max); the
 * scores are bit-identical to those of the same call without the flag.
 *
 * CSA2_INDEX_BLOCK_KEYS16 (score-free mode over FP8 or MXFP4 planes, not with
 * CSA2_INDEX_SHARED_PLANE): block_keys holds uint16_t entries, the top 16 bits
 * of each block key, which are all the select reads of them (it ranks blocks
 * by the keys' top 12 bits); half the bytes of the 32-bit keys.  The same flag
 * must then be given to csa2_topk_rescore.  Such keys cannot feed
 * csa2_candidate_pool, which ranks blocks by the full key.
 * Other bits must be 0.
 */
#define CSA2_INDEX_SHARED_PLANE 1
#define CSA2_INDEX_BLOCK_KEYS16 2
typedef struct csa2_index_args {
    uint32_t struct_size;       /* sizeof(csa2_index_args) */
    int32_t mode;               /* CSA2_MODE_FULL | CSA2_MODE_REINDEX */
    int32_t rows;               /* query rows, >= 0 */
    int32_t heads;              /* indexer heads H_I */
    int32_t dim;                /* indexer head dim D_I */
    int32_t ratio;              /* compression ratio m, 1 or 2 */
    int32_t q_dtype;            /* element type of q */
    int32_t k_dtype;            /* element type of k */
    int32_t n_blocks;           /* REINDEX: candidate blocks per row (ignored for FULL) */
    int32_t block_rows;         /* REINDEX: rows per candidate block, 1..64.  FULL with block_max:
                                 * rows per pooled block, a power of two in 4..64.  Else ignored. */
    int32_t flags;              /* CSA2_INDEX_SHARED_PLANE, CSA2_INDEX_BLOCK_KEYS16, or 0 */
    int64_t width;              /* columns per score row (FULL: >= every n_visible) */
    const void* q;              /* [rows, heads, dim] */
    const float* w;             /* [rows, heads] effective head weights */
    const void* k;              /* index-key plane [*, dim] */
    const float* k_scale;       /* FP8: [*] per-row scale, same row numbering as k; else NULL */
    const int64_t* row_base;    /* [rows] first plane row of the query's sequence */
    const int64_t* pos;         /* [rows] absolute query positions, >= 0 */
    const int32_t* cand;        /* REINDEX: [rows, n_blocks] block ids, ascending, -1 padded; else NULL */
    float scale;                /* score scale (dim^-1/2 * heads^-1/2 in the pages' model) */
    int32_t _pad1;
    float* scores;              /* out: [rows, width] float32; NULL selects score-free mode (see
                                 * csa2_topk_rescore; FULL, FP8 or MXFP4 64 x 128, or BF16 64 x 128
                                 * with CSA2_INDEX_SHARED_PLANE; block_keys required, key_hist NULL) */
    uint32_t* key_hist;         /* optional out: [rows, 4096], or NULL.  The call zeroes it, then
                                 * counts every valid score of row r in bin key(score) >> 20, where
                                 * key is the order-preserving 32-bit key csa2_topk_select ranks by
                                 * (bits | 0x80000000 for scores >= +0, ~bits below, NaN as -inf,
                                 * -0 as +0).  Passing it on to csa2_topk_select saves that call a
                                 * full pass over the scores of rows wider than 65536 columns (it
                                 * reads narrower rows once and does not use it).  NULL in
                                 * score-free mode. */
    float* block_max;           /* optional out, FULL only: [rows, ceil(width / block_rows)], or NULL.
                                 * Block b of row r gets the block score csa2_candidate_pool ranks:
                                 * the largest score over its visible columns, with NaN read as -inf
                                 * and +-inf clipped to +-FLT_MAX; the block holding the newest
                                 * visible row ((n_visible - 1) / block_rows) gets +inf; blocks with
                                 * no visible column get -inf.  Written in the same pass as the
                                 * scores (no second read of them). */
    uint32_t* block_keys;       /* score-free mode only (scores == NULL), out: [rows, ceil(width / 8)]
                                 * (uint16_t entries, the keys' top 16 bits, with
                                 * CSA2_INDEX_BLOCK_KEYS16).
                                 * Entry b holds the largest key of the valid columns 8b .. 8b+7,
                                 * or 0 when none is valid; a column's key is its order key (as for
                                 * key_hist), except that a NaN score counts as 0x007FFFFE, just
                                 * below -inf (so the candidate pool can still tell NaN from -inf). */
    const uint8_t* q_scale_e8m0; /* MXFP4: [rows, heads, dim / 32] E8M0 block scales of q; else NULL */
    const uint8_t* k_scale_e8m0; /* MXFP4: [*, dim / 32] E8M0 block scales of k, same row numbering as
                                  * k; else NULL */
} csa2_index_args;

int32_t csa2_indexer_score(const csa2_index_args* args, csa2_stream_t stream);

/* Score-free FULL top-k.
 *
 * Writing a [rows, width] score matrix only to read it back for the top-k
 * costs more than the scoring itself reads when rows are 1M columns wide.  In
 * score-free mode (csa2_indexer_score with scores == NULL, which requires FULL
 * mode and block_keys, and key_hist NULL) the scores stay on chip: the call
 * writes the per-8-column block keys only.  csa2_topk_rescore then takes the
 * same arguments and returns the top-k: it counts the block keys' top 12 bits
 * per row and finds the bin b1 holding each row's k-th largest block key (the
 * k blocks with the largest keys hold k columns with keys in bins >= b1, so
 * every selected column has a key in a bin >= b1), re-scores exactly the
 * blocks whose block key reaches b1 (every selected column lies in one), with
 * the same arithmetic as the scoring pass, and runs the exact select of
 * csa2_topk_select over their columns in bins >= b1.  The result is bit-identical to
 * csa2_topk_select over the scores csa2_indexer_score would have written.
 *
 * BF16 planes whose rows share one plane (CSA2_INDEX_SHARED_PLANE: a prefill
 * chunk, whose score matrix would be rows x width floats) take another route
 * to the same result: the k best blocks by block key (ties to the lower
 * block) are chosen, their 8 k columns re-scored with the FULL pass's
 * arithmetic (the REINDEX kernel), and the exact select runs over those.
 * Every selected column lies in a chosen block: its score is at least T, the
 * k-th largest block key, so its block's key is too; all blocks with a key
 * above T are chosen, and if the k-th largest score equals T, the
 * lowest-numbered columns with score T lie in the lowest-numbered blocks with
 * key T, as many of which are chosen as the k slots leave.
 *
 * args: as given to the score-free csa2_indexer_score call (block_keys is now
 * an input; key_hist NULL; scores and block_max are ignored).
 * out: [rows, k] int32, ascending plane rows, -1 padded.
 * Supported: FP8-E4M3 or MXFP4 q and k with (heads, dim) = (64, 128), rows <
 * 1024 and 8192 <= width < 2^24; or BF16 q and k with (heads, dim) = (64, 128)
 * and CSA2_INDEX_SHARED_PLANE, any rows and width < 2^31; 1 <= k <= 2048; else
 * CSA2_ERR_UNSUPPORTED.  The workspace size covers either route.
 */
size_t csa2_topk_rescore_workspace_size(int32_t rows, int64_t width, int32_t k);

int32_t csa2_topk_rescore(const csa2_index_args* args, int32_t k, int32_t* out, void* workspace,
                          size_t workspace_bytes, csa2_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Per-row top-k of indexer scores.
 *
 * Selects, per row, the k valid columns with the largest scores, ranking by
 * score descending and breaking ties by the lower column; NaN ranks as -inf
 * and -0 equals +0.  The chosen columns are written in increasing column
 * order, mapped to plane rows (FULL: the column itself; REINDEX:
 * cand[r, i] * block_rows + t, which is increasing when the candidate blocks
 * are ascending), followed by -1 when fewer than k columns are valid
 * ("DeepSeek-V4.1-Flash 架构解剖", fig. 2d REUSE: selected [rows, 512],
 * ascending, -1 filled; special module "indexer": -1 means the history is
 * shorter than k).  Validity is the same as in csa2_indexer_score: FULL
 * column c < (pos[r] + 1) / ratio, REINDEX through cand.  Row r of `out`
 * holds plane-relative rows (without row_base), the numbering
 * csa2_sparse_attn_* expects in `idx`.
 *
 * Supported: 1 <= k <= 2048; width < 2^31.
 */
typedef struct csa2_topk_args {
    uint32_t struct_size;       /* sizeof(csa2_topk_args) */
    int32_t rows;               /* score rows, >= 0 */
    int32_t k;                  /* selections per row */
    int32_t ratio;              /* compression ratio m, 1 or 2 */
    int32_t n_blocks;           /* REINDEX: candidate blocks per row; 0 selects FULL validity */
    int32_t block_rows;         /* REINDEX: rows per block */
    int64_t width;              /* columns per score row (REINDEX: n_blocks * block_rows) */
    const float* scores;        /* [rows, width] */
    const int64_t* pos;         /* [rows] absolute query positions */
    const int32_t* cand;        /* REINDEX: [rows, n_blocks]; NULL for FULL */
    int32_t* out;               /* out: [rows, k] int32 */
    const uint32_t* key_hist;   /* optional: [rows, 4096] histogram csa2_indexer_score wrote for exactly
                                 * these scores and this validity, or NULL */
} csa2_topk_args;

/* Bytes of workspace csa2_topk_select needs for these sizes: 0 for rows up to 65536 columns wide (one
 * workgroup per row; key_hist is then not read), and for 1024 or more rows. */
size_t csa2_topk_workspace_size(int32_t rows, int64_t width, int32_t k);

int32_t csa2_topk_select(const csa2_topk_args* args, void* workspace, size_t workspace_bytes,
                         csa2_stream_t stream);

/* The same top-k for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the workspace is a
 * fixed array of CSA2_TOPK_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per
 * GPU, held until the process ends.  Results are identical to csa2_topk_select's.
 *
 *   - No hipMalloc / hipFree or allocating library call is made.  The first call on a
 *     device looks up that device's array (hipGetSymbolAddress, with the device current);
 *     the call uses the current device, which must be the stream's.
 *   - Sizes whose csa2_topk_workspace_size exceeds CSA2_TOPK_NOALLOC_SCRATCH_BYTES return
 *     CSA2_ERR_WORKSPACE before anything is launched (40 MiB covers, e.g., 256 rows of
 *     2^20 columns; rows >= 1024 and widths up to 65536 need no workspace at all).
 *   - Every call on one GPU shares that GPU's array and leaves its contents behind; the
 *     call's own kernels initialise everything they read, so nothing needs clearing.
 *     Calls that overlap on one GPU (concurrent streams, several host threads) race on
 *     the array: serialise them.
 * Other arguments, validation and status codes as for csa2_topk_select.
 */
#define CSA2_TOPK_NOALLOC_SCRATCH_BYTES (40u << 20)

size_t csa2_topk_noalloc_scratch_bytes(void);

int32_t csa2_topk_select_noalloc(const csa2_topk_args* args, csa2_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Hierarchical candidate pool of the FULL owner layer.
 *
 * From the FULL layer's own score rows, cut into blocks of block_rows
 * consecutive rows (8, the index plane's page height, in the pages' model):
 *
 *   block score  = max over the block's visible columns of the score, NaN read
 *                  as -inf and +-inf clipped to +-FLT_MAX;
 *   newest block = the one holding row (pos + 1) / ratio - 1, pinned to +inf;
 *   cand[r, :]   = the n_cand best of the ceil(n_visible / block_rows) blocks,
 *                  by block score descending and the lower block id on ties,
 *                  written ascending and padded with -1.
 *
 * ("DeepSeek-V4.1-Flash 架构解剖", special module "indexer", fig. 3b second
 * level and fig. 3 candidate blocks; "DeepSeek-V4.1-Flash 结构说明" section 5.2;
 * "万字长文解析DeekSeekV4.1flash" section 4 and appendix A.11.)  The result is
 * the cand argument of the REINDEX calls (csa2_indexer_score,
 * csa2_topk_select) of the layers that share this owner's plane.
 *
 * Block scores come from block_keys (written by a score-free
 * csa2_indexer_score pass), else from block_max (what csa2_indexer_score wrote
 * in the scoring pass), else are computed here from scores into the workspace.
 *
 * Supported: block_rows a power of two in 4..64; 1 <= n_cand <= 2048;
 * width < 2^31.
 */
typedef struct csa2_pool_args {
    uint32_t struct_size;       /* sizeof(csa2_pool_args) */
    int32_t rows;               /* score rows, >= 0 */
    int32_t ratio;              /* compression ratio m, 1 or 2 */
    int32_t block_rows;         /* rows per block */
    int32_t n_cand;             /* blocks kept per row (2048 in the pages' model) */
    int32_t _pad0;
    int64_t width;              /* columns per FULL score row */
    const float* scores;        /* [rows, width] FULL scores, or NULL when block_max is given */
    const float* block_max;     /* [rows, ceil(width / block_rows)] from csa2_indexer_score, or NULL */
    const int64_t* pos;         /* [rows] absolute query positions */
    int32_t* cand;              /* out: [rows, n_cand] block ids */
    const uint32_t* block_keys; /* [rows, ceil(width / 8)] from a score-free csa2_indexer_score, or NULL;
                                 * when given (block_rows must be 8) the block scores are derived
                                 * from it and scores / block_max are ignored */
} csa2_pool_args;

/* Bytes of workspace csa2_candidate_pool needs (enough with or without block_max). */
size_t csa2_candidate_pool_workspace_size(int32_t rows, int64_t width, int32_t block_rows, int32_t n_cand);

int32_t csa2_candidate_pool(const csa2_pool_args* args, void* workspace, size_t workspace_bytes,
                            csa2_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Sparse sink attention.
 *
 * For query row r, head h and the entry multiset S(r) = {valid SWA entries}
 * plus {kv row row_base[r] + idx[r, i] : 0 <= idx[r, i] < (pos[r] + 1) / ratio}
 * (no de-duplication; -1 and out-of-range indices are skipped):
 *
 *   s_j      = softmax_scale * <q[r, h, :], v_j>
 *   o[r, h]  = sum_j e^{s_j} v_j / (e^{sink[h]} + sum_j e^{s_j})
 *   out[r,h] = o[r, h] with pair (D-R+2i, D-R+2i+1) rotated by -pos[r] * inv_freq[i]
 *
 * K and V are the same stored row; q arrives already rotated; the sink is an
 * unscaled logit without a value ("DeepSeek-V4-Pro 架构解剖", attention merge
 * fig. 2d formula; "DeepSeek-V4.1-Flash 架构解剖", "四种层合并出来的是什么形状"
 * and "出来之后"; "DeepSeek-V4.1-Flash 结构说明", sections 4.1 and 6.1).  An
 * empty S gives out = 0.
 *
 * SWA source:
 *   decode  (csa2_sparse_attn_decode): one ring per query row, swa [rows, window, dim];
 *           slot s holds position pos - ((pos - s) mod window), absent if negative
 *           (structure page, section 4.4: the ring is written at start_pos mod 128).
 *   prefill (csa2_sparse_attn_prefill): one linear array swa [swa_rows, dim] whose
 *           row t holds position swa_pos0 + t, shared by all query rows; query r
 *           sees positions max(0, pos[r] - window + 1) .. pos[r] that the array holds.
 *
 * Storage: q and out are F32 or BF16 [rows, heads, dim].  kv is F32 or BF16
 * [*, dim], or FP4_E2M1 packed [*, dim/2] bytes with kv_scale = E8M0 bytes
 * [*, dim/32] (one power-of-two scale per 32 elements).  swa is F32 or BF16,
 * or FP8_E4M3 with swa_scale = float32 per swa row ([rows, window] in decode,
 * [swa_rows] in prefill).  With the inline-scale types kv rows are
 * dim/2 + dim/16 bytes (FP4_E2M1_E4M3G16) and swa rows dim + dim/32 bytes
 * (FP8_E4M3_E8M0G32); the shapes above then count bytes in their last axis.
 *
 * Supported: (heads, dim, rope_dim) in {(4, 64, 16), (64, 512, 64)}; window
 * a multiple of 16 in [16, 1024] and topk a multiple of 16 in [0, 2048]; F32 only together with F32 everywhere (the
 * (4, 64, 16) shape); otherwise BF16 q/out with kv BF16 or FP4 and swa BF16
 * or FP8, or kv FP4_E2M1_E4M3G16 with swa FP8_E4M3_E8M0G32 (scales inline:
 * kv_scale and swa_scale NULL).  rope_inv_freq holds rope_dim/2 float64 frequencies in device
 * memory (see csa2_rope_inv_freq).
 *
 * Decode splits each row's entries over `splits` workgroups (a decode batch
 * has few rows, and one workgroup per row would leave most of the GPU idle):
 * with more than one split each workgroup writes its partial softmax state
 * (running max, sum, unnormalised values, per head) to the workspace and a
 * second kernel merges the splits' states, normalises, rotates and stores.
 * splits = 0 lets the library choose (256 / rows, at most 8, at most 4 from
 * 32 rows on, at most one per pair of 16-entry tiles); 1..8 asks for that
 * many.  csa2_attn_workspace_size returns the bytes for the
 * same arguments (0 when no split is made, and for prefill); decode returns
 * CSA2_ERR_WORKSPACE when the workspace is smaller.
 */
typedef struct csa2_attn_args {
    uint32_t struct_size;       /* sizeof(csa2_attn_args) */
    int32_t rows;               /* query rows, >= 0 */
    int32_t heads;              /* query heads H */
    int32_t dim;                /* latent dim D */
    int32_t rope_dim;           /* rotated tail R */
    int32_t topk;               /* idx entries per row */
    int32_t ratio;              /* compression ratio m, 1 or 2 */
    int32_t window;             /* SWA window W */
    int32_t q_dtype;
    int32_t kv_dtype;
    int32_t swa_dtype;
    int32_t out_dtype;
    int32_t splits;             /* decode: workgroups per row splitting its entries,
                                 * 0 = the library's choice, at most 8; prefill: ignored, 0..8 */
    int32_t _pad0;
    int64_t swa_rows;           /* prefill: rows of the linear SWA array */
    int64_t swa_pos0;           /* prefill: position of linear SWA row 0 */
    const void* q;              /* [rows, heads, dim], rope tail already rotated */
    const int64_t* pos;         /* [rows] absolute positions, >= 0 */
    const int32_t* idx;         /* [rows, topk] plane-relative selected rows, -1 padded */
    const void* kv;             /* main plane rows */
    const uint8_t* kv_scale;    /* FP4: E8M0 [*, dim/32]; else NULL */
    const int64_t* kv_row_base; /* [rows] first kv row of the query's sequence */
    const void* swa;            /* SWA rows (ring or linear, see above) */
    const float* swa_scale;     /* FP8: per-row scales; else NULL */
    const float* sink;          /* [heads] */
    const double* rope_inv_freq;/* [rope_dim/2] device float64 */
    float softmax_scale;        /* dim^-1/2 in the pages' model */
    int32_t _pad1;
    void* out;                  /* out: [rows, heads, dim] */
} csa2_attn_args;

/* Bytes of workspace csa2_sparse_attn_decode needs for these sizes and splits (see above). */
size_t csa2_attn_workspace_size(int32_t rows, int32_t heads, int32_t dim, int32_t window, int32_t topk,
                                int32_t splits);

int32_t csa2_sparse_attn_decode(const csa2_attn_args* args, void* workspace, size_t workspace_bytes,
                                csa2_stream_t stream);

int32_t csa2_sparse_attn_prefill(const csa2_attn_args* args, csa2_stream_t stream);

/* ------------------------------------------------------------------------ */
/* The FULL layer's write path: compressor, main row and index key.
 *
 * For the token rows of one call (rows of one sequence consecutive, at
 * consecutive positions), with D = 512 latent channels and a 128-wide key:
 *   kv[r] = wkv . x[r]; at ratio 2 also score[r] = wgate . x[r]  (FP32)
 *   group j covers positions [j*ratio, j*ratio + ratio - 1] (no overlap);
 *   latent_j = RMSNorm(pooled) * norm_w, where pooled is, per channel, the
 *              softmax over the group's positions of score weighting kv
 *              (ratio 1: kv itself);
 *   main row j  = latent_j with its last 64 dims rotated at position j*ratio
 *                 (adjacent pairs, angles pos * rope_inv_freq[i]);
 *   index key j = RMSNorm(wk . latent_j) * knorm_w, with its last 64 dims
 *                 rotated the same way.
 * Row j of both planes is written at plane row row_base[r] + j by the token
 * row r that completes group j.  ("万字长文解析DeekSeekV4.1flash" appendix
 * A.15.1 and §6.2; "DeepSeek-V4.1-Flash 架构解剖", special module
 * "compressor": FP32 pooling, non-overlapping groups, rotation before the
 * write, the indexer's wk reads the latent before rotation; special module
 * "indexer", key side: wk -> k_norm -> rotation -> the index plane;
 * "DeepSeek-V4.1-Flash 结构说明" §4: the rotation position of a compressed
 * entry is its group's first token.)  k_norm is an RMSNorm with a learned
 * weight.
 *
 * Ratio 2 tail state: a token at an even position whose group partner is not
 * the next row of the call leaves its kv and score in tail_kv / tail_score
 * [slot[r]]; a token at an odd position whose partner is not the previous row
 * of the call pools with the tail state of its slot, which must hold position
 * pos - 1 (the caller's contract).  Tail state read and written in one call
 * is consistent (reads see the state the call started with).
 *
 * Storage of the written rows (plane row n):
 *   main_dtype  F32 / BF16 [n, 512]; FP4_E2M1 packed [n, 256] + E8M0
 *               main_scale_out [n, 16] (one scale per 32: 2^ceil(log2(amax/6)));
 *               FP4_E2M1_E4M3G16 [n, 288] inline (E4M3 scale per 16 =
 *               E4M3(amax/6) clamped to [2^-9, 448]).
 *   idx_dtype   F32 / BF16 [n, 128]; FP8_E4M3 [n, 128] + float32 idx_scale_out
 *               [n] (amax/448, 1 for a zero row); FP4_E2M1 packed [n, 64] +
 *               E8M0 idx_scale_out [n, 4].
 * E4M3 and E2M1 round to nearest even and saturate (448, 6); the scaled
 * values are formed in float32 with IEEE division.
 *
 * Supported: dim 512, idx_dim 128, rope_dim 64, ratio 1 or 2, d_in a positive
 * multiple of 64.  x and the weights are bf16; x, wkv, wgate and wk 16-byte
 * aligned.  wgate, tail_kv and tail_score are required at ratio 2 and NULL at
 * ratio 1.  workspace: csa2_compress_workspace_size bytes, 256-byte aligned.
 * All pointers are device memory owned by the caller.
 */
typedef struct csa2_compress_args {
    uint32_t struct_size;       /* sizeof(csa2_compress_args) */
    int32_t rows;               /* token rows R, >= 0 */
    int32_t d_in;               /* hidden width of x and the projections' inputs */
    int32_t ratio;              /* 1 or 2 */
    int32_t dim;                /* latent width, 512 */
    int32_t idx_dim;            /* index key width, 128 */
    int32_t rope_dim;           /* rotated tail, 64 */
    int32_t main_dtype;         /* see above */
    int32_t idx_dtype;          /* see above */
    int32_t _pad0;
    const void* x;              /* [R, d_in] bf16 hidden rows */
    const int64_t* pos;         /* [R] absolute positions, >= 0 */
    const int32_t* slot;        /* [R] tail-state slot of the row's sequence, >= 0 */
    const int64_t* row_base;    /* [R] first plane row of the row's sequence */
    const void* wkv;            /* [dim, d_in] bf16 */
    const void* wgate;          /* ratio 2: [dim, d_in] bf16; else NULL */
    const float* norm_w;        /* [dim] */
    const void* wk;             /* [idx_dim, dim] bf16 */
    const float* knorm_w;       /* [idx_dim] */
    const double* rope_inv_freq;/* [rope_dim / 2] (see csa2_rope_inv_freq) */
    float eps;                  /* RMSNorm epsilon of the latent, >= 0 */
    float k_eps;                /* RMSNorm epsilon of the key, >= 0 */
    float* tail_kv;             /* ratio 2: [slots, dim] in/out; else NULL */
    float* tail_score;          /* ratio 2: [slots, dim] in/out; else NULL */
    void* main_out;             /* main plane */
    void* main_scale_out;       /* FP4_E2M1: E8M0 [*, dim / 32]; else NULL */
    void* idx_out;              /* index plane */
    void* idx_scale_out;        /* FP8: float32 [*]; FP4_E2M1: E8M0 [*, idx_dim / 32]; else NULL */
} csa2_compress_args;

size_t csa2_compress_workspace_size(int32_t rows, int32_t d_in, int32_t ratio);

int32_t csa2_compress(const csa2_compress_args* args, void* workspace, size_t workspace_bytes,
                      csa2_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Host helper: RoPE frequencies in float64, written to HOST memory.
 *
 * out[i] = theta^(-2i/rope_dim) for i < rope_dim/2 ("DeepSeek-V4.1-Flash
 * 结构说明", section 6.1: 32 frequencies base^(-2i/64), adjacent-pair
 * rotation).  With yarn_factor > 1 and yarn_orig_len > 0 each frequency is
 * interpolated by the YaRN NTK-by-parts rule (section 6.3 splits the
 * frequencies into three bands by how many turns they make within the
 * original length; the band formula is the YaRN paper's, with alpha = 1 and
 * beta = 32): r = yarn_orig_len * f / (2 pi); g = clamp((r - 1) / 31, 0, 1);
 * f' = (1 - g) f / yarn_factor + g f.
 * Returns CSA2_ERR_INVALID_ARG for odd or non-positive rope_dim, theta <= 1,
 * yarn_factor < 1 or a NULL out.
 */
int32_t csa2_rope_inv_freq(int32_t rope_dim, double theta, double yarn_factor, int64_t yarn_orig_len,
                           double* out);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */

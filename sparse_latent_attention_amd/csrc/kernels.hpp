// Internal launch interface between the C ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

struct IndexParams {
    const void* q;
    const float* w;
    const void* k;
    const float* k_scale;
    const int64_t* row_base;
    const int64_t* pos;
    const int32_t* cand;
    float* scores;
    uint32_t* key_hist;  // optional [rows, 4096]
    float* block_max;    // optional [rows, bm_blocks] (FULL only)
    uint32_t* block_keys;  // optional [rows, ceil(width / kKeyBlock)] (FULL only)
    const uint8_t* q_e8;   // MXFP4 query: E8M0 [rows, heads, dim / 32]
    const uint8_t* k_e8;   // MXFP4 keys: E8M0 [*, dim / 32]
    int64_t width;
    int64_t cols_per_wg;
    int64_t bm_blocks;   // ceil(width / bm_rows)
    int32_t n_blocks;
    int32_t block_rows;
    int32_t bm_rows;     // rows per pooled block (power of two, 4..64)
    int32_t ratio;
    float scale;
    bool shared_plane;   // every row reads the plane rows of row_base[0]
    bool bk16;           // block_keys holds uint16_t entries: the keys' top 16 bits
};

hipError_t launch_indexer_score(const IndexParams& p, int rows, int heads, int dim, int dtype, bool reindex,
                                hipStream_t stream);
bool indexer_supported(int heads, int dim, int dtype);

struct TopkParams {
    const float* scores;
    const int64_t* pos;
    const int32_t* cand;
    int32_t* out;
    const uint32_t* key_hist;  // optional [rows, 4096] from the indexer
    int64_t width;
    int32_t k;
    int32_t ratio;
    int32_t n_blocks;  // 0: FULL validity
    int32_t block_rows;
    int32_t col_group;  // FULL validity over groups: column c valid iff c < ceil(n_visible / col_group)
    // Candidate pool from block keys: when set, column c of row r ranks by the pool's
    // block score of pool_keys[r * width + c] (the newest valid column pinned to +inf)
    // instead of scores.
    const uint32_t* pool_keys;
    // With pool_keys: rank column c by the plain block key pool_keys[r * width + c] instead (the
    // largest score of an 8-column block, NaN as -inf; no pinning): the best blocks of a score row.
    bool plain_keys;
};

// Bytes of workspace the launch plan for (rows, width) needs (0: one workgroup per row).
size_t topk_workspace_bytes(int rows, int64_t width);
hipError_t launch_topk_select(const TopkParams& p, int rows, void* workspace, hipStream_t stream);

// Pieces of the wide-row select used by the score-free path: the threshold bin
// of the k-th key from a key histogram, and the exact select over per-segment
// (key, column) lists of capacity cap (a longer list falls back to p.scores).
void topk_plan(int rows, int64_t width, int& chunk, int& nseg, int min_chunk);
// Per-row histograms of block keys' top 12 bits as [rows, parts, 4096] partial
// counts (parts = block_key_hist_parts(nbk_row)).
int block_key_hist_parts(int64_t nbk_row);
hipError_t launch_block_key_hist(const uint32_t* bkeys, bool bk16, int64_t nbk_row, int rows, uint32_t* hist,
                                 hipStream_t stream);
hipError_t launch_topk_threshold(const TopkParams& p, int rows, const uint32_t* key_hist, int parts, uint32_t* b1,
                                 hipStream_t stream);
hipError_t launch_topk_final(const TopkParams& p, int rows, const uint32_t* cand_keys, const int32_t* cand_cols,
                             const uint32_t* seg_count, int nseg, int cap, hipStream_t stream);

// Re-scoring of candidate blocks for the score-free FP8 FULL path.
bool indexer_rescore_supported(int heads, int dim, int dtype);
hipError_t launch_indexer_rescore(const IndexParams& p, int rows, int dtype, const uint32_t* b1, int chunk, int nseg,
                                  uint32_t* cand_keys, int32_t* cand_cols, uint32_t* seg_count, hipStream_t stream);

// Block scores of the candidate pool from FULL score rows (out: [rows, nb]).
hipError_t launch_block_max(const float* scores, const int64_t* pos, int ratio, int64_t width, int block_rows,
                            int rows, float* out, hipStream_t stream);

struct AttnParams {
    const void* q;
    const int64_t* pos;
    const int32_t* idx;
    const void* kv;
    const uint8_t* kv_scale;
    const int64_t* kv_row_base;
    const void* swa;
    const float* swa_scale;
    const float* sink;
    const double* inv_freq;
    void* out;
    int64_t swa_rows;
    int64_t swa_pos0;
    int32_t rows;
    int32_t topk;
    int32_t ratio;
    int32_t window;
    float scale_log2;  // softmax_scale * log2(e)
    int32_t splits;    // decode: workgroups per row that split its entries (1: none)
    float* part;       // splits > 1: partial softmax states [rows, head groups, splits, 16 x (2 + dim)]
};

// Decode attention plan: splits of each row's entries over workgroups (1 = no split), and the
// workspace bytes their partial states take.
int attn_decode_splits(int rows, int heads, int dim, int window, int topk, int requested);
size_t attn_decode_workspace(int rows, int heads, int dim, int splits);

struct AttnShape {
    int heads, dim, rope_dim;
    int q_dtype, kv_dtype, swa_dtype, out_dtype;
};

bool attn_supported(const AttnShape& s);
hipError_t launch_sparse_attn(const AttnParams& p, const AttnShape& s, bool decode, hipStream_t stream);

// The FULL layer's write path (compress.hip).
struct CompressParams {
    const uint16_t* x;       // [rows, d_in] bf16
    const int64_t* pos;      // [rows]
    const int32_t* slot;     // [rows] tail-state slot
    const int64_t* row_base; // [rows]
    const uint16_t* wkv;     // [512, d_in] bf16
    const uint16_t* wgate;   // [512, d_in] bf16 (ratio 2)
    const float* norm_w;     // [512]
    const uint16_t* wk;      // [128, 512] bf16
    const float* knorm_w;    // [128]
    const double* inv_freq;  // [32]
    float* tail_kv;          // [slots, 512] (ratio 2)
    float* tail_score;       // [slots, 512] (ratio 2)
    void* main_out;
    void* main_scale_out;
    void* idx_out;
    void* idx_scale_out;
    float* partial;          // workspace [ksplit, rows, nproj]
    float eps, k_eps;
    int rows, d_in, nproj, ksplit;
};

bool compress_supported(int main_dtype, int idx_dtype);
hipError_t launch_compress(const CompressParams& p, int ratio, int main_dtype, int idx_dtype, hipStream_t stream);

}  // namespace csa2

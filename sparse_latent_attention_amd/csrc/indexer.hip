// Lightning-indexer scores (FULL and REINDEX) for gfx950.
//
//   score[r, c] = scale * sum_h w[r, h] * ReLU(<q[r, h, :], k[row(r, c), :]>)
//
// ("DeepSeek-V4.1-Flash 架构解剖", special module "indexer", fig. 3b and the
// score formula; per-head ReLU from "万字长文解析DeekSeekV4.1flash", appendix
// A.15.2; REINDEX column mapping from the anatomy page, fig. 2c.)
//
// Design.  The work is a stream over key rows: every key row is read once and
// used by all indexer heads of one query row, so the kernel is bound by HBM
// (132 B per key row in FP8, 256 B in BF16) and needs the matrix cores only to
// keep the 64 x 128 multiply-adds per key row below the memory time.  Each
// wave holds the query row's 64 heads as MFMA A operands in registers for the
// whole launch and streams 64 key rows per step straight from HBM into B
// operands (no LDS): lane l loads row l%16 of a 16-row tile, k-group l/16,
// 64 contiguous bytes per row per load instruction.  The 16x16 result tile
// holds 4 heads x 1 column per lane, so the head reduction is 16 in-lane
// multiply-adds plus a 3-shuffle reduce-scatter across the 4 lane groups that
// leaves lane l with column l of the 64 -- one coalesced 256-byte store.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

namespace {

// NaN rule: a NaN dot stays NaN through the per-head ReLU, so a score with
// one is NaN (and ranks as -inf).  A NaN can only come from the inputs: a key
// row holding a NaN makes its dot with every head NaN, a NaN in the query
// makes every dot of that head NaN.  Both cases are carried without a NaN
// test per dot:
//   * relu_bits: ReLU as an integer max on the float's bits (one
//     instruction): negative values, -0 and -inf become +0; positive values,
//     +inf and NaNs with the sign bit clear pass unchanged;
//   * nan_guard: each lane's weighted head sum starts from 0 x (its first raw
//     dot), which is +-0, or NaN when that dot is NaN -- a NaN key row thus
//     makes every column sum NaN, whatever the sign bits of its NaN dots;
//   * a query row holding a NaN is found once per row (frag_has_nan) and its
//     scores are set to NaN.
// (Dots beyond the float32 range are outside the inputs the path takes.)
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }
__device__ __forceinline__ float nan_guard(float raw_dot) { return raw_dot * 0.f; }

// Whether a query operand fragment holds a NaN element.
__device__ __forceinline__ bool frag_has_nan(const bf16x8& f) {
    const u32x4 d = __builtin_bit_cast(u32x4, f);
    uint32_t m = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) m |= ((d[e] & 0x7fff7fffu) + 0x007f007fu) & 0x80008000u;  // |half| > 0x7f80
    return m != 0u;
}
__device__ __forceinline__ bool frag_has_nan(const F32x8& f) {
    bool n = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) n |= f.v[e] != f.v[e];
    return n;
}
// FP8-E4M3 codes: a byte is NaN iff its low 7 bits are all ones (zero-byte test on the complement).
__device__ __forceinline__ bool frag_has_nan(const i32x8& f) {
    uint32_t m = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t v = ~(uint32_t)f[e] & 0x7f7f7f7fu;
        m |= (v - 0x01010101u) & ~v & 0x80808080u;
    }
    return m != 0u;
}

// Plane row of column c and whether it is valid.
template <bool REINDEX>
__device__ __forceinline__ bool column_row(const IndexParams& p, int r, int64_t c, int64_t nv, int64_t base,
                                           int64_t& prow) {
    if (!REINDEX) {
        prow = base + c;
        return c < nv;
    }
    const int64_t i = c / p.block_rows;
    const int64_t t = c - i * p.block_rows;
    if (i >= p.n_blocks) return false;
    const int32_t b = p.cand[(int64_t)r * p.n_blocks + i];
    if (b < 0) return false;
    const int64_t jr = (int64_t)b * p.block_rows + t;
    prow = base + jr;
    return jr < nv;
}

// A 64-bit value the whole wave holds, moved to scalar registers (it feeds
// buffer descriptors, which must be uniform).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// 16-byte load of key-row bytes.  (Non-temporal loads were measured and
// rejected: with each 128-byte row read as two 64-byte halves by separate
// instructions they ran ~12% slower than ordinary loads.)
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Element-type specific operand loaders.  A "step" covers 32 k-elements for
// F32/BF16 (one 16x16x32 MFMA) and all 128 for FP8 (one 16x16x128 MFMA).
template <int KT, int DI>
struct IdxOps;

template <int DI>
struct IdxOps<CSA2_BF16, DI> {
    static constexpr int kSteps = DI / 32;
    typedef bf16x8 Frag;
    // k-group g of step s: elements 32s + 8g .. +8 (64 contiguous bytes per row per step)
    static __device__ __forceinline__ Frag load(const void* base, int64_t row, int s, int g) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + row * DI + 32 * s + 8 * g;
        return __builtin_bit_cast(Frag, ld16(p));
    }
    static __device__ __forceinline__ Frag zero() { return __builtin_bit_cast(Frag, u32x4{0, 0, 0, 0}); }
    static __device__ __forceinline__ f32x4 mma(f32x4 c, Frag a, Frag b) { return Mma<__bf16>::k32(c, a, b); }
};

template <int DI>
struct IdxOps<CSA2_F32, DI> {
    static constexpr int kSteps = DI / 32;
    typedef F32x8 Frag;
    static __device__ __forceinline__ Frag load(const void* base, int64_t row, int s, int g) {
        const float* p = reinterpret_cast<const float*>(base) + row * DI + 32 * s + 8 * g;
        Frag f;
        f32x4 a = __builtin_bit_cast(f32x4, ld16(p));
        f32x4 b = __builtin_bit_cast(f32x4, ld16(p + 4));
        f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
        f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
        return f;
    }
    static __device__ __forceinline__ Frag zero() {
        Frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = 0.f;
        return f;
    }
    static __device__ __forceinline__ f32x4 mma(f32x4 c, const Frag& a, const Frag& b) { return Mma<float>::k32(c, a, b); }
};

template <>
struct IdxOps<CSA2_FP8_E4M3, 128> {
    static constexpr int kSteps = 1;
    typedef i32x8 Frag;
    // k-group g holds bytes 16g..16g+15 and 64+16g..64+16g+15 of the row, so each
    // of the two loads covers 64 contiguous bytes per row across the 4 groups.
    static __device__ __forceinline__ Frag load(const void* base, int64_t row, int, int g) {
        const uint8_t* p = reinterpret_cast<const uint8_t*>(base) + row * 128 + 16 * g;
        u32x4 a = ld16(p);
        u32x4 b = ld16(p + 64);
        Frag f;
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
        return f;
    }
    static __device__ __forceinline__ Frag zero() { return Frag{0, 0, 0, 0, 0, 0, 0, 0}; }
    static __device__ __forceinline__ f32x4 mma(f32x4 c, Frag a, Frag b) { return mma_fp8_k128(c, a, b); }
};

// Head reduction and output of one 64-column step.  v[u] holds, in lane
// (g, n), the weighted ReLU sum over heads 4g..4g+3 (of every head tile) for
// column 16u + n.  A reduce-scatter over the 4 lane groups leaves lane l with
// column cb + l, which is scaled, stored (one coalesced 256-byte store), and
// optionally counted into the LDS key histogram and folded into block scores.
//
// SCORES = false keeps the scores on chip; BKEYS then records, in the
// workgroup's LDS array bkl, the largest order key of every kKeyBlock columns
// (0 when none is valid), relative to the workgroup's first column c0.
// Reduce over the 4 lane groups and scatter: lane l ends with column l of the
// step.  Every column's sum is formed as (g0 + g2) + (g1 + g3) up to the order of
// single additions, so the rounding does not depend on the column's position.
__device__ __forceinline__ float reduce_scatter(const float (&v)[4], int lane) {
    const bool hi = (lane & 32) != 0;
    const bool mid = (lane & 16) != 0;
    float k0 = hi ? v[2] : v[0];
    float k1 = hi ? v[3] : v[1];
    k0 += shfl_xor(hi ? v[0] : v[2], 32);
    k1 += shfl_xor(hi ? v[1] : v[3], 32);
    float kk = mid ? k1 : k0;
    kk += shfl_xor(mid ? k0 : k1, 16);
    return kk;
}

template <bool HIST, bool BMAX, bool SCORES = true, bool BKEYS = false>
__device__ __forceinline__ void store_step(const IndexParams& p, int r, int64_t nv, int64_t cb, int64_t c_end,
                                           int lane, const float (&v)[4], float sc, bool valid, float* srow,
                                           uint32_t* hist, uint32_t* bkl = nullptr, int64_t c0 = 0) {
    const float kk = reduce_scatter(v, lane);
    const int64_t c_out = cb + lane;
    const float score = valid ? sc * kk : kNegInf;
    if (c_out < c_end) {
        if (SCORES) srow[c_out] = score;
        if (HIST && valid) atomicAdd(&hist[order_key(score) >> 20], 1u);
    }
    if (BKEYS) {
        // Score-free mode: block keys only (the select counts them); a block
        // without valid columns has key 0.
        uint32_t bk = valid ? block_key(score) : 0u;
#pragma unroll
        for (int o = 1; o < kKeyBlock; o <<= 1) bk = max(bk, shfl_xor(bk, o));
        if ((lane & (kKeyBlock - 1)) == 0 && c_out < c_end) bkl[(c_out - c0) / kKeyBlock] = bk;
    }
    if (BMAX) {
        // Block score over bm_rows consecutive columns = lanes (blocks never
        // straddle a 64-column step): NaN as -inf, infinities clipped, invalid
        // columns -inf; the block of the newest visible row is pinned to +inf.
        float bm = valid ? pool_value(score) : kNegInf;
        for (int o = 1; o < p.bm_rows; o <<= 1) bm = fmaxf(bm, shfl_xor(bm, o));
        if ((lane & (p.bm_rows - 1)) == 0 && c_out < c_end) {
            const int64_t blk = c_out / p.bm_rows;
            p.block_max[(int64_t)r * p.bm_blocks + blk] = (blk == (nv - 1) / p.bm_rows) ? kPosInf : bm;
        }
    }
}

// Columns of a workgroup beyond the visible prefix: -inf scores, -inf block
// scores, empty (0) block keys.
template <bool BMAX, bool SCORES = true, bool BKEYS = false>
__device__ __forceinline__ void store_invisible(const IndexParams& p, int r, int64_t cb, int64_t c_end, int lane,
                                                float* srow, uint32_t* bkl = nullptr, int64_t c0 = 0) {
    const int64_t c_out = cb + lane;
    if (SCORES && c_out < c_end) srow[c_out] = kNegInf;
    if (BKEYS && (lane & (kKeyBlock - 1)) == 0 && c_out < c_end) bkl[(c_out - c0) / kKeyBlock] = 0u;
    if (BMAX && (lane & (p.bm_rows - 1)) == 0 && c_out < c_end)
        p.block_max[(int64_t)r * p.bm_blocks + c_out / p.bm_rows] = kNegInf;
}

}  // namespace

template <int KT, int HI, int DI, bool REINDEX, bool HIST, bool BMAX>
__global__ __launch_bounds__(256) void indexer_score_kernel(const IndexParams p) {
    // Per-workgroup histogram of the score keys' top 12 bits (one row per workgroup).
    __shared__ uint32_t hist[HIST ? kKeyBins : 1];
    typedef IdxOps<KT, DI> Ops;
    typedef typename Ops::Frag Frag;
    constexpr int HT = (HI + 15) / 16;  // 16-head MFMA tiles
    constexpr int S = Ops::kSteps;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int r = blockIdx.y;

    const int64_t nv = (p.pos[r] + 1) / p.ratio;
    const int64_t base = p.row_base[r];
    const int64_t c_begin = (int64_t)blockIdx.x * p.cols_per_wg;
    const int64_t c_end = c_begin + p.cols_per_wg < p.width ? c_begin + p.cols_per_wg : p.width;
    const int64_t c_live = REINDEX ? c_end : (nv < c_end ? nv : c_end);
    float* srow = p.scores + (int64_t)r * p.width;

    // Query fragments (A operands, heads as rows) and head weights, kept for the whole launch.
    Frag qa[HT][S];
    float wr[HT][4];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        const int h = 16 * t + li;
#pragma unroll
        for (int s = 0; s < S; ++s)
            qa[t][s] = (h < HI) ? Ops::load(p.q, (int64_t)r * HI + h, s, g) : Ops::zero();
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int hw = 16 * t + 4 * g + rr;
            wr[t][rr] = (hw < HI) ? p.w[(int64_t)r * HI + hw] : 0.f;
        }
    }
    bool qn = false;
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int s = 0; s < S; ++s) qn |= frag_has_nan(qa[t][s]);
    const float row_scale = __ballot(qn) != 0ull ? __builtin_nanf("") : p.scale;  // NaN query: NaN scores

    if (HIST) {
        for (int b = threadIdx.x; b < kKeyBins; b += 256) hist[b] = 0u;
        __syncthreads();
    }

    // One step = 64 consecutive columns of this wave: the key rows of 4 tiles of
    // 16 (B operands) and the output column's scale.  Steps are software
    // pipelined: the next step's loads are issued before this step's MFMAs.
    struct Step {
        Frag kb[4][S];
        float sc;     // score scale of this lane's output column
        bool valid;   // this lane's output column is valid
    };
    auto issue = [&](int64_t cb, Step& st) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t c = cb + 16 * u + li;
            int64_t prow = 0;
            const bool valid = (c < c_end) && column_row<REINDEX>(p, r, c, nv, base, prow);
#pragma unroll
            for (int s = 0; s < S; ++s) st.kb[u][s] = valid ? Ops::load(p.k, prow, s, g) : Ops::zero();
        }
        const int64_t c_out = cb + lane;
        int64_t prow = 0;
        st.valid = (c_out < c_end) && column_row<REINDEX>(p, r, c_out, nv, base, prow);
        st.sc = row_scale;
        if (KT == CSA2_FP8_E4M3 && st.valid) st.sc *= p.k_scale[prow];
    };
    auto finish = [&](int64_t cb, const Step& st) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float acc_sum = 0.f;
#pragma unroll
            for (int t = 0; t < HT; ++t) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < S; ++s) acc = Ops::mma(acc, qa[t][s], st.kb[u][s]);
                if (t == 0) acc_sum = nan_guard(acc[0]);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc_sum += wr[t][rr] * relu_bits(acc[rr]);
            }
            v[u] = acc_sum;
        }
        store_step<HIST, BMAX>(p, r, nv, cb, c_end, lane, v, st.sc, st.valid, srow, hist);
    };

    int64_t cb = c_begin + 64 * wave;
    Step A, B;
    if (cb < c_live) issue(cb, A);
    while (cb < c_live) {
        if (cb + 256 < c_live) issue(cb + 256, B);
        finish(cb, A);
        cb += 256;
        if (cb >= c_live) break;
        if (cb + 256 < c_live) issue(cb + 256, A);
        finish(cb, B);
        cb += 256;
    }
    for (; cb < c_end; cb += 256) store_invisible<BMAX>(p, r, cb, c_end, lane, srow);  // nothing visible here
    if (HIST) {
        __syncthreads();
        uint32_t* gh = p.key_hist + (int64_t)r * kKeyBins;
        for (int b = threadIdx.x; b < kKeyBins; b += 256)
            if (hist[b]) atomicAdd(&gh[b], hist[b]);
    }
}

// ---------------------------------------------------------------------------
// FULL rows that share one BF16 plane (64 heads x 128), as in a prefill chunk.
// Every row reads the same key rows, so a workgroup of 8 waves takes 8 query
// rows -- one per wave, its 64 heads x 128 held in registers as A operands as
// in indexer_score_kernel -- and streams its column range through LDS in
// stages of 64 key rows: each stage is read from memory once and feeds all 8
// rows (indexer_score_kernel re-reads every key row for every query row).
// Consecutive workgroup ids take consecutive row groups of one column range,
// so the workgroups resident together share that range's key rows in L2.
// Per column the arithmetic is that of indexer_score_kernel (the same MFMA
// chains and head reduction), so the scores are identical.
constexpr int kChunkRows = 8;       // query rows per workgroup, one per wave
constexpr int kChunkKeys = 128;     // key rows per LDS stage (64 measured ~3 % slower)

// LDS byte offset of 16-byte chunk c (0..15) of staged key row k: rows are 256
// bytes, the chunk index XOR-ed with the row's low 4 bits.  A B-operand read
// (16 rows, 4 chunks) is then free of bank conflicts; padded rows (a stride of
// 272 bytes) measured 2.7 conflict cycles per LDS cycle with rocprofv3.
__device__ __forceinline__ int stage_off(int k, int c) { return 256 * k + 16 * (c ^ (k & 15)); }

// Output of one 64-column step of the chunk kernel: the scores, or (BK, score-free mode) only the block
// key of each 8 columns -- the largest order key of the valid ones, NaN as kNanBlockKey, 0 for none.
template <bool BK>
__device__ __forceinline__ void chunk_store(const IndexParams& p, int r, int64_t nv, int64_t cb, int64_t c_end,
                                            int lane, const float (&v)[4], float sc, bool valid, float* srow) {
    if constexpr (!BK) {
        store_step<false, false>(p, r, nv, cb, c_end, lane, v, sc, valid, srow, nullptr);
    } else {
        const float kk = reduce_scatter(v, lane);
        const float score = valid ? sc * kk : kNegInf;
        uint32_t bk = valid ? block_key(score) : 0u;
#pragma unroll
        for (int o = 1; o < kKeyBlock; o <<= 1) bk = max(bk, shfl_xor(bk, o));
        const int64_t c_out = cb + lane;
        if ((lane & (kKeyBlock - 1)) == 0 && c_out < c_end)
            p.block_keys[(int64_t)r * ((p.width + kKeyBlock - 1) / kKeyBlock) + c_out / kKeyBlock] = bk;
    }
}

template <bool BK>
__device__ __forceinline__ void chunk_store_invisible(const IndexParams& p, int r, int64_t cb, int64_t c_end, int lane,
                                                      float* srow) {
    if constexpr (!BK) {
        store_invisible<false>(p, r, cb, c_end, lane, srow);
    } else {
        const int64_t c_out = cb + lane;
        if ((lane & (kKeyBlock - 1)) == 0 && c_out < c_end)
            p.block_keys[(int64_t)r * ((p.width + kKeyBlock - 1) / kKeyBlock) + c_out / kKeyBlock] = 0u;
    }
}

template <int ROWS, int KEYS, bool BK>
__global__ __launch_bounds__(64 * ROWS) void indexer_chunk_kernel(const IndexParams p, int rows) {
    typedef IdxOps<CSA2_BF16, 128> Ops;
    typedef Ops::Frag Frag;
    constexpr int HT = 4, S = Ops::kSteps;
    constexpr int NT = 64 * ROWS;
    constexpr int NCH = KEYS * 16 / NT;  // 16-byte chunks each thread stages
    static_assert(KEYS % 64 == 0 && NCH * NT == KEYS * 16, "whole 64-column steps, whole chunks per thread");
    __shared__ __attribute__((aligned(16))) uint8_t tile[2][KEYS * 256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int r0 = blockIdx.x * ROWS;
    const int r = r0 + wave;
    const bool live = r < rows;
    const int rq = live ? r : rows - 1;  // an idle wave (past the last row) still stages tiles
    const int64_t base = p.row_base[0];
    const int64_t nv = (p.pos[rq] + 1) / p.ratio;
    int64_t nvg = 0;  // columns some row of the group sees
    for (int j = 0; j < ROWS; ++j) {
        const int64_t v = (p.pos[min(r0 + j, rows - 1)] + 1) / p.ratio;
        nvg = v > nvg ? v : nvg;
    }
    const int64_t c0 = (int64_t)blockIdx.y * p.cols_per_wg;
    const int64_t c1 = c0 + p.cols_per_wg < p.width ? c0 + p.cols_per_wg : p.width;
    const int64_t c_live = nvg < c1 ? nvg : c1;
    float* srow = BK ? nullptr : p.scores + (int64_t)rq * p.width;

    Frag qa[HT][S];
    float wr[HT][4];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
#pragma unroll
        for (int s = 0; s < S; ++s) qa[t][s] = Ops::load(p.q, (int64_t)rq * 64 + 16 * t + li, s, g);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) wr[t][rr] = p.w[(int64_t)rq * 64 + 16 * t + 4 * g + rr];
    }
    wait_vmem_all();  // q and w are in registers before the staging loop starts loading
    bool qn = false;
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int s = 0; s < S; ++s) qn |= frag_has_nan(qa[t][s]);
    const float row_scale = __ballot(qn) != 0ull ? __builtin_nanf("") : p.scale;  // NaN query: NaN scores

    // Staging: chunk i = thread + NT j of the stage is 16-byte chunk i % 16 of key row i / 16
    // (consecutive threads read consecutive bytes; zeros past the visible columns).
    auto fetch = [&](int64_t cs, u32x4 (&x)[NCH]) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int ci = threadIdx.x + NT * j;
            const int64_t c = cs + ci / 16;
            x[j] = u32x4{0u, 0u, 0u, 0u};
            if (c < c_live) x[j] = ld16(reinterpret_cast<const uint8_t*>(p.k) + (base + c) * 256 + 16 * (ci % 16));
        }
    };
    auto put = [&](int b, const u32x4 (&x)[NCH]) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int ci = threadIdx.x + NT * j;
            *reinterpret_cast<u32x4*>(tile[b] + stage_off(ci / 16, ci % 16)) = x[j];
        }
    };

    int64_t cs = c0;
    int b = 0;
    if (cs < c_live) {
        u32x4 x[NCH];
        fetch(cs, x);
        put(0, x);
    }
    __syncthreads();
    for (; cs < c_live; cs += KEYS) {
        // The next stage's loads are in flight while this stage is computed.  After the last
        // stage this fetches nothing and stages zeros: unconditional, so the compiler's wait
        // insertion sees every staged value consumed before the next fetch.
        u32x4 x[NCH];
        fetch(cs + KEYS, x);
        float vlast[4];  // the stage's last 64 scores, stored after the staging writes (below)
        if (live) {
            const uint8_t* tb = tile[b];
            // B operands of the next 16 keys are read from LDS while this 16 keys' MFMAs run
            auto read_kb = [&](int kk, Frag (&kb)[S]) {
#pragma unroll
                for (int s = 0; s < S; ++s)
                    kb[s] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(tb + stage_off(kk + li, 4 * s + g)));
            };
            Frag kn[S];
            read_kb(0, kn);
#pragma unroll
            for (int st = 0; st < KEYS / 64; ++st) {
                float v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    Frag kb[S];
#pragma unroll
                    for (int s = 0; s < S; ++s) kb[s] = kn[s];
                    if (64 * st + 16 * u + 16 < KEYS) read_kb(64 * st + 16 * u + 16, kn);
                    float acc_sum = 0.f;
#pragma unroll
                    for (int t = 0; t < HT; ++t) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < S; ++s) acc = Ops::mma(acc, qa[t][s], kb[s]);
                        if (t == 0) acc_sum = nan_guard(acc[0]);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) acc_sum += wr[t][rr] * relu_bits(acc[rr]);
                    }
                    v[u] = acc_sum;
                }
                if (st + 1 < KEYS / 64) {
                    const int64_t cb = cs + 64 * st;
                    const int64_t c_out = cb + lane;
                    chunk_store<BK>(p, rq, nv, cb, c1, lane, v, row_scale, c_out < c1 && c_out < nv, srow);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) vlast[u] = v[u];
                }
            }
        }
        // The staging writes wait for the next stage's loads; the score stores issued after them
        // (the stage's last step) are then not waited for before the barrier.
        put(b ^ 1, x);
        if (live) {
            const int64_t cb = cs + KEYS - 64;
            const int64_t c_out = cb + lane;
            chunk_store<BK>(p, rq, nv, cb, c1, lane, vlast, row_scale, c_out < c1 && c_out < nv, srow);
        }
        __syncthreads();
        b ^= 1;
    }
    if (live)
        for (; cs < c1; cs += 64) chunk_store_invisible<BK>(p, rq, cs, c1, lane, srow);  // nothing visible here
}

// Steps of key-row loads each wave keeps in flight in the streaming FULL
// kernels, and the most 64-column steps one wave makes (a workgroup covers
// <= 4096 columns).
constexpr int kStreamDepth = 2;
constexpr int kStreamMaxSteps = 16;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9-family descriptor
constexpr int kNT = 2;                  // non-temporal cache policy of a buffer load

// ---- 64-key steps of a quantised index plane, staged through LDS ---------------
//
// A step is 64 consecutive key rows.  Lane l's 16-byte load j covers key
// j * (64 / kLoads) + l / kChunks, chunk l % kChunks, so one load instruction
// reads 1 KiB of whole rows.  In LDS, chunk c of key kk sits at position
// c ^ swz(kk) of the key's row, which keeps both the writes and the MFMA-layout
// reads free of bank conflicts.  Each lane also loads the 32-bit scale word of
// key (step start + lane).  The same code serves the scoring pass and the
// re-scoring of candidates, so both compute a column's score identically.

// FP8-E4M3 keys: 128-byte rows, one float32 scale per key that multiplies the
// score (scales are positive and ReLU commutes with a positive factor).  The
// FP8 query's per-(row, head) scale is folded into w by the caller.  One
// 16x16x128 MFMA with unit block scales per 16 keys x 16 heads; lane (g, n)
// holds bytes 16g..16g+15 and 64+16g..64+16g+15 of its row (the query
// fragments use the same k order).
struct Fp8Keys {
    static constexpr int kRowBytes = 128, kChunks = 8, kLoads = 8;
    static constexpr bool kScaleInScore = true;
    static constexpr bool kDense = false;
    static __device__ __forceinline__ int swz(int kk) { return (kk >> 1) & 7; }
    static __device__ __forceinline__ void frag(const uint8_t* my, const uint32_t*, int kk, int g, i32x8& kb,
                                                uint32_t& ksc) {
        const int sw = swz(kk);
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(my + kk * 128 + 16 * (g ^ sw));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(my + kk * 128 + 16 * ((g + 4) ^ sw));
        kb[0] = a0[0]; kb[1] = a0[1]; kb[2] = a0[2]; kb[3] = a0[3];
        kb[4] = a1[0]; kb[5] = a1[1]; kb[6] = a1[2]; kb[7] = a1[3];
        ksc = 127u;
    }
    static __device__ __forceinline__ f32x4 mma(const i32x8& qa, uint32_t, const i32x8& kb, uint32_t) {
        return mma_fp8_k128(f32x4{0.f, 0.f, 0.f, 0.f}, qa, kb);
    }
    static __device__ __forceinline__ void query(const IndexParams& p, int64_t head, int g, i32x8& qa, uint32_t& qs) {
        qa = IdxOps<CSA2_FP8_E4M3, 128>::load(p.q, head, 0, g);
        qs = 127u;
    }
    static __device__ __forceinline__ const void* scale_base(const IndexParams& p, int64_t row) {
        return p.k_scale + row;
    }
    // Factor of the output column's score: the key row's float32 scale (a NaN scale makes the
    // score NaN, as the decoded row is NaN).
    static __device__ __forceinline__ float score_scale(float scale, uint32_t sw, bool q_nan) {
        return q_nan ? __builtin_nanf("") : scale * __uint_as_float(sw);
    }
    // Whether the query row holds an E4M3 NaN code (the lanes together hold all of it).
    static __device__ __forceinline__ bool query_nan(const i32x8 (&qa)[4], const uint32_t (&)[4]) {
        return __ballot(frag_has_nan(qa[0]) || frag_has_nan(qa[1]) || frag_has_nan(qa[2]) ||
                        frag_has_nan(qa[3])) != 0ull;
    }
};

// MXFP4 keys and query (E2M1 with one E8M0 scale per 32 elements): 64-byte
// rows plus a 4-byte word of block scales per row.  The MFMA takes FP4
// operands with their block scales directly: lane (g, n) holds elements
// 32g..32g+31 (16 bytes, operand dwords 0-3) of row n and that block's scale
// byte.
struct Fp4Keys {
    static constexpr int kRowBytes = 64, kChunks = 4, kLoads = 4;
    static constexpr bool kScaleInScore = false;
    static constexpr bool kDense = false;
    static __device__ __forceinline__ int swz(int kk) { return (kk >> 2) & 3; }
    static __device__ __forceinline__ void frag(const uint8_t* my, const uint32_t* scl, int kk, int g, i32x8& kb,
                                                uint32_t& ksc) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(my + kk * 64 + 16 * (g ^ swz(kk)));
        kb[0] = a[0]; kb[1] = a[1]; kb[2] = a[2]; kb[3] = a[3];
        kb[4] = 0; kb[5] = 0; kb[6] = 0; kb[7] = 0;
        ksc = (scl[kk] >> (8 * g)) & 0xffu;
    }
    static __device__ __forceinline__ f32x4 mma(const i32x8& qa, uint32_t qs, const i32x8& kb, uint32_t ksc) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, kb, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, (int)qs,
                                                                0, (int)ksc);
    }
    static __device__ __forceinline__ void query(const IndexParams& p, int64_t head, int g, i32x8& qa, uint32_t& qs) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(p.q) + head * 64 + 16 * g);
        qa[0] = a[0]; qa[1] = a[1]; qa[2] = a[2]; qa[3] = a[3];
        qa[4] = 0; qa[5] = 0; qa[6] = 0; qa[7] = 0;
        qs = p.q_e8[head * 4 + g];
    }
    static __device__ __forceinline__ const void* scale_base(const IndexParams& p, int64_t row) {
        return p.k_e8 + 4 * row;
    }
    // E8M0 byte 255 encodes NaN: a key with a NaN block scale has a NaN dot with every head, and
    // a query with one has a NaN dot in that head for every key, so the score is NaN either
    // way.  Set here explicitly rather than left to how the matrix core treats a NaN scale.
    static __device__ __forceinline__ float score_scale(float scale, uint32_t sw, bool q_nan) {
        const uint32_t ff = ~sw;  // a byte of sw is 0xff iff that byte of ff is zero
        const bool k_nan = ((ff - 0x01010101u) & ~ff & 0x80808080u) != 0u;
        return (k_nan || q_nan) ? __builtin_nanf("") : scale;
    }
    // Whether any E8M0 scale of the query row is 255 (the lanes together hold all of them).
    static __device__ __forceinline__ bool query_nan(const i32x8 (&)[4], const uint32_t (&qs)[4]) {
        return __ballot(qs[0] == 255u || qs[1] == 255u || qs[2] == 255u || qs[3] == 255u) != 0ull;
    }
};

template <class KF>
__device__ __forceinline__ void stage_put(uint8_t* my, uint32_t* scl, const u32x4 (&v)[KF::kLoads], uint32_t sw,
                                          int lane) {
#pragma unroll
    for (int j = 0; j < KF::kLoads; ++j) {
        const int kk = j * (64 / KF::kLoads) + lane / KF::kChunks;
        *reinterpret_cast<u32x4*>(my + kk * KF::kRowBytes + 16 * ((lane % KF::kChunks) ^ KF::swz(kk))) = v[j];
    }
    if (!KF::kScaleInScore) scl[lane] = sw;
}

// v[u] (lane (g, n)): sum over heads 4g..4g+3 of every 16-head tile t of
// w * ReLU(q . k) for key 16u + n of the staged step.
template <class KF>
__device__ __forceinline__ void step_sums(const uint8_t* my, const uint32_t* scl, const i32x8 (&qa)[4],
                                          const uint32_t (&qs)[4], const float (&wr)[4][4], int g, int li,
                                          float (&v)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        i32x8 kb;
        uint32_t ksc;
        KF::frag(my, scl, 16 * u + li, g, kb, ksc);
        float acc_sum = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const f32x4 acc = KF::mma(qa[t], qs[t], kb, ksc);
            if (t == 0) acc_sum = nan_guard(acc[0]);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc_sum = fmaf(wr[t][rr], relu_bits(acc[rr]), acc_sum);
        }
        v[u] = acc_sum;
    }
}

// Query fragments (A operands: heads as rows, 16 per tile), their block scales
// and the head weights of query row r (64 heads).
template <class KF>
__device__ __forceinline__ void load_query(const IndexParams& p, int r, int g, int li, i32x8 (&qa)[4],
                                           uint32_t (&qs)[4], float (&wr)[4][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        KF::query(p, (int64_t)r * 64 + 16 * t + li, g, qa[t], qs[t]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) wr[t][rr] = p.w[(int64_t)r * 64 + 16 * t + 4 * g + rr];
    }
}

// FULL scoring of a quantised plane (64 heads x 128) with coalesced,
// non-temporal key-row loads.
//
// A FULL row's key rows are contiguous in the plane, so a wave's 64-key step is
// one contiguous span (8 KiB FP8, 4 KiB MXFP4), loaded as whole 128-byte lines
// (non-temporal: each byte is read once), staged in the wave's LDS slot and
// read back in the MFMA operand layout.  Loads go through buffer descriptors
// that cover exactly the workgroup's visible key rows and their scales: a load
// past the visible prefix returns zeros instead of touching memory, so no
// address is clamped and no branch guards a load (a branch there made the
// compiler drain every outstanding load at the join).  The per-lane offset is
// fixed for the launch and the step offset is a scalar.  DEPTH steps of loads
// are in flight per wave while the matrix cores work on the step in LDS.
template <class KF, bool HIST, bool BMAX, int DEPTH, bool SCORES, bool BKEYS>
__global__ __launch_bounds__(256) void indexer_stream_kernel(const IndexParams p) {
    __shared__ uint32_t hist[HIST ? kKeyBins : 1];
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][64 * KF::kRowBytes];
    __shared__ uint32_t scl_all[4][KF::kScaleInScore ? 1 : 64];
    __shared__ __attribute__((aligned(16))) uint32_t bkl[BKEYS ? 256 * kStreamMaxSteps / kKeyBlock : 1];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int li = lane & 15;
    const int r = blockIdx.y;

    const int64_t nv = uniform64((p.pos[r] + 1) / p.ratio);
    const int64_t base = uniform64(p.row_base[r]);
    const int64_t c_begin = (int64_t)blockIdx.x * p.cols_per_wg;
    const int64_t c_end = c_begin + p.cols_per_wg < p.width ? c_begin + p.cols_per_wg : p.width;
    const int64_t c_live = nv < c_end ? nv : c_end;
    float* srow = p.scores + (int64_t)r * p.width;
    uint8_t* my = stage[wave];
    uint32_t* scl = scl_all[wave];

    i32x8 qa[4];
    uint32_t qs[4];
    float wr[4][4];
    load_query<KF>(p, r, g, li, qa, qs, wr);
    const bool q_nan = KF::query_nan(qa, qs);
    if (HIST) {
        for (int b = threadIdx.x; b < kKeyBins; b += 256) hist[b] = 0u;
        __syncthreads();
    }

    // Descriptors over this workgroup's visible rows [c_begin, c_live).
    const int n_live = c_live > c_begin ? (int)(c_live - c_begin) : 0;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.k) + (base + c_begin) * KF::kRowBytes), (short)0,
        n_live * KF::kRowBytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(KF::scale_base(p, base + c_begin)), (short)0, n_live * 4, kRsrcWord3);
    const int voff = (lane / KF::kChunks) * KF::kRowBytes + (lane % KF::kChunks) * 16;

    struct Buf {
        u32x4 v[KF::kLoads];
        uint32_t sw;  // scale word of key (step start + lane)
    };
    auto issue = [&](int64_t cb, Buf& b) {
        const int so = (int)(cb - c_begin) * KF::kRowBytes;
#pragma unroll
        for (int j = 0; j < KF::kLoads; ++j)
            b.v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, voff, so + 1024 * j, kNT));
        b.sw = __builtin_amdgcn_raw_buffer_load_b32(srs, lane * 4, (int)(cb - c_begin) * 4, 0);
    };
    auto step = [&](int64_t cb, Buf& b) {
        stage_put<KF>(my, scl, b.v, b.sw, lane);
        const float sc = KF::score_scale(p.scale, b.sw, q_nan);
        const bool valid = cb + lane < c_live;
        // Unconditional: past the visible rows the descriptor turns the loads into zeros.
        issue(cb + 256 * DEPTH, b);
        float v[4];
        step_sums<KF>(my, scl, qa, qs, wr, g, li, v);
        store_step<HIST, BMAX, SCORES, BKEYS>(p, r, nv, cb, c_end, lane, v, sc, valid, srow, hist, bkl, c_begin);
    };

    // At most kStreamMaxSteps steps per wave: the step loop is unrolled
    // completely, so the compiler's memory-counter waits see the loads in
    // flight exactly instead of draining them at a loop back edge.
    const int64_t cb0 = c_begin + 64 * wave;
    Buf bufs[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(cb0 + 256 * d, bufs[d]);
#pragma unroll
    for (int it = 0; it < kStreamMaxSteps; ++it) {
        const int64_t cb = cb0 + 256 * it;
        if (cb >= c_live) break;
        step(cb, bufs[it % DEPTH]);
    }
    int64_t cb = cb0;
    if (c_live > cb0) cb += 256 * ((c_live - cb0 + 255) / 256);
    for (; cb < c_end; cb += 256) store_invisible<BMAX, SCORES, BKEYS>(p, r, cb, c_end, lane, srow, bkl, c_begin);
    if (BKEYS) {  // the workgroup's block keys in one contiguous burst (32-bit, or their top 16 bits)
        __syncthreads();
        const int nbk = (int)((c_end - c_begin + kKeyBlock - 1) / kKeyBlock);
        const int64_t at = (int64_t)r * ((p.width + kKeyBlock - 1) / kKeyBlock) + c_begin / kKeyBlock;
        if (p.bk16 && (at & 1) == 0) {  // pairs of keys as 32-bit stores
            uint32_t* gk = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.block_keys) + at);
            for (int i = threadIdx.x; 2 * i < nbk; i += 256) {
                if (2 * i + 1 < nbk)
                    __builtin_nontemporal_store((bkl[2 * i] >> 16) | (bkl[2 * i + 1] & 0xffff0000u), gk + i);
                else
                    __builtin_nontemporal_store((uint16_t)(bkl[2 * i] >> 16), reinterpret_cast<uint16_t*>(gk + i));
            }
        } else if (p.bk16) {
            uint16_t* gk = reinterpret_cast<uint16_t*>(p.block_keys) + at;
            for (int i = threadIdx.x; i < nbk; i += 256) __builtin_nontemporal_store((uint16_t)(bkl[i] >> 16), gk + i);
        } else {
            uint32_t* gk = p.block_keys + at;
            for (int i = threadIdx.x; i < nbk; i += 256) __builtin_nontemporal_store(bkl[i], gk + i);
        }
    }
    if (HIST) {
        __syncthreads();
        uint32_t* gh = p.key_hist + (int64_t)r * kKeyBins;
        for (int b = threadIdx.x; b < kKeyBins; b += 256)
            if (hist[b]) atomicAdd(&gh[b], hist[b]);
    }
}

// Re-scoring for the top-k of FULL scores that were never written.
//
// Segment seg of row r covers columns [seg * chunk, (seg + 1) * chunk).  b1[r]
// is the bin holding the row's k-th largest block key (the select counts the
// block keys the score-free pass wrote).  The k blocks with the largest keys hold k distinct
// columns with keys in bins >= b1, so the row's k-th largest column key is in
// a bin >= b1 too: every selected column has a key in bin >= b1, and so has
// the largest key of its kKeyBlock-column block.  One wave handles one segment on its own (no
// barriers).  It loads the block keys of up to kRescoreGroups x 256 blocks at once, before its
// query (lane l of group i holds blocks 256 i + 4 l .. 256 i + 4 l + 3), queues in column order
// the blocks whose key reaches bin b1 in an LDS list (each lane's place from a wave prefix sum of
// the lanes' counts), then re-scores the queue 8 blocks (one 64-key step) at a time with exactly
// the scoring pass's arithmetic, appending the (key, column) pairs of valid columns in bins >= b1,
// in column order, to the segment's list (capacity chunk, so it never overflows).  Segments with
// more than kRescoreQueue queued blocks (heavy ties) queue and re-score one group at a time.
// seg_count gets the list length.
constexpr int kRescoreGroups = 8;    // groups of 256 blocks whose keys are loaded together
constexpr int kRescoreQueue = 256;   // queued blocks per wave (one group always fits)

// The four block keys of lanes' group slot (as 32-bit keys; 16-bit keys are their top halves), and a
// bit per key whose block is queued.  VEC: one 8- or 16-byte load (the row's keys are a multiple of 4
// long and 16-byte aligned); otherwise four loads.  Blocks past blk_hi read as 0 (not queued); the
// load itself stays inside the row.
template <bool BK16, bool VEC>
__device__ __forceinline__ void rescore_load_keys(const uint32_t* bkeys, const uint16_t* bkeys16, int64_t b,
                                                  int64_t blk_hi, int64_t nbk_row, uint32_t (&raw)[BK16 ? 2 : 4]) {
    if constexpr (VEC) {
        const int64_t bq = b + 4 <= nbk_row ? b : nbk_row - 4;
        if constexpr (BK16) {
            const uint2 v = *reinterpret_cast<const uint2*>(bkeys16 + bq);
            raw[0] = v.x; raw[1] = v.y;
        } else {
            const u32x4 v = *reinterpret_cast<const u32x4*>(bkeys + bq);
            raw[0] = v[0]; raw[1] = v[1]; raw[2] = v[2]; raw[3] = v[3];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t bc = b + e < blk_hi ? b + e : blk_hi - 1;
            if constexpr (BK16) {
                const uint32_t k = bkeys16[bc];
                if (e & 1) raw[e >> 1] |= k << 16;
                else raw[e >> 1] = k;
            } else {
                raw[e] = bkeys[bc];
            }
        }
    }
}

template <bool BK16>
__device__ __forceinline__ uint32_t rescore_take(const uint32_t (&raw)[BK16 ? 2 : 4], int64_t b, int64_t blk_hi,
                                                 uint32_t b1) {
    uint32_t tk = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t k = BK16 ? (e & 1 ? raw[e >> 1] & 0xffff0000u : raw[e >> 1] << 16) : raw[e];
        if (b + e < blk_hi && k != 0u && (k >> 20) >= b1) tk |= 1u << e;
    }
    return tk;
}

// Appends the queued blocks of one group (tk: this lane's bits for blocks b .. b + 3) to q8 at n_q, in
// column order, and returns how many the wave queued.  Each lane's place is the number of queued
// blocks of the lanes before it: the prefix sum of the lane counts (0..4) from their three bit planes.
__device__ __forceinline__ int rescore_queue(int32_t* q8, int n_q, uint32_t tk, int64_t b) {
    const uint32_t c = (uint32_t)__builtin_popcount(tk);
    const uint64_t m0 = __ballot(c & 1u), m1 = __ballot(c & 2u), m2 = __ballot(c & 4u);
    auto below = [](uint64_t m) {
        return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    };
    int at = n_q + (int)(below(m0) + 2u * below(m1) + 4u * below(m2));
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (tk & (1u << e)) q8[at++] = (int32_t)(b + e);
    return __builtin_popcountll(m0) + 2 * __builtin_popcountll(m1) + 4 * __builtin_popcountll(m2);
}

template <class KF, bool BK16, bool VEC>
__global__ __launch_bounds__(256) void indexer_rescore_kernel(const IndexParams p, const uint32_t* b1_in, int chunk,
                                                              int nseg, uint32_t* cand_keys, int32_t* cand_cols,
                                                              uint32_t* seg_count) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][64 * KF::kRowBytes];
    __shared__ uint32_t scl_all[4][KF::kScaleInScore ? 1 : 64];
    __shared__ int32_t queue[4][kRescoreQueue];
    constexpr int KW = BK16 ? 2 : 4;  // dwords of a lane's four keys
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int r = blockIdx.y;
    const int seg = 4 * blockIdx.x + wave;
    if (seg >= nseg) return;  // no barriers in this kernel: waves are independent

    const int64_t nv = uniform64((p.pos[r] + 1) / p.ratio);
    const int64_t base = uniform64(p.row_base[r]);
    const int64_t n_valid = nv < p.width ? nv : p.width;
    const uint32_t b1 = __builtin_amdgcn_readfirstlane(b1_in[r]);
    const int64_t c_lo = (int64_t)seg * chunk;
    const int64_t c_hi = c_lo + chunk < n_valid ? c_lo + chunk : n_valid;
    if (c_hi <= c_lo) {  // nothing visible in this segment
        if (lane == 0) seg_count[(int64_t)r * nseg + seg] = 0u;
        return;
    }
    const int64_t nbk_row = (p.width + kKeyBlock - 1) / kKeyBlock;
    const uint32_t* bkeys = p.block_keys + (int64_t)r * nbk_row;
    const uint16_t* bkeys16 = reinterpret_cast<const uint16_t*>(p.block_keys) + (int64_t)r * nbk_row;
    const int64_t blk_lo = c_lo / kKeyBlock, blk_hi = (c_hi + kKeyBlock - 1) / kKeyBlock;
    uint32_t* okeys = cand_keys + ((int64_t)r * nseg + seg) * chunk;
    int32_t* ocols = cand_cols + ((int64_t)r * nseg + seg) * chunk;
    uint8_t* my = stage[wave];
    uint32_t* scl = scl_all[wave];
    int32_t* q8 = queue[wave];

    // The first keys are in flight before the query is loaded: queueing needs only the keys.
    uint32_t raw[kRescoreGroups][KW];
#pragma unroll
    for (int i = 0; i < kRescoreGroups; ++i)
        rescore_load_keys<BK16, VEC>(bkeys, bkeys16, blk_lo + 256 * i + 4 * lane, blk_hi, nbk_row, raw[i]);

    i32x8 qa[4];
    uint32_t qs[4];
    float wr[4][4];
    load_query<KF>(p, r, g, li, qa, qs, wr);
    const bool q_nan = KF::query_nan(qa, qs);
    // the row's visible key rows and their scales; loads beyond them return zeros
    const int n_rows = (int)n_valid;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.k) + base * KF::kRowBytes), (short)0,
        n_rows * KF::kRowBytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(KF::scale_base(p, base)), (short)0, n_rows * 4, kRsrcWord3);

    uint32_t n_out = 0;
    // A step re-scores queued blocks head .. head+cnt-1 (cnt 1..8) and appends their candidates.  Its
    // loads (issue) and its arithmetic (finish) are separate so that the next step's key rows are in
    // flight while a step is computed; two register sets alternate (no copy between them, which would
    // wait for the loads).
    struct StepLoads {
        u32x4 buf[KF::kLoads];
        uint32_t sw;
    };
    auto issue = [&](int head, int cnt, StepLoads& L) {
#pragma unroll
        for (int j = 0; j < KF::kLoads; ++j) {
            // key kk of the step = row kk % 8 of queued block kk / 8; past the queue: an
            // offset beyond the descriptor -> zeros
            const int kk = j * (64 / KF::kLoads) + lane / KF::kChunks;
            const int blk = kk >> 3;
            const int row = blk < cnt ? q8[head + blk] * kKeyBlock + (kk & 7) : n_rows;
            L.buf[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     krs, row * KF::kRowBytes + 16 * (lane % KF::kChunks), 0, kNT));
        }
        const int my_blk = lane / kKeyBlock;
        const int64_t col = my_blk < cnt
            ? (int64_t)q8[head + my_blk] * kKeyBlock + (lane % kKeyBlock) : n_valid;
        L.sw = __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(col < n_valid ? col : n_valid) * 4, 0, 0);
    };
    auto finish = [&](int head, int cnt, const StepLoads& L) {
        const int my_blk = lane / kKeyBlock;
        const int64_t col = my_blk < cnt
            ? (int64_t)q8[head + my_blk] * kKeyBlock + (lane % kKeyBlock) : n_valid;
        stage_put<KF>(my, scl, L.buf, L.sw, lane);
        float v[4];
        step_sums<KF>(my, scl, qa, qs, wr, g, li, v);
        const float kk = reduce_scatter(v, lane);
        const bool valid = col < n_valid;
        const float sc = KF::score_scale(p.scale, L.sw, q_nan);
        const uint32_t key = order_key(sc * kk);
        const bool take = valid && (key >> 20) >= b1;
        const uint64_t m = __ballot(take);
        if (take) {
            const uint32_t at = n_out + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            okeys[at] = key;
            ocols[at] = (int32_t)col;
        }
        n_out += (uint32_t)__builtin_popcountll(m);
    };
    StepLoads la, lb;
    // Re-scores queue entries 0 .. n_q - 1.  The first four steps run straight-line with the next
    // step's loads in flight: every issue is unconditional (an empty step's loads fall past the
    // descriptors and return zeros) so the loads keep one order on every path and the compiler waits
    // for exactly the older step; only the arithmetic is skipped for empty steps.  (In a loop the
    // compiler loses that order at the back edge and waits for both steps.)  Further steps, rare, run
    // one at a time.
    auto drain = [&](int n_q) {
        auto cnt_at = [&](int h) { return n_q - h < 8 ? n_q - h : 8; };  // <= 0: an empty step
        issue(0, cnt_at(0), la);
        issue(8, cnt_at(8), lb);
        if (n_q > 0) finish(0, cnt_at(0), la);
        issue(16, cnt_at(16), la);
        if (n_q > 8) finish(8, cnt_at(8), lb);
        issue(24, cnt_at(24), lb);
        if (n_q > 16) finish(16, cnt_at(16), la);
        if (n_q > 24) finish(24, cnt_at(24), lb);
        for (int h = 32; h < n_q; h += 8) {
            issue(h, cnt_at(h), la);
            finish(h, cnt_at(h), la);
        }
    };

    for (int64_t b0 = blk_lo;;) {
        uint32_t tk[kRescoreGroups];
        int total = 0;
#pragma unroll
        for (int i = 0; i < kRescoreGroups; ++i) {
            tk[i] = rescore_take<BK16>(raw[i], b0 + 256 * i + 4 * lane, blk_hi, b1);
            total += (int)__builtin_popcount(tk[i]);
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) total += (int)shfl_xor((uint32_t)total, o);
        total = __builtin_amdgcn_readfirstlane(total);
        if (total <= kRescoreQueue) {  // the usual case: one queue for all groups
            int n_q = 0;
#pragma unroll
            for (int i = 0; i < kRescoreGroups; ++i) n_q += rescore_queue(q8, n_q, tk[i], b0 + 256 * i + 4 * lane);
            drain(n_q);
        } else {  // heavy ties: a group at a time, its keys read again
            for (int i = 0; i < kRescoreGroups; ++i) {
                uint32_t rw[KW];
                const int64_t b = b0 + 256 * i + 4 * lane;
                rescore_load_keys<BK16, VEC>(bkeys, bkeys16, b, blk_hi, nbk_row, rw);
                drain(rescore_queue(q8, 0, rescore_take<BK16>(rw, b, blk_hi, b1), b));
            }
        }
        b0 += 256 * kRescoreGroups;
        if (b0 >= blk_hi) break;
#pragma unroll
        for (int i = 0; i < kRescoreGroups; ++i)
            rescore_load_keys<BK16, VEC>(bkeys, bkeys16, b0 + 256 * i + 4 * lane, blk_hi, nbk_row, raw[i]);
    }
    if (lane == 0) seg_count[(int64_t)r * nseg + seg] = n_out;
}

template <class KF, bool BK16>
static void launch_rescore_kf(const IndexParams& p, bool vec, dim3 grid, const uint32_t* b1, int chunk, int nseg,
                              uint32_t* cand_keys, int32_t* cand_cols, uint32_t* seg_count, hipStream_t stream) {
    if (vec)
        hipLaunchKernelGGL((indexer_rescore_kernel<KF, BK16, true>), grid, dim3(256), 0, stream, p, b1, chunk, nseg,
                           cand_keys, cand_cols, seg_count);
    else
        hipLaunchKernelGGL((indexer_rescore_kernel<KF, BK16, false>), grid, dim3(256), 0, stream, p, b1, chunk, nseg,
                           cand_keys, cand_cols, seg_count);
}

hipError_t launch_indexer_rescore(const IndexParams& p, int rows, int dtype, const uint32_t* b1, int chunk, int nseg,
                                  uint32_t* cand_keys, int32_t* cand_cols, uint32_t* seg_count, hipStream_t stream) {
    const dim3 grid((unsigned)((nseg + 3) / 4), (unsigned)rows);
    const int64_t nbk_row = (p.width + kKeyBlock - 1) / kKeyBlock;
    const bool vec = nbk_row >= 4 && nbk_row % 4 == 0 && reinterpret_cast<uintptr_t>(p.block_keys) % 16 == 0;
    if (dtype == CSA2_FP4_E2M1 && p.bk16)
        launch_rescore_kf<Fp4Keys, true>(p, vec, grid, b1, chunk, nseg, cand_keys, cand_cols, seg_count, stream);
    else if (dtype == CSA2_FP4_E2M1)
        launch_rescore_kf<Fp4Keys, false>(p, vec, grid, b1, chunk, nseg, cand_keys, cand_cols, seg_count, stream);
    else if (p.bk16)
        launch_rescore_kf<Fp8Keys, true>(p, vec, grid, b1, chunk, nseg, cand_keys, cand_cols, seg_count, stream);
    else
        launch_rescore_kf<Fp8Keys, false>(p, vec, grid, b1, chunk, nseg, cand_keys, cand_cols, seg_count, stream);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// REINDEX scoring over 8-row candidate blocks (64 heads x 128; BF16, FP8 or
// MXFP4 index planes).
//
// Column c = 8 i + t of a row is plane row cand[r, i] * 8 + t
// ("DeepSeek-V4.1-Flash 架构解剖", fig. 2c REINDEX: only the 2048 x 8 candidate
// rows are scored).  A 64-column step is 8 consecutive candidate blocks, i.e.
// 8 runs of 8 consecutive key rows (2 KiB each in BF16), so the gather reads
// whole blocks: one load instruction covers whole key rows of one block (BF16:
// 4 rows, FP8: 8 rows) or of two (MXFP4: 16 rows of 64 B).  Each wave loads
// the candidate ids of all its steps up front (lane 8 i' + k holds slot k of
// its step i') and moves each step's 8 ids to scalar registers, so no load
// address waits on an id load inside the step loop.  The rows go through the
// wave's LDS slot into the MFMA operand layout as in the FULL streaming
// kernel, DEPTH steps of loads in flight.  Rows that are not valid (slot -1,
// or past the visible prefix) load a valid row of the same plane instead --
// the plane's first row, or the block's first -- and their columns get -inf.

// BF16 key rows: 256 bytes, sixteen 16-byte chunks, chunk c of key kk at
// position c ^ (kk & 15) (conflict-free for both the staging writes and the
// B-operand reads); no per-row scale.
struct Bf16Keys {
    static constexpr int kRowBytes = 256, kChunks = 16, kLoads = 16;
    static constexpr bool kScaleInScore = true;  // no scale word is staged
    static constexpr bool kDense = true;
    static __device__ __forceinline__ int swz(int kk) { return kk & 15; }
};

// v[u] (lane (g, n)) for BF16 keys: the per-row kernel's arithmetic (four
// 16x16x32 MFMAs per head tile, the NaN guard, integer-max ReLU).
__device__ __forceinline__ void step_sums_bf16(const uint8_t* my, const bf16x8 (&qa)[4][4], const float (&wr)[4][4],
                                               int g, int li, float (&v)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int kk = 16 * u + li;
        bf16x8 kb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            kb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(my + kk * 256 + 16 * ((4 * s + g) ^ (kk & 15))));
        // the four head tiles' chains interleaved (independent accumulators between dependent MFMAs)
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = Mma<__bf16>::k32(acc[t], qa[t][s], kb[s]);
        float acc_sum = nan_guard(acc[0][0]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc_sum += wr[t][rr] * relu_bits(acc[t][rr]);
        v[u] = acc_sum;
    }
}

#ifndef CSA2_REINDEX_MAX_STEPS
#define CSA2_REINDEX_MAX_STEPS 8
#endif
constexpr int kReindexMaxSteps = CSA2_REINDEX_MAX_STEPS;  // 64-column steps per wave at most (the loop is unrolled)

#ifndef CSA2_REINDEX_MIN_WG
#define CSA2_REINDEX_MIN_WG 1
#endif
// SEQ: a FULL row read as its consecutive 8-row blocks (slot i is block i; p.cand is not read):
// the same staged stream over every visible row.
template <class KF, bool HIST, int DEPTH, bool SEQ = false>
__global__ __launch_bounds__(256, CSA2_REINDEX_MIN_WG) void indexer_reindex_kernel(const IndexParams p, int steps_per_wave) {
    __shared__ uint32_t hist[HIST ? kKeyBins : 1];
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][64 * KF::kRowBytes];
    __shared__ uint32_t scl_all[4][KF::kScaleInScore ? 1 : 64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int r = blockIdx.y;
    const int64_t nv = uniform64((p.pos[r] + 1) / p.ratio);
    const int64_t base = uniform64(p.row_base[r]);
    const int nb = p.n_blocks;
    const int n_steps = (nb + 7) / 8;
    const int step0 = blockIdx.x * 4 * steps_per_wave + wave;  // this wave's steps: step0 + 4 i
    float* srow = p.scores + (int64_t)r * p.width;
    uint8_t* my = stage[wave];
    uint32_t* scl = scl_all[wave];
    const uint8_t* plane = reinterpret_cast<const uint8_t*>(p.k) + base * KF::kRowBytes;

    // Candidate ids of this wave's steps first (every load address depends on them): creg[h] in
    // lane 8 i' + k holds slot k of step 8 h + i' (-1 past the row's slots; the last register
    // serves the loads issued past the last step).
    const int32_t* crow = SEQ ? nullptr : p.cand + (int64_t)r * nb;
    int32_t creg[kReindexMaxSteps / 8 + 1];
#pragma unroll
    for (int h = 0; h < kReindexMaxSteps / 8; ++h) {
        const int i = 8 * h + (lane >> 3);
        const int slot = 8 * (step0 + 4 * i) + (lane & 7);
        creg[h] = (i < steps_per_wave && slot < nb) ? (SEQ ? slot : crow[slot]) : -1;
    }
    creg[kReindexMaxSteps / 8] = -1;

    // Query fragments and head weights of row r (in flight while the first steps' loads are issued).
    typedef typename std::conditional<KF::kDense, bf16x8[4][4], i32x8[4]>::type QFrags;
    QFrags qa;
    uint32_t qs[4];
    float wr[4][4];
    if constexpr (KF::kDense) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int s = 0; s < 4; ++s) qa[t][s] = IdxOps<CSA2_BF16, 128>::load(p.q, (int64_t)r * 64 + 16 * t + li, s, g);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) wr[t][rr] = p.w[(int64_t)r * 64 + 16 * t + 4 * g + rr];
            qs[t] = 0u;
        }
    } else {
        load_query<KF>(p, r, g, li, qa, qs, wr);
    }

    if (HIST) {
        for (int b = threadIdx.x; b < kKeyBins; b += 256) hist[b] = 0u;
        __syncthreads();
    }

    // Set once the query is in: a NaN in it makes every score NaN.
    bool q_nan = false;
    float row_scale = p.scale;

    struct Buf {
        u32x4 v[KF::kLoads];
        uint32_t sw;  // scale word of this lane's column (FP8: float bits; MXFP4: 4 E8M0 bytes)
        bool ok;      // this lane's column is valid
    };
    auto issue = [&](int i, Buf& b) {
        // Per slot: the block's first row and how many of its rows are visible (uniform).
        const uint8_t* bp[8];
        int lim[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int32_t c = __builtin_amdgcn_readlane(creg[i >> 3], ((i & 7) << 3) + k);
            const int64_t rem = nv - (int64_t)c * 8;
            const int l = c < 0 ? 0 : (rem >= 8 ? 8 : (rem <= 0 ? 0 : (int)rem));
            lim[k] = l;
            bp[k] = l > 0 ? plane + (int64_t)c * 8 * KF::kRowBytes : plane;
        }
        constexpr int per = 64 / KF::kLoads;  // keys per load instruction
#pragma unroll
        for (int j = 0; j < KF::kLoads; ++j) {
            const int kk = j * per + lane / KF::kChunks;
            const int kA = (j * per) / 8, kB = (j * per + per - 1) / 8;
            const bool second = kA != kB && (kk >> 3) != kA;
            const uint8_t* q = second ? bp[kB] : bp[kA];
            const int l = second ? lim[kB] : lim[kA];
            const int t = kk & 7;
            // non-temporal: each block is read once (measured ~10 % faster than ordinary loads here)
            b.v[j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(q + ((t < l ? t * KF::kRowBytes : 0) + 16 * (lane % KF::kChunks))));
        }
        const int32_t c = __shfl(creg[i >> 3], ((i & 7) << 3) + (lane >> 3), 64);
        const int t = lane & 7;
        b.ok = c >= 0 && (int64_t)c * 8 + t < nv;
        if constexpr (!KF::kDense) {
            const int64_t row = b.ok ? base + (int64_t)c * 8 + t : base;
            b.sw = *reinterpret_cast<const uint32_t*>(KF::scale_base(p, row));
        } else {
            b.sw = 0u;
        }
    };
    auto step = [&](int i, Buf& b) {
        stage_put<KF>(my, scl, b.v, b.sw, lane);
        float sc;
        if constexpr (KF::kDense) sc = row_scale;
        else sc = KF::score_scale(p.scale, b.sw, q_nan);
        const bool valid = b.ok;
        // Unconditional: past the wave's last step the ids are -1 and the loads read the plane's
        // first row.
        issue(i + DEPTH, b);
        // Scheduling fence: the compiler would otherwise pull the next step's staging (and the
        // wait for its loads) into this step's MFMA chains, stalling them on memory.
        __builtin_amdgcn_sched_barrier(0);
        float v[4];
        if constexpr (KF::kDense) step_sums_bf16(my, qa, wr, g, li, v);
        else step_sums<KF>(my, scl, qa, qs, wr, g, li, v);
        const float kk = reduce_scatter(v, lane);
        const int64_t c_out = (int64_t)(step0 + 4 * i) * 64 + lane;
        const float score = valid ? sc * kk : kNegInf;
        if (c_out < p.width) {
            srow[c_out] = score;
            if (HIST && valid) atomicAdd(&hist[order_key(score) >> 20], 1u);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // steps this wave makes (wave-uniform)
    const int n_mine = step0 < n_steps ? min(steps_per_wave, (n_steps - step0 + 3) / 4) : 0;
    Buf bufs[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, bufs[d]);
    if constexpr (KF::kDense) {
        bool qn = false;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s) qn |= frag_has_nan(qa[t][s]);
        q_nan = __ballot(qn) != 0ull;
    } else {
        q_nan = KF::query_nan(qa, qs);
    }
    row_scale = q_nan ? __builtin_nanf("") : p.scale;
#pragma unroll
    for (int it = 0; it < kReindexMaxSteps; ++it) {
        if (it >= n_mine) break;
        step(it, bufs[it % DEPTH]);
    }
    if (HIST) {
        __syncthreads();
        uint32_t* gh = p.key_hist + (int64_t)r * kKeyBins;
        for (int b = threadIdx.x; b < kKeyBins; b += 256)
            if (hist[b]) atomicAdd(&gh[b], hist[b]);
    }
}

__global__ __launch_bounds__(256) void key_hist_zero_kernel(uint32_t* h, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) h[i] = 0u;
}

// ---------------------------------------------------------------------------
template <int KT, int HI, int DI, bool REINDEX>
static hipError_t launch_one(const IndexParams& p, int rows, hipStream_t stream) {
    const int64_t chunks = (p.width + p.cols_per_wg - 1) / p.cols_per_wg;
    dim3 grid((unsigned)chunks, (unsigned)rows);
    const bool hist = p.key_hist != nullptr;
    const bool bmax = !REINDEX && p.block_max != nullptr;
    if (hist) {
        const int64_t nh = (int64_t)rows * kKeyBins;
        hipLaunchKernelGGL(key_hist_zero_kernel, dim3((unsigned)((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024)),
                           dim3(256), 0, stream, p.key_hist, nh);
    }
    if constexpr (!REINDEX) {
        if (bmax) {
            if (hist) hipLaunchKernelGGL((indexer_score_kernel<KT, HI, DI, false, true, true>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((indexer_score_kernel<KT, HI, DI, false, false, true>), grid, dim3(256), 0, stream, p);
            return hipGetLastError();
        }
    }
    if (hist) hipLaunchKernelGGL((indexer_score_kernel<KT, HI, DI, REINDEX, true, false>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((indexer_score_kernel<KT, HI, DI, REINDEX, false, false>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <class KF>
static hipError_t launch_stream_full(const IndexParams& p, int rows, hipStream_t stream) {
    if (p.cols_per_wg > 256 * kStreamMaxSteps || p.cols_per_wg % 256 != 0) return hipErrorInvalidValue;
    const int64_t chunks = (p.width + p.cols_per_wg - 1) / p.cols_per_wg;
    dim3 grid((unsigned)chunks, (unsigned)rows);
    const bool hist = p.key_hist != nullptr;
    if (hist) {
        const int64_t nh = (int64_t)rows * kKeyBins;
        hipLaunchKernelGGL(key_hist_zero_kernel, dim3((unsigned)((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024)),
                           dim3(256), 0, stream, p.key_hist, nh);
    }
    constexpr int D = kStreamDepth;
    if (p.scores == nullptr) {
        // scores kept on chip: block keys only (validated by the caller); the select counts them itself
        if (p.block_max != nullptr)
            hipLaunchKernelGGL((indexer_stream_kernel<KF, false, true, D, false, true>), grid, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((indexer_stream_kernel<KF, false, false, D, false, true>), grid, dim3(256), 0, stream, p);
    } else if (p.block_max != nullptr) {
        if (hist) hipLaunchKernelGGL((indexer_stream_kernel<KF, true, true, D, true, false>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((indexer_stream_kernel<KF, false, true, D, true, false>), grid, dim3(256), 0, stream, p);
    } else {
        if (hist) hipLaunchKernelGGL((indexer_stream_kernel<KF, true, false, D, true, false>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((indexer_stream_kernel<KF, false, false, D, true, false>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

// Steps of loads in flight per wave and waves per launch of the REINDEX kernel (BF16 rows, quantised
// rows); build-time constants so launch shapes can be swept.
#ifndef CSA2_REINDEX_DEPTH
#define CSA2_REINDEX_DEPTH 1
#endif
#ifndef CSA2_REINDEX_WAVES_BF16
#define CSA2_REINDEX_WAVES_BF16 1024
#endif
#ifndef CSA2_REINDEX_WAVES_Q
#define CSA2_REINDEX_WAVES_Q 2048
#endif
constexpr int kReindexDepth = CSA2_REINDEX_DEPTH;

// REINDEX over 8-row blocks: as many waves as fit the chip in one round (BF16: ~300 registers,
// one wave per SIMD; FP8 / MXFP4: two), each taking up to kReindexMaxSteps steps of its row.
// SEQ: a FULL row's consecutive blocks (p.n_blocks = its width in blocks).
template <class KF, bool SEQ = false>
static hipError_t launch_reindex(const IndexParams& p, int rows, hipStream_t stream) {
    const int n_steps = (p.n_blocks + 7) / 8;
    const int64_t total = (int64_t)n_steps * rows;
    const int64_t waves = KF::kDense ? CSA2_REINDEX_WAVES_BF16 : CSA2_REINDEX_WAVES_Q;
    int64_t spw = (total + waves - 1) / waves;
    if (spw < 1) spw = 1;
    if (spw > kReindexMaxSteps) spw = kReindexMaxSteps;
    const int per_wg = 4 * (int)spw;
    const dim3 grid((unsigned)((n_steps + per_wg - 1) / per_wg), (unsigned)rows);
    if (p.key_hist != nullptr) {
        const int64_t nh = (int64_t)rows * kKeyBins;
        hipLaunchKernelGGL(key_hist_zero_kernel, dim3((unsigned)((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024)),
                           dim3(256), 0, stream, p.key_hist, nh);
        hipLaunchKernelGGL((indexer_reindex_kernel<KF, true, kReindexDepth, SEQ>), grid, dim3(256), 0, stream, p,
                           (int)spw);
    } else {
        hipLaunchKernelGGL((indexer_reindex_kernel<KF, false, kReindexDepth, SEQ>), grid, dim3(256), 0, stream, p,
                           (int)spw);
    }
    return hipGetLastError();
}

// FULL rows of BF16 keys (64 x 128) with scores and nothing else per block: the REINDEX kernel's
// staged stream over the row's consecutive 8-row blocks, whose scores are bit-identical to the
// per-row kernel's.
#ifndef CSA2_FULL_BF16_SEQ
#define CSA2_FULL_BF16_SEQ 1
#endif
static bool full_bf16_seq(const IndexParams& p) {
    return CSA2_FULL_BF16_SEQ && !p.shared_plane && p.scores != nullptr && p.block_max == nullptr &&
           p.block_keys == nullptr && p.width > 0 && (p.width + 7) / 8 < (1LL << 31);
}

static hipError_t launch_full_bf16_seq(IndexParams p, int rows, hipStream_t stream) {
    p.n_blocks = (int32_t)((p.width + 7) / 8);
    p.block_rows = 8;
    p.cand = nullptr;
    return launch_reindex<Bf16Keys, true>(p, rows, stream);
}

// Rows sharing one BF16 plane: scores only (no histogram, no block scores), or in score-free mode
// (scores == NULL) the block keys only.
static bool chunk_path(const IndexParams& p, int rows, int heads, int dim, int dtype, bool reindex) {
    if (!p.shared_plane || reindex || heads != 64 || dim != 128 || dtype != CSA2_BF16) return false;
    if (p.key_hist != nullptr || p.block_max != nullptr) return false;
    if (p.scores == nullptr) return p.block_keys != nullptr;  // score-free: any number of rows
    return rows >= kChunkRows && p.block_keys == nullptr;
}

static hipError_t launch_chunk(IndexParams p, int rows, hipStream_t stream) {
    // 8192 columns per workgroup, more when the grid's second dimension (<= 65535) needs it
    int64_t cw = 8192;
    const int64_t need = (p.width + 65534) / 65535;
    if (need > cw) cw = (need + kChunkKeys - 1) / kChunkKeys * kChunkKeys;
    p.cols_per_wg = cw;
    const dim3 grid((unsigned)((rows + kChunkRows - 1) / kChunkRows), (unsigned)((p.width + cw - 1) / cw));
    if (p.scores == nullptr)
        hipLaunchKernelGGL((indexer_chunk_kernel<kChunkRows, kChunkKeys, true>), grid, dim3(64 * kChunkRows), 0, stream, p,
                           rows);
    else
        hipLaunchKernelGGL((indexer_chunk_kernel<kChunkRows, kChunkKeys, false>), grid, dim3(64 * kChunkRows), 0, stream,
                           p, rows);
    return hipGetLastError();
}

hipError_t launch_indexer_score(const IndexParams& p, int rows, int heads, int dim, int dtype, bool reindex,
                                hipStream_t stream) {
    if (chunk_path(p, rows, heads, dim, dtype, reindex)) return launch_chunk(p, rows, stream);
    if (heads == 64 && dim == 128) {
        const bool blocks8 = reindex && p.block_rows == 8;  // the pages' 8-row candidate blocks
        if (dtype == CSA2_BF16) return blocks8 ? launch_reindex<Bf16Keys>(p, rows, stream)
                                     : reindex ? launch_one<CSA2_BF16, 64, 128, true>(p, rows, stream)
                                     : full_bf16_seq(p) ? launch_full_bf16_seq(p, rows, stream)
                                                        : launch_one<CSA2_BF16, 64, 128, false>(p, rows, stream);
        if (dtype == CSA2_FP8_E4M3) return blocks8 ? launch_reindex<Fp8Keys>(p, rows, stream)
                                         : reindex ? launch_one<CSA2_FP8_E4M3, 64, 128, true>(p, rows, stream)
                                                   : launch_stream_full<Fp8Keys>(p, rows, stream);
        if (dtype == CSA2_FP4_E2M1) return blocks8 ? launch_reindex<Fp4Keys>(p, rows, stream)
                                         : reindex ? hipErrorInvalidValue : launch_stream_full<Fp4Keys>(p, rows, stream);
        if (dtype == CSA2_F32) return reindex ? launch_one<CSA2_F32, 64, 128, true>(p, rows, stream)
                                              : launch_one<CSA2_F32, 64, 128, false>(p, rows, stream);
    }
    if (heads == 4 && dim == 32) {
        if (dtype == CSA2_F32) return reindex ? launch_one<CSA2_F32, 4, 32, true>(p, rows, stream)
                                              : launch_one<CSA2_F32, 4, 32, false>(p, rows, stream);
        if (dtype == CSA2_BF16) return reindex ? launch_one<CSA2_BF16, 4, 32, true>(p, rows, stream)
                                               : launch_one<CSA2_BF16, 4, 32, false>(p, rows, stream);
    }
    return hipErrorInvalidValue;
}

bool indexer_rescore_supported(int heads, int dim, int dtype) {
    return heads == 64 && dim == 128 && (dtype == CSA2_FP8_E4M3 || dtype == CSA2_FP4_E2M1);
}

bool indexer_supported(int heads, int dim, int dtype) {
    if (heads == 64 && dim == 128)
        return dtype == CSA2_BF16 || dtype == CSA2_FP8_E4M3 || dtype == CSA2_F32 || dtype == CSA2_FP4_E2M1;
    if (heads == 4 && dim == 32) return dtype == CSA2_F32 || dtype == CSA2_BF16;
    return false;
}

}  // namespace csa2

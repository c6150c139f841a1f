// Per-row top-k of indexer scores for gfx950.
//
// Contract ("DeepSeek-V4.1-Flash 架构解剖", fig. 2d REUSE and special module
// "indexer"): the k valid columns with the largest scores, ties to the lower
// column, NaN ranked as -inf, -0 equal to +0; written in increasing column
// order as plane rows, then -1 padding.
//
// Exact select.  Scores map to an order-preserving 32-bit key
//   key(s) = bits(s) | 0x80000000 for s >= +0, ~bits(s) for s < 0,
// after NaN -> -inf and -0 -> +0, so key order is score order.  Three
// histogram passes over bits [31:20], [19:8] and [7:0] (LDS bins) fix the k-th
// largest key T and the number n_gt of keys above it.  A final pass walks the
// positions in column order, 1024 at a time; a position is taken if key > T,
// or key == T and fewer than k - n_gt equal keys precede it, and lands in slot
// (#greater before it) + min(#equal before it, k - n_gt).  Slots are computed
// with wave ballots and one barrier per 1024 positions, and come out in column
// order, so nothing is sorted.
//
// Two ways to feed that select:
//   * narrow rows or many rows: one 1024-thread workgroup per row reads the
//     score row twice -- a histogram of the keys' top 12 bits gives the bin b1
//     of the k-th largest key, then the keys in bins >= b1 are compacted in
//     column order into LDS, where the select runs (more than kLdsCand such
//     keys, i.e. heavy ties: the select reads the row from memory instead);
//   * wide rows (the 1M-column decode): the row is cut into chunks handled by
//     separate workgroups.  (1) each chunk adds its 12-bit histogram into a
//     per-row global histogram; (2) each chunk's workgroup finds from it the
//     bin b1 of the k-th largest key and (3) compacts, in column order, the
//     (key, column) pairs of its valid keys whose bin is >= b1 -- every key
//     >= T is among them -- into its own slot range; (4) one workgroup per row
//     runs the exact select over that short, still column-ordered list.  A
//     chunk with more than kCap such keys (heavy ties) makes step 4 fall back
//     to reading the full row, so the result is exact in every case.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCap = 1024;      // candidates kept per chunk
constexpr int kMaxSegs = 256;   // chunks per row in the wide-row path

// Validity of column c of row r.
__device__ __forceinline__ bool col_valid(const TopkParams& p, int r, int64_t c, int64_t nv) {
    if (p.n_blocks == 0) return c < nv;
    const int64_t i = c / p.block_rows;
    const int32_t b = p.cand[(int64_t)r * p.n_blocks + i];
    if (b < 0) return false;
    return (int64_t)b * p.block_rows + (c - i * p.block_rows) < nv;
}

// Plane row written to the output for column c (valid columns only).
__device__ __forceinline__ int32_t col_to_row(const TopkParams& p, int r, int32_t c) {
    if (p.n_blocks == 0) return c;
    const int32_t i = c / p.block_rows;
    return p.cand[(int64_t)r * p.n_blocks + i] * p.block_rows + (c - i * p.block_rows);
}

struct Lds {
    uint32_t hist[4096];
    uint32_t wave_tot[kWaves];
    uint32_t sel[2];
    uint32_t flags_cnt[2][2 * kWaves];
    uint32_t seg_start[kMaxSegs + 1];
};

// Set bits of m below this lane.
__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Block-wide exclusive suffix sum (sum of v over threads with a larger index).
__device__ __forceinline__ uint32_t block_suffix_excl(uint32_t v, Lds& s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(x, o, 64);
        if (lane + o < 64) x += y;
    }
    if (lane == 0) s.wave_tot[wave] = x;
    __syncthreads();
    uint32_t later = 0;
    for (int w = wave + 1; w < kWaves; ++w) later += s.wave_tot[w];
    __syncthreads();
    return later + x - v;
}

// Sum of all bins (4096) of s.hist, returned to every thread.
__device__ __forceinline__ uint32_t hist_total(Lds& s) {
    const int t = threadIdx.x;
    const uint32_t local = s.hist[4 * t] + s.hist[4 * t + 1] + s.hist[4 * t + 2] + s.hist[4 * t + 3];
    const uint32_t later = block_suffix_excl(local, s);
    if (t == 0) s.sel[0] = later + local;
    __syncthreads();
    const uint32_t total = s.sel[0];
    __syncthreads();
    return total;
}

// Scanning bins from the top, the bin where the running count first reaches
// `need` (>= 1, <= total), and the count in the bins above it.
__device__ __forceinline__ void find_bin(Lds& s, int nbins, uint32_t need, uint32_t& bin, uint32_t& above_out) {
    const int per = nbins / kThreads;
    const int t = threadIdx.x;
    int b0 = 0, b1 = 0;
    if (per > 0) {
        b0 = per * t;
        b1 = b0 + per;
    } else if (t < nbins) {
        b0 = t;
        b1 = t + 1;
    }
    uint32_t local = 0;
    for (int b = b0; b < b1; ++b) local += s.hist[b];
    uint32_t above = block_suffix_excl(local, s);
    for (int b = b1 - 1; b >= b0; --b) {
        const uint32_t h = s.hist[b];
        if (above < need && above + h >= need) {
            s.sel[0] = (uint32_t)b;
            s.sel[1] = above;
        }
        above += h;
    }
    __syncthreads();
    bin = s.sel[0];
    above_out = s.sel[1];
    __syncthreads();
}

// Rank key of a pool column from its block key (the newest column pinned to +inf).
__device__ __forceinline__ uint32_t pool_rank_key(uint32_t bk, bool newest) {
    return newest ? 0xff800000u : order_key(pool_value_of_block_key(bk));
}

// What a row holds: scores, candidate-pool block keys (ranked by the pool's block score, the
// newest block pinned) or plain block keys (ranked as the largest score of the block, NaN as -inf).
constexpr int kSrcScores = 0, kSrcPool = 1, kSrcKeys = 2;

// Positions of the full row: column i, validity from the row geometry.
template <int SRC>
struct RowSrc {
    const TopkParams* p;
    const float* srow;
    const uint32_t* krow;
    int64_t nv;
    int r;
    int n;
    // the 32-bit word of column i (score bits or block key)
    __device__ __forceinline__ uint32_t raw(int i) const {
        return SRC == kSrcScores ? __float_as_uint(srow[i]) : krow[i];
    }
    __device__ __forceinline__ uint32_t key_of(uint32_t w, int i) const {
        if (SRC == kSrcPool) return pool_rank_key(w, i == nv - 1);
        if (SRC == kSrcKeys) return w == kNanBlockKey ? 0x007fffffu : w;  // a NaN block ranks as -inf
        return order_key(__uint_as_float(w));
    }
    __device__ __forceinline__ bool get(int i, uint32_t& key, int32_t& col) const {
        col = i;
        if (!col_valid(*p, r, i, nv)) return false;
        key = key_of(raw(i), i);
        return true;
    }
};

// Positions of the filtered candidate list: segment-major, column order within.
struct CandSrc {
    const uint32_t* keys;      // [nseg][cap] of this row
    const int32_t* cols;       // [nseg][cap]
    const uint32_t* seg_start; // LDS prefix of the segment counts, [nseg + 1]
    int nseg;
    int cap;
    int n;
    __device__ __forceinline__ bool get(int i, uint32_t& key, int32_t& col) const {
        int lo = 0, hi = nseg;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((int)seg_start[mid] <= i) lo = mid;
            else hi = mid;
        }
        const int j = i - (int)seg_start[lo];
        key = keys[(int64_t)lo * cap + j];
        col = cols[(int64_t)lo * cap + j];
        return true;
    }
};

// Candidates copied into LDS: a dense, column-ordered list.
constexpr int kLdsCand = 4096;
struct LdsCandSrc {
    const uint32_t* keys;
    const int32_t* cols;
    int n;
    __device__ __forceinline__ bool get(int i, uint32_t& key, int32_t& col) const {
        key = keys[i];
        col = cols[i];
        return true;
    }
};

template <class Src>
// known_b1 >= 0: every position holds a valid key, and the bin of the k-th largest key and the
// count above it (known_above1) are already known -- pass 1 is skipped.
__device__ __forceinline__ void select_core(const Src& src, const TopkParams& p, int r, Lds& s, int known_b1 = -1,
                                            uint32_t known_above1 = 0) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int32_t* orow = p.out + (int64_t)r * p.k;
    const uint32_t k = (uint32_t)p.k;
    const int n = src.n;

    uint32_t total = (uint32_t)n;
    if (known_b1 < 0) {
        // pass 1: bits [31:20]
        for (int b = tid; b < 4096; b += kThreads) s.hist[b] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            uint32_t key;
            int32_t col;
            if (src.get(i, key, col)) atomicAdd(&s.hist[key >> 20], 1u);
        }
        __syncthreads();
        total = hist_total(s);
    }
    const bool select_all = total <= k;
    uint32_t T = 0, n_gt = 0;
    if (!select_all) {
        uint32_t b1, above1, b2, above2, b3, above3;
        if (known_b1 >= 0) {
            b1 = (uint32_t)known_b1;
            above1 = known_above1;
        } else {
            find_bin(s, 4096, k, b1, above1);
        }
        // pass 2: bits [19:8] of keys in bin b1
        for (int b = tid; b < 4096; b += kThreads) s.hist[b] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            uint32_t key;
            int32_t col;
            if (src.get(i, key, col) && (key >> 20) == b1) atomicAdd(&s.hist[(key >> 8) & 0xfffu], 1u);
        }
        __syncthreads();
        find_bin(s, 4096, k - above1, b2, above2);
        // pass 3: bits [7:0] of keys with prefix (b1, b2)
        const uint32_t pre = (b1 << 12) | b2;
        for (int b = tid; b < 256; b += kThreads) s.hist[b] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            uint32_t key;
            int32_t col;
            if (src.get(i, key, col) && (key >> 8) == pre) atomicAdd(&s.hist[key & 0xffu], 1u);
        }
        __syncthreads();
        find_bin(s, 256, k - above1 - above2, b3, above3);
        T = (pre << 8) | b3;
        n_gt = above1 + above2 + above3;
    }
    const uint32_t need = select_all ? 0u : k - n_gt;  // equal keys to take, lowest columns first
    const uint32_t goal = select_all ? total : k;

    // ordered compaction
    uint32_t gt_base = 0, eq_base = 0;
    int buf = 0;
    for (int cs = 0; cs < n; cs += kThreads) {
        const int i = cs + tid;
        uint32_t key = 0;
        int32_t col = -1;
        bool gt = false, eq = false;
        if (i < n && src.get(i, key, col)) {
            gt = select_all || key > T;
            eq = !select_all && key == T;
        }
        const uint64_t mgt = __ballot(gt);
        const uint64_t meq = __ballot(eq);
        const uint32_t gt_lane = __builtin_amdgcn_mbcnt_hi((uint32_t)(mgt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mgt, 0u));
        const uint32_t eq_lane = __builtin_amdgcn_mbcnt_hi((uint32_t)(meq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)meq, 0u));
        if (lane == 0) {
            s.flags_cnt[buf][wave] = (uint32_t)__builtin_popcountll(mgt);
            s.flags_cnt[buf][kWaves + wave] = (uint32_t)__builtin_popcountll(meq);
        }
        __syncthreads();
        uint32_t gt_before = gt_base, eq_before = eq_base, gt_all = 0, eq_all = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t a = s.flags_cnt[buf][w], b = s.flags_cnt[buf][kWaves + w];
            if (w < wave) {
                gt_before += a;
                eq_before += b;
            }
            gt_all += a;
            eq_all += b;
        }
        gt_before += gt_lane;
        eq_before += eq_lane;
        if (gt || (eq && eq_before < need)) orow[gt_before + (eq_before < need ? eq_before : need)] = col_to_row(p, r, col);
        gt_base += gt_all;
        eq_base += eq_all;
        buf ^= 1;
        if (gt_base + (eq_base < need ? eq_base : need) >= goal) break;
    }
    for (int i = (int)goal + tid; i < p.k; i += kThreads) orow[i] = -1;
}

template <int SRC>
__device__ __forceinline__ RowSrc<SRC> row_src(const TopkParams& p, int r) {
    RowSrc<SRC> src;
    src.p = &p;
    src.r = r;
    src.nv = (p.pos[r] + 1) / p.ratio;
    if (p.col_group > 1) src.nv = (src.nv + p.col_group - 1) / p.col_group;
    src.srow = p.scores + (int64_t)r * p.width;
    src.krow = SRC != kSrcScores ? p.pool_keys + (int64_t)r * p.width : nullptr;
    src.n = (p.n_blocks == 0) ? (int)(src.nv < p.width ? src.nv : p.width) : (int)p.width;
    return src;
}

}  // namespace


// ---- wide-row path ----------------------------------------------------------

__global__ __launch_bounds__(256) void topk_zero_kernel(uint32_t* buf, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) buf[i] = 0u;
}

// grid (nseg, rows): 12-bit histogram of one chunk, added into hist[r][4096].
template <int SRC>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const TopkParams p, uint32_t* hist, int chunk) {
    __shared__ uint32_t h[4096];
    const int r = blockIdx.y;
    const int tid = threadIdx.x;
    const RowSrc<SRC> src = row_src<SRC>(p, r);
    for (int b = tid; b < 4096; b += kThreads) h[b] = 0;
    __syncthreads();
    const int c0 = blockIdx.x * chunk;
    const int c1 = (c0 + chunk < src.n) ? c0 + chunk : src.n;
    for (int i = c0 + tid; i < c1; i += kThreads) {
        uint32_t key;
        int32_t col;
        if (src.get(i, key, col)) atomicAdd(&h[key >> 20], 1u);
    }
    __syncthreads();
    uint32_t* g = hist + (int64_t)r * 4096;
    for (int b = tid; b < 4096; b += kThreads)
        if (h[b]) atomicAdd(&g[b], h[b]);
}

// Bin of row r's k-th largest key (0 when every valid key is selected), from
// `parts` histograms of the row ([parts, 4096], added in order); every thread
// of the workgroup gets it.
__device__ __forceinline__ uint32_t row_threshold_bin(const TopkParams& p, const uint32_t* hist, int parts, Lds& s) {
    static_assert(4 * kThreads == 4096, "four bins per thread");
    const int t = threadIdx.x;
    // Thread t adds bins t + 1024e (e < 4) over the parts, eight parts' loads in
    // flight at once (a part index past the end re-reads the last part, whose
    // values are then dropped).
    const uint32_t* hr = hist + t;
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
    for (int q0 = 0; q0 < parts; q0 += 8) {
        uint32_t v[8][4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t q = q0 + j < parts ? q0 + j : parts - 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[j][e] = hr[q * 4096 + e * kThreads];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += q0 + j < parts ? v[j][e] : 0u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s.hist[e * kThreads + t] = acc[e];
    __syncthreads();
    // One suffix scan over the threads' four-bin groups gives both the total
    // and, for the group that holds it, the bin where the count from the top
    // reaches k.
    const uint32_t need = (uint32_t)p.k;
    const uint32_t h0 = s.hist[4 * t], h1 = s.hist[4 * t + 1], h2 = s.hist[4 * t + 2], h3 = s.hist[4 * t + 3];
    uint32_t above = block_suffix_excl(h0 + h1 + h2 + h3, s);
    if (t == 0) s.sel[1] = above + h0 + h1 + h2 + h3;
    const uint32_t hv[4] = {h0, h1, h2, h3};
#pragma unroll
    for (int b = 3; b >= 0; --b) {
        if (above < need && above + hv[b] >= need) s.sel[0] = (uint32_t)(4 * t + b);
        above += hv[b];
    }
    __syncthreads();
    return s.sel[1] > need ? s.sel[0] : 0u;
}

// grid rows: row_threshold_bin of each row into b1_out.
__global__ __launch_bounds__(kThreads) void topk_threshold_kernel(const TopkParams p, const uint32_t* hist,
                                                                  uint32_t* b1_out, int parts) {
    __shared__ Lds s;
    const int r = blockIdx.x;
    const uint32_t b1 = row_threshold_bin(p, hist + (int64_t)r * parts * 4096, parts, s);
    if (threadIdx.x == 0) b1_out[r] = b1;
}

// grid (nseg, rows): ordered compaction of the chunk's keys with bin >= b1.
// Each sweep covers kSweep columns: wave w owns a contiguous 1024-column slice,
// lane l holds columns base + 64j + l (j < 16) in registers, so one barrier per
// sweep (to add up the waves' counts) is the only synchronisation.
constexpr int kPerLane = 16;
constexpr int kSweep = kThreads * kPerLane;

// One workgroup per row over the full score row, in two passes over memory.
// The first counts the valid keys' top 12 bits, which gives the bin b1 of the
// k-th largest key; the second copies the valid keys in bins >= b1 (in column
// order) into LDS, where select_core finishes without touching memory again.
// A row with more than kLdsCand such keys (heavy ties) is selected from
// memory instead.  Sweeps as in topk_filter_kernel: wave w owns a contiguous
// 1024-column slice and lane l its columns base + 64j + l (j < 16), whose
// loads are all in flight before any is used.
template <int SRC>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(const TopkParams p) {
    __shared__ Lds s;
    __shared__ uint32_t lkeys[kLdsCand];
    __shared__ int32_t lcols[kLdsCand];
    __shared__ uint32_t cnt[2][kWaves];
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RowSrc<SRC> src = row_src<SRC>(p, r);
    const int n = src.n;
    const uint32_t k = (uint32_t)p.k;

    for (int b = tid; b < 4096; b += kThreads) s.hist[b] = 0u;
    __syncthreads();
    for (int cs = 0; cs < n; cs += kSweep) {
        const int wbase = cs + wave * (kSweep / kWaves);
        uint32_t vals[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int i = wbase + 64 * j + lane;
            vals[j] = (i < n) ? src.raw(i) : 0u;
        }
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int i = wbase + 64 * j + lane;
            if (i < n && col_valid(p, r, i, src.nv)) atomicAdd(&s.hist[src.key_of(vals[j], i) >> 20], 1u);
        }
    }
    __syncthreads();
    const uint32_t total = hist_total(s);
    uint32_t b1 = 0, above = 0;
    if (total > k) find_bin(s, 4096, k, b1, above);
    const uint32_t n_cand = total > k ? above + s.hist[b1] : total;  // valid keys with bin >= b1
    __syncthreads();  // every thread has read the histogram
    if (n_cand > (uint32_t)kLdsCand) {
        select_core(src, p, r, s);
        return;
    }
    uint32_t n_out = 0;
    int buf = 0;
    for (int cs = 0; cs < n && n_out < n_cand; cs += kSweep) {
        const int wbase = cs + wave * (kSweep / kWaves);
        uint32_t vals[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int i = wbase + 64 * j + lane;
            vals[j] = (i < n) ? src.raw(i) : 0u;
        }
        uint32_t keys[kPerLane];
        uint64_t masks[kPerLane];
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int i = wbase + 64 * j + lane;
            keys[j] = src.key_of(vals[j], i);
            const bool take = i < n && col_valid(p, r, i, src.nv) && (keys[j] >> 20) >= b1;
            masks[j] = __ballot(take);
            mine += (uint32_t)__builtin_popcountll(masks[j]);
        }
        if (lane == 0) cnt[buf][wave] = mine;
        __syncthreads();
        uint32_t off = n_out, all = 0;
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) off += cnt[buf][w];
            all += cnt[buf][w];
        }
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const uint64_t m = masks[j];
            if ((m >> lane) & 1ull) {
                const uint32_t at = off + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                lkeys[at] = keys[j];
                lcols[at] = wbase + 64 * j + lane;
            }
            off += (uint32_t)__builtin_popcountll(m);
        }
        n_out += all;
        buf ^= 1;
    }
    __syncthreads();
    LdsCandSrc lsrc;
    lsrc.keys = lkeys;
    lsrc.cols = lcols;
    lsrc.n = (int)n_cand;
    select_core(lsrc, p, r, s);
}

// One workgroup per FULL score row (no candidate blocks: the valid columns are
// the visible prefix) of at most kRegCols columns, read once: each thread loads
// 64 scores (16 x 16-byte buffer loads; thread (w, l) owns columns
// 4096 w + 256 j + 4 l + e, so each load instruction covers 1 KiB of the row)
// and keeps only their keys' 12-bit bins, two to a register (bin 0 marks a
// column past the visible prefix: no valid key is in a bin below 7).  The
// histogram gives the bin b1 of the k-th largest key; the columns in bins >=
// b1 are compacted into LDS in column order -- per wave in (j, lane, e) order
// with lane offsets from three bit-plane ballots of the lane counts, waves in
// turn -- their scores are read again (about 1 % of the row, from L2) for the
// full keys, and select_core finishes from its second pass (its first would
// find b1 again).  More than kLdsCand such columns (heavy ties): select_core
// over the row in memory, as in topk_select_kernel.
constexpr int kRegCols = kThreads * 64;

__global__ __launch_bounds__(kThreads) void topk_regs_kernel(const TopkParams p) {
    __shared__ Lds s;
    __shared__ uint32_t lkeys[kLdsCand];
    __shared__ int32_t lcols[kLdsCand];
    __shared__ uint32_t wtot[kWaves];
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RowSrc<kSrcScores> src = row_src<kSrcScores>(p, r);
    const int n = src.n;
    const uint32_t k = (uint32_t)p.k;
    const int cbase = 4096 * wave + 4 * lane;
    // the visible prefix as a buffer: loads past it return zeros, so none needs a branch
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(src.srow), (short)0, (n > 0 ? n : 0) * 4, 0x00020000);
    for (int b = tid; b < 4096; b += kThreads) s.hist[b] = 0u;
    uint32_t bp[32];  // bins of columns 4j + e (j < 16, e < 4): entry (4j + e) / 2, half (4j + e) % 2
    {
        u32x4 v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (cbase + 256 * j), 0, 0));
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            uint32_t bins[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t live = 0u - (uint32_t)(cbase + 256 * j + e < n);  // all ones or zero
                bins[e] = (order_key(__uint_as_float(v[j][e])) >> 20) & live;
            }
            bp[2 * j] = bins[0] | (bins[1] << 16);
            bp[2 * j + 1] = bins[2] | (bins[3] << 16);
        }
    }
    __syncthreads();  // histogram cleared
#pragma unroll
    for (int q = 0; q < 32; ++q) {
        atomicAdd(&s.hist[bp[q] & 0xffffu], 1u);
        atomicAdd(&s.hist[bp[q] >> 16], 1u);
    }
    __syncthreads();
    const uint32_t total = hist_total(s) - s.hist[0];  // valid keys (bin 0: past the prefix)
    uint32_t b1 = 0, above = 0;
    if (total > k) find_bin(s, 4096, k, b1, above);  // b1 >= 7: bin 0 is never reached
    const uint32_t n_cand = total > k ? above + s.hist[b1] : total;  // valid keys with bin >= b1
    __syncthreads();  // every thread has read the histogram
    if (n_cand > (uint32_t)kLdsCand) {
        select_core(src, p, r, s);
        return;
    }
    // bin 0 (not valid) is below b1 whenever b1 is used; with total <= k every valid key is taken
    auto bin_at = [&](int j, int e) { return (bp[2 * j + (e >> 1)] >> (16 * (e & 1))) & 0xffffu; };
    auto take = [&](uint32_t bin) { return bin != 0u && bin >= b1; };
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) mine += take(bin_at(j, e)) ? 1u : 0u;
    uint32_t wsum = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) wsum += __shfl_xor(wsum, o, 64);
    if (lane == 0) wtot[wave] = wsum;
    __syncthreads();
    uint32_t off = 0;
    for (int w = 0; w < wave; ++w) off += wtot[w];
    // the columns again, from a value the compiler cannot match with the first pass's (it would
    // otherwise keep all 64 column numbers alive across the histogram, in scratch)
    int cb = cbase;
    asm volatile("" : "+v"(cb));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        uint32_t cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) cnt += take(bin_at(j, e)) ? 1u : 0u;
        const uint64_t p0 = __ballot(cnt & 1u), p1 = __ballot(cnt & 2u), p2 = __ballot(cnt & 4u);
        uint32_t at = off + mbcnt64(p0) + 2u * mbcnt64(p1) + 4u * mbcnt64(p2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (take(bin_at(j, e))) {
                lcols[at] = cb + 256 * j + e;
                ++at;
            }
        }
        off += (uint32_t)(__builtin_popcountll(p0) + 2 * __builtin_popcountll(p1) + 4 * __builtin_popcountll(p2));
    }
    __syncthreads();
    // the candidates' full keys, from their scores (read again: the row has just gone through L2)
    for (int i = tid; i < (int)n_cand; i += kThreads) lkeys[i] = order_key(src.srow[lcols[i]]);
    __syncthreads();
    LdsCandSrc lsrc;
    lsrc.keys = lkeys;
    lsrc.cols = lcols;
    lsrc.n = (int)n_cand;
    select_core(lsrc, p, r, s, (int)b1, above);
}

// Each workgroup first finds its row's threshold bin b1 from the row's histogram
// (the same for every segment of the row; this spares a launch between the
// histogram and the filter).
template <int SRC>
__global__ __launch_bounds__(kThreads) void topk_filter_kernel(const TopkParams p, const uint32_t* hist,
                                                               uint32_t* cand_keys, int32_t* cand_cols,
                                                               uint32_t* seg_count, int chunk, int nseg) {
    __shared__ Lds s;
    __shared__ uint32_t cnt[2][kWaves];
    const int r = blockIdx.y, seg = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RowSrc<SRC> src = row_src<SRC>(p, r);
    const uint32_t b1 = row_threshold_bin(p, hist + (int64_t)r * 4096, 1, s);
    const int64_t base = ((int64_t)r * nseg + seg) * kCap;
    const int c0 = seg * chunk;
    const int c1 = (c0 + chunk < src.n) ? c0 + chunk : src.n;
    uint32_t n_out = 0;
    int buf = 0;
    for (int cs = c0; cs < c1; cs += kSweep) {
        const int wbase = cs + wave * (kSweep / kWaves);
        // All loads first (in flight together), then the keys and ballots.
        uint32_t vals[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int i = wbase + 64 * j + lane;
            vals[j] = (i < c1) ? src.raw(i) : 0u;
        }
        uint32_t keys[kPerLane];
        uint64_t masks[kPerLane];
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int i = wbase + 64 * j + lane;
            keys[j] = src.key_of(vals[j], i);
            const bool take = i < c1 && col_valid(p, r, i, src.nv) && (keys[j] >> 20) >= b1;
            masks[j] = __ballot(take);
            mine += (uint32_t)__builtin_popcountll(masks[j]);
        }
        if (lane == 0) cnt[buf][wave] = mine;
        __syncthreads();
        uint32_t off = n_out, all = 0;
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) off += cnt[buf][w];
            all += cnt[buf][w];
        }
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const uint64_t m = masks[j];
            if ((m >> lane) & 1ull) {
                const uint32_t at = off + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                if (at < (uint32_t)kCap) {
                    cand_keys[base + at] = keys[j];
                    cand_cols[base + at] = wbase + 64 * j + lane;
                }
            }
            off += (uint32_t)__builtin_popcountll(m);
        }
        n_out += all;
        buf ^= 1;
    }
    if (tid == 0) seg_count[(int64_t)r * nseg + seg] = n_out;
}

// grid rows: exact select over the candidates (or the full row after an overflow:
// a list longer than its capacity `cap`).
template <int SRC>
__global__ __launch_bounds__(kThreads) void topk_final_kernel(const TopkParams p, const uint32_t* cand_keys,
                                                              const int32_t* cand_cols, const uint32_t* seg_count,
                                                              int nseg, int cap) {
    __shared__ Lds s;
    __shared__ uint32_t lkeys[kLdsCand];
    __shared__ int32_t lcols[kLdsCand];
    const int r = blockIdx.x;
    // segment starts: one count per thread (nseg <= kMaxSegs < kThreads), block-wide scan
    const int t = threadIdx.x;
    const uint32_t c = t < nseg ? seg_count[(int64_t)r * nseg + t] : 0u;
    const uint64_t over_m = __ballot(c > (uint32_t)cap);
    if ((threadIdx.x & 63) == 0) s.flags_cnt[0][threadIdx.x >> 6] = over_m != 0;
    const uint32_t later = block_suffix_excl(c, s);  // counts of segments after t
    if (t == 0) s.sel[1] = later + c;                // total
    __syncthreads();
    const uint32_t total = s.sel[1];
    if (t <= nseg) s.seg_start[t] = total - later - c;
    if (t == 0) {
        uint32_t over = 0;
        for (int w = 0; w < kWaves; ++w) over |= s.flags_cnt[0][w];
        s.sel[0] = over;
    }
    __syncthreads();
    const bool overflow = s.sel[0] != 0;
    const int n = (int)s.seg_start[nseg];
    __syncthreads();
    if (overflow) {
        select_core(row_src<SRC>(p, r), p, r, s);
        return;
    }
    CandSrc src;
    src.keys = cand_keys + (int64_t)r * nseg * cap;
    src.cols = cand_cols + (int64_t)r * nseg * cap;
    src.seg_start = s.seg_start;
    src.nseg = nseg;
    src.cap = cap;
    src.n = n;
    if (n > kLdsCand) {
        select_core(src, p, r, s);
        return;
    }
    // the usual case: few candidates, read once into LDS and selected from there
    for (int i = threadIdx.x; i < n; i += kThreads) {
        uint32_t key;
        int32_t col;
        src.get(i, key, col);
        lkeys[i] = key;
        lcols[i] = col;
    }
    __syncthreads();
    LdsCandSrc lsrc;
    lsrc.keys = lkeys;
    lsrc.cols = lcols;
    lsrc.n = n;
    select_core(lsrc, p, r, s);
}

// ---------------------------------------------------------------------------
// Launch plan for the wide-row path; nseg == 0 means one workgroup per row.  A
// chunk is at least 4096 columns, and min_chunk when that still leaves >= 512
// workgroups (the filter pass sweeps kSweep columns per workgroup at a time, so
// smaller chunks leave lanes idle).
#ifndef CSA2_TOPK_WIDE_MIN
#define CSA2_TOPK_WIDE_MIN 8192
#endif
void topk_plan(int rows, int64_t width, int& chunk, int& nseg, int min_chunk) {
    chunk = 0;
    nseg = 0;
    if (rows <= 0 || rows >= 1024 || width < CSA2_TOPK_WIDE_MIN) return;
    int64_t target = 4096 / rows;
    if (target < 1) target = 1;
    int64_t c = (width + target - 1) / target;
    if (c < 4096) c = 4096;
    // full sweeps when that still leaves >= 512 workgroups
    if (c < min_chunk && (int64_t)rows * ((width + min_chunk - 1) / min_chunk) >= 512) c = min_chunk;
    const int64_t min_c = (width + kMaxSegs - 1) / kMaxSegs;
    if (c < min_c) c = min_c;
    c = (c + 1023) / 1024 * 1024;
    chunk = (int)c;
    nseg = (int)((width + c - 1) / c);
    if (nseg < 2) chunk = nseg = 0;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t topk_workspace_bytes(int rows, int64_t width) {
    int chunk, nseg;
    topk_plan(rows, width, chunk, nseg, kSweep);
    if (nseg == 0) return 0;
    return align256((size_t)rows * 4096 * 4) + align256((size_t)rows * nseg * 4) +
           2 * align256((size_t)rows * nseg * kCap * 4);
}

template <int SRC>
static hipError_t launch_topk_src(const TopkParams& p, int rows, void* ws, hipStream_t stream) {
    int chunk, nseg;
    topk_plan(rows, p.width, chunk, nseg, kSweep);
    if (nseg == 0) {
        if (SRC == kSrcScores && p.n_blocks == 0 && p.width <= kRegCols && p.width % 4 == 0 &&
            reinterpret_cast<uintptr_t>(p.scores) % 16 == 0)
            hipLaunchKernelGGL(topk_regs_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL(topk_select_kernel<SRC>, dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
    char* w = reinterpret_cast<char*>(ws);
    uint32_t* hist = reinterpret_cast<uint32_t*>(w);
    w += align256((size_t)rows * 4096 * 4);
    uint32_t* seg_count = reinterpret_cast<uint32_t*>(w);
    w += align256((size_t)rows * nseg * 4);
    uint32_t* keys = reinterpret_cast<uint32_t*>(w);
    w += align256((size_t)rows * nseg * kCap * 4);
    int32_t* cols = reinterpret_cast<int32_t*>(w);

    const uint32_t* h = p.key_hist;
    if (h == nullptr) {  // no histogram from the indexer: build it here
        const int64_t nh = (int64_t)rows * 4096;
        hipLaunchKernelGGL(topk_zero_kernel, dim3((unsigned)((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024)),
                           dim3(256), 0, stream, hist, nh);
        hipLaunchKernelGGL(topk_hist_kernel<SRC>, dim3((unsigned)nseg, (unsigned)rows), dim3(kThreads), 0, stream, p,
                           hist, chunk);
        h = hist;
    }
    hipLaunchKernelGGL(topk_filter_kernel<SRC>, dim3((unsigned)nseg, (unsigned)rows), dim3(kThreads), 0, stream, p, h,
                       keys, cols, seg_count, chunk, nseg);
    hipLaunchKernelGGL(topk_final_kernel<SRC>, dim3((unsigned)rows), dim3(kThreads), 0, stream, p, keys, cols,
                       seg_count, nseg, kCap);
    return hipGetLastError();
}

hipError_t launch_topk_select(const TopkParams& p, int rows, void* ws, hipStream_t stream) {
    if (p.pool_keys == nullptr) return launch_topk_src<kSrcScores>(p, rows, ws, stream);
    if (p.plain_keys) return launch_topk_src<kSrcKeys>(p, rows, ws, stream);
    return launch_topk_src<kSrcPool>(p, rows, ws, stream);
}

// grid (nseg, rows): histogram of the block keys' top 12 bits, per row.  Each
// workgroup counts seg_len consecutive keys of its row in LDS and writes all
// 4096 bins to its own slot hist[(r * nseg + seg) * 4096 ...] (no atomics, no
// zeroing; topk_threshold_kernel adds the slots).  Keys of 0 (blocks without a
// valid column) are not counted.  BK16: the keys are the uint16_t top halves.
template <int NT, bool VEC, bool BK16>
__global__ __launch_bounds__(NT) void block_key_hist_kernel(const uint32_t* bkeys, int64_t nbk_row, int seg_len,
                                                            uint32_t* hist) {
    __shared__ uint32_t h[4096];
    const int r = blockIdx.y;
    for (int b = threadIdx.x; b < 4096; b += NT) h[b] = 0u;
    __syncthreads();
    const int64_t i0 = (int64_t)blockIdx.x * seg_len;
    const int64_t i1 = i0 + seg_len < nbk_row ? i0 + seg_len : nbk_row;
    if (BK16) {
        const uint16_t* row = reinterpret_cast<const uint16_t*>(bkeys) + (int64_t)r * nbk_row;
        if (VEC) {  // 16-byte loads: the segment and the row are multiples of 8 keys, 16-byte aligned
            for (int64_t i = i0 + 8 * threadIdx.x; i < i1; i += 8 * NT) {
                const u32x4 k = *reinterpret_cast<const u32x4*>(row + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = k[e] & 0xffffu, hi = k[e] >> 16;
                    if (lo != 0u) atomicAdd(&h[lo >> 4], 1u);
                    if (hi != 0u) atomicAdd(&h[hi >> 4], 1u);
                }
            }
        } else {
            for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) {
                const uint32_t k = row[i];
                if (k != 0u) atomicAdd(&h[k >> 4], 1u);
            }
        }
    } else {
        const uint32_t* row = bkeys + (int64_t)r * nbk_row;
        if (VEC) {  // 16-byte loads: the segment and the row are multiples of 4 keys, 16-byte aligned
            for (int64_t i = i0 + 4 * threadIdx.x; i < i1; i += 4 * NT) {
                const u32x4 k = *reinterpret_cast<const u32x4*>(row + i);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (k[e] != 0u) atomicAdd(&h[k[e] >> 20], 1u);
            }
        } else {
            for (int64_t i = i0 + threadIdx.x; i < i1; i += NT) {
                const uint32_t k = row[i];
                if (k != 0u) atomicAdd(&h[k >> 20], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t* g = hist + ((int64_t)r * gridDim.x + blockIdx.x) * 4096;
    for (int b = threadIdx.x; b < 4096; b += NT) g[b] = h[b];
}

constexpr int kBkhThreads = 1024;
constexpr int kBkhSeg = 16384;

int block_key_hist_parts(int64_t nbk_row) { return (int)((nbk_row + kBkhSeg - 1) / kBkhSeg); }

hipError_t launch_block_key_hist(const uint32_t* bkeys, bool bk16, int64_t nbk_row, int rows, uint32_t* hist,
                                 hipStream_t stream) {
    const dim3 grid((unsigned)((nbk_row + kBkhSeg - 1) / kBkhSeg), (unsigned)rows);
    const bool vec = nbk_row % (bk16 ? 8 : 4) == 0 && reinterpret_cast<uintptr_t>(bkeys) % 16 == 0;
    if (bk16 && vec)
        hipLaunchKernelGGL((block_key_hist_kernel<kBkhThreads, true, true>), grid, dim3(kBkhThreads), 0, stream, bkeys,
                           nbk_row, kBkhSeg, hist);
    else if (bk16)
        hipLaunchKernelGGL((block_key_hist_kernel<kBkhThreads, false, true>), grid, dim3(kBkhThreads), 0, stream, bkeys,
                           nbk_row, kBkhSeg, hist);
    else if (vec)
        hipLaunchKernelGGL((block_key_hist_kernel<kBkhThreads, true, false>), grid, dim3(kBkhThreads), 0, stream, bkeys,
                           nbk_row, kBkhSeg, hist);
    else
        hipLaunchKernelGGL((block_key_hist_kernel<kBkhThreads, false, false>), grid, dim3(kBkhThreads), 0, stream,
                           bkeys, nbk_row, kBkhSeg, hist);
    return hipGetLastError();
}

hipError_t launch_topk_threshold(const TopkParams& p, int rows, const uint32_t* key_hist, int parts, uint32_t* b1,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(topk_threshold_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, p, key_hist, b1, parts);
    return hipGetLastError();
}

hipError_t launch_topk_final(const TopkParams& p, int rows, const uint32_t* cand_keys, const int32_t* cand_cols,
                             const uint32_t* seg_count, int nseg, int cap, hipStream_t stream) {
    hipLaunchKernelGGL(topk_final_kernel<kSrcScores>, dim3((unsigned)rows), dim3(kThreads), 0, stream, p, cand_keys,
                       cand_cols, seg_count, nseg, cap);
    return hipGetLastError();
}

}  // namespace csa2

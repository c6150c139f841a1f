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
//   * rows up to 65536 columns (and any row of 1024 or more rows): one
//     1024-thread workgroup per row.  topk_regs_kernel reads the row once into
//     registers, finds a bin floor the k-th largest key cannot lie below (from
//     the threads' largest bins, or from the histogram of every key), and
//     compacts the keys above it in column order into LDS, where the select
//     runs; topk_select_kernel does the same in two reads of the row for the
//     other sources (candidate-pool and block keys, unaligned rows).  More than
//     kLdsCand candidates, i.e. heavy ties: the select reads the row from
//     memory instead;
//   * wider rows (the 1M-column decode): the row is cut into chunks handled by
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
    uint32_t sel[3];
    uint32_t flags_cnt[2][2 * kWaves];
    uint32_t seg_start[kMaxSegs + 1];
};

// Set bits of m below this lane.
__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over the wave (lane i: lanes 0..i) in registers: DPP shifts within each
// row of 16 lanes, then the row broadcasts of lanes 15 and 31 (rows 1, 3 and 2, 3).
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Sum over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_incl(x), 63);
}

// Block-wide exclusive suffix sum (sum of v over threads with a larger index).
__device__ __forceinline__ uint32_t block_suffix_excl(uint32_t v, Lds& s) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t incl = wave_prefix_incl(v);
    const uint32_t wtotal = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (lane == 0) s.wave_tot[wave] = wtotal;
    __syncthreads();
    uint32_t later = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) later += w > wave ? s.wave_tot[w] : 0u;
    __syncthreads();
    return later + (wtotal - incl);
}

// Scanning bins from the top, the bin where the running count first reaches
// `need` (>= 1) and the count in the bins above it; returns the count over all
// bins (bin and above_out are meaningful only when it is >= need).
__device__ __forceinline__ uint32_t find_bin_total(Lds& s, int nbins, uint32_t need, uint32_t& bin,
                                                   uint32_t& above_out) {
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
    if (t == 0) s.sel[2] = above + local;
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
    const uint32_t total = s.sel[2];
    __syncthreads();
    return total;
}

__device__ __forceinline__ void find_bin(Lds& s, int nbins, uint32_t need, uint32_t& bin, uint32_t& above_out) {
    (void)find_bin_total(s, nbins, need, bin, above_out);
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
    uint32_t b1 = (uint32_t)known_b1, above1 = known_above1;
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
        total = find_bin_total(s, 4096, k, b1, above1);  // b1, above1 used only when total > k
    }
    const bool select_all = total <= k;
    uint32_t T = 0, n_gt = 0;
    if (!select_all) {
        uint32_t b2, above2, b3, above3;
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
    uint32_t b1 = 0, above = 0;
    const uint32_t total = find_bin_total(s, 4096, k, b1, above);
    if (total <= k) b1 = above = 0;
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

// One workgroup per score row of at most kRegCols columns, read once.  Thread
// (w, l) owns columns 256 J w + 256 j + 4 l + e (j < J, e < 4; J = 4, 8 or 16
// as the width needs), each load instruction covering 1 KiB of the row.  A
// column that is not valid (past the visible prefix, or of a candidate block
// that is -1 or not yet visible) gets key 0, below every valid key (a valid
// key is at least 0x007fffff, bin 7).
//
// Bin floor F: the k-th largest valid key T lies in a bin >= F, where
//   * k <= kThreads: F is the bin of the k-th largest of the threads' largest
//     bins -- k threads hold a key in a bin >= F, k distinct columns, so T is
//     in such a bin too.  This costs one LDS atomic per thread instead of one
//     per key: an LDS atomic wave instruction keeps the CU's LDS busy for about
//     25 cycles, and counting every key was half of a 64K-wide row's select;
//   * otherwise -- k > kThreads, fewer than k threads hold a valid key, or more
//     than kLdsCand keys lie in bins >= the first F -- F is the bin of the k-th
//     largest key from the histogram of every key (1, every valid key, when
//     there are at most k).
// The valid keys in bins >= F -- every key >= T is among them -- are compacted
// in column order into LDS (per wave in (j, lane, e) order, lane offsets from
// three bit-plane ballots of the lane counts, waves in turn) and select_core
// finishes there.  J = 16 keeps only the 12-bit bins, two to a register, and
// reads the candidates' scores again (a few per cent of the row, from L2).
// More than kLdsCand candidates even then (heavy ties): select_core over the
// row in memory, as in topk_select_kernel.
//
// BLK: 0 FULL validity (the visible prefix); 8 candidate blocks of 8 rows (the
// four columns of a load are in one block: one id per load); 1 candidate
// blocks of any height (one id per column).
constexpr int kRegCols = kThreads * 64;

template <int J, int BLK>
__global__ __launch_bounds__(kThreads) void topk_regs_kernel(const TopkParams p) {
    constexpr bool kKeys = J <= 8;  // full keys in registers (else bins, two per register)
    constexpr int kHeld = kKeys ? 4 * J : 2 * J;
    __shared__ Lds s;
    __shared__ uint32_t lkeys[kLdsCand];
    __shared__ int32_t lcols[kLdsCand];
    __shared__ uint32_t wtot[kWaves];
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const RowSrc<kSrcScores> src = row_src<kSrcScores>(p, r);
    const int n = src.n;  // FULL: the visible prefix within the row; blocks: the width
    const int64_t nv = src.nv;
    const uint32_t k = (uint32_t)p.k;
    const int cbase = 256 * J * wave + 4 * lane;
    // the n columns as a buffer: loads past them return zeros, so none needs a branch
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(src.srow), (short)0, (n > 0 ? n : 0) * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(BLK != 0 ? p.cand + (int64_t)r * p.n_blocks : p.cand), (short)0,
        BLK != 0 ? p.n_blocks * 4 : 0, 0x00020000);
    for (int b = tid; b < 4096; b += kThreads) s.hist[b] = 0u;
    uint32_t held[kHeld];  // keys of columns (j, e) at 4 j + e, or their bins at (4 j + e) / 2, half (4 j + e) % 2
    uint32_t mx = 0;       // largest bin of this thread's valid keys (0: none)
    // Loads in groups of at most 8 (16 with BLK 8 would hold 80 registers of loads at once).
    constexpr int JH = J < 8 ? J : 8;
#pragma unroll
    for (int h = 0; h < J; h += JH) {
        u32x4 v[JH];
        int32_t ids[JH];
#pragma unroll
        for (int jj = 0; jj < JH; ++jj)
            v[jj] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (cbase + 256 * (h + jj)), 0, 0));
        if (BLK == 8) {
#pragma unroll
            for (int jj = 0; jj < JH; ++jj)
                ids[jj] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rc, 4 * ((cbase + 256 * (h + jj)) >> 3), 0, 0);
        }
#pragma unroll
        for (int jj = 0; jj < JH; ++jj) {
            const int j = h + jj;
            // BLK 8: rows t < lim of this load's block are visible (0 for a slot of -1)
            int lim = 8;
            if (BLK == 8) {
                const int64_t rem = nv - (int64_t)ids[jj] * 8;
                lim = ids[jj] < 0 ? 0 : (rem >= 8 ? 8 : (rem <= 0 ? 0 : (int)rem));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = cbase + 256 * j + e;
                bool ok = c < n;
                if (BLK == 8) {
                    ok = ok & ((c & 7) < lim);
                } else if (BLK == 1) {
                    const int bi = c / p.block_rows;
                    const int32_t id = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rc, 4 * bi, 0, 0);
                    ok = ok & (id >= 0) & ((int64_t)id * p.block_rows + (c - bi * p.block_rows) < nv);
                }
                const uint32_t key = order_key(__uint_as_float(v[jj][e])) & (0u - (uint32_t)ok);
                mx = max(mx, key >> 20);
                if (kKeys) held[4 * j + e] = key;
                else if (e & 1) held[(4 * j + e) / 2] |= (key >> 20) << 16;
                else held[(4 * j + e) / 2] = key >> 20;
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the next group's loads behind this group's use
    }
    auto bin_at = [&](int j, int e) -> uint32_t {
        if (kKeys) return held[4 * j + e] >> 20;
        return (held[(4 * j + e) / 2] >> (16 * (e & 1))) & 0xffffu;
    };
    // Keys in bins >= fb: this thread's offset among them (column order) and their count.
    auto count_floor = [&](uint32_t fb, uint32_t& off_out, uint32_t& n_out) {
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) mine += bin_at(j, e) >= fb ? 1u : 0u;
        const uint32_t wsum = wave_sum(mine);
        if (lane == 0) wtot[wave] = wsum;
        __syncthreads();
        uint32_t o = 0, all = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t t = wtot[w];
            o += w < wave ? t : 0u;
            all += t;
        }
        off_out = o;
        n_out = all;
    };
    // The floor from the threads' largest bins (k <= kThreads); from every key when k is larger,
    // fewer than k threads hold a valid key, or more than kLdsCand keys lie above the first floor.
    uint32_t floor_bin = 1, off = 0, n_cand = 0, above_unused;
    bool fits = false;
    if (k <= (uint32_t)kThreads) {
        __syncthreads();  // histogram cleared
        if (mx != 0u) atomicAdd(&s.hist[mx], 1u);
        __syncthreads();
        if (find_bin_total(s, 4096, k, floor_bin, above_unused) >= k) {
            count_floor(floor_bin, off, n_cand);
            fits = n_cand <= (uint32_t)kLdsCand;
        }
        if (!fits)
            for (int b = tid; b < 4096; b += kThreads) s.hist[b] = 0u;
    }
    if (!fits) {
        __syncthreads();  // histogram cleared
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (bin_at(j, e) != 0u) atomicAdd(&s.hist[bin_at(j, e)], 1u);
        __syncthreads();
        uint32_t fb;
        // at most k valid keys: floor 1, every one of them (bin >= 7; bin 0 is not valid)
        floor_bin = find_bin_total(s, 4096, k, fb, above_unused) >= k ? fb : 1u;
        count_floor(floor_bin, off, n_cand);
        if (n_cand > (uint32_t)kLdsCand) {
            select_core(src, p, r, s);
            return;
        }
    }
    auto take = [&](uint32_t bin) { return bin >= floor_bin; };
    // the columns again, from a value the compiler cannot match with the first pass's (it would
    // otherwise keep all the column numbers alive across the histogram, in scratch)
    int cb = cbase;
    asm volatile("" : "+v"(cb));
#pragma unroll
    for (int j = 0; j < J; ++j) {
        uint32_t cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) cnt += take(bin_at(j, e)) ? 1u : 0u;
        const uint64_t p0 = __ballot(cnt & 1u), p1 = __ballot(cnt & 2u), p2 = __ballot(cnt & 4u);
        uint32_t at = off + mbcnt64(p0) + 2u * mbcnt64(p1) + 4u * mbcnt64(p2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (take(bin_at(j, e))) {
                lcols[at] = cb + 256 * j + e;
                if (kKeys) lkeys[at] = held[4 * j + e];
                ++at;
            }
        }
        off += (uint32_t)(__builtin_popcountll(p0) + 2 * __builtin_popcountll(p1) + 4 * __builtin_popcountll(p2));
    }
    __syncthreads();
    if (!kKeys) {
        // the candidates' full keys, from their scores (read again: the row has just gone through L2)
        for (int i = tid; i < (int)n_cand; i += kThreads) lkeys[i] = order_key(src.srow[lcols[i]]);
        __syncthreads();
    }
    LdsCandSrc lsrc;
    lsrc.keys = lkeys;
    lsrc.cols = lcols;
    lsrc.n = (int)n_cand;
    select_core(lsrc, p, r, s);
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

// Rows up to this width take one workgroup per row (topk_regs_kernel where it applies): no
// histogram from the indexer and no workspace.
#ifndef CSA2_TOPK_REGS_MAX
#define CSA2_TOPK_REGS_MAX 65536
#endif
static_assert(CSA2_TOPK_REGS_MAX <= kRegCols, "row kernel width");

size_t topk_workspace_bytes(int rows, int64_t width) {
    if (width <= CSA2_TOPK_REGS_MAX) return 0;
    int chunk, nseg;
    topk_plan(rows, width, chunk, nseg, kSweep);
    if (nseg == 0) return 0;
    return align256((size_t)rows * 4096 * 4) + align256((size_t)rows * nseg * 4) +
           2 * align256((size_t)rows * nseg * kCap * 4);
}

template <int J>
static void launch_regs_j(const TopkParams& p, int rows, hipStream_t stream) {
    if (p.n_blocks == 0)
        hipLaunchKernelGGL((topk_regs_kernel<J, 0>), dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
    else if (p.block_rows == 8)
        hipLaunchKernelGGL((topk_regs_kernel<J, 8>), dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((topk_regs_kernel<J, 1>), dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
}

template <int SRC>
static hipError_t launch_topk_src(const TopkParams& p, int rows, void* ws, hipStream_t stream) {
    int chunk = 0, nseg = 0;
    if (p.width > CSA2_TOPK_REGS_MAX) topk_plan(rows, p.width, chunk, nseg, kSweep);
    if (nseg == 0) {
        if (SRC == kSrcScores && p.width > 0 && p.width <= kRegCols && p.width % 4 == 0 &&
            reinterpret_cast<uintptr_t>(p.scores) % 16 == 0) {
            if (p.width <= 16 * kThreads) launch_regs_j<4>(p, rows, stream);
            else if (p.width <= 32 * kThreads) launch_regs_j<8>(p, rows, stream);
            else launch_regs_j<16>(p, rows, stream);
        } else {
            hipLaunchKernelGGL(topk_select_kernel<SRC>, dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
        }
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

// Per-row top-k of indexer scores for gfx950 (one 1024-thread workgroup per row).
//
// Contract ("DeepSeek-V4.1-Flash 架构解剖", fig. 2d REUSE and special module
// "indexer"): the k valid columns with the largest scores, ties to the lower
// column, NaN ranked as -inf, -0 equal to +0; written in increasing column
// order as plane rows, then -1 padding.
//
// Method: exact radix select on a 32-bit order-preserving key, then one
// ordered compaction pass.
//   key(s) = bits(s) | 0x80000000 for s >= +0, ~bits(s) for s < 0, after
//   mapping NaN to -inf and -0 to +0, so key order == score order.
//   Passes 1-3 histogram bits [31:20], [19:8] and [7:0] of the keys that share
//   the prefix found so far (4096/4096/256 LDS bins) and fix, digit by digit,
//   the k-th largest key T and the count n_gt of keys above it.
//   The compaction walks the row in column order, 1024 columns at a time; a
//   column is taken if key > T, or key == T and fewer than k - n_gt equal keys
//   precede it.  Its output slot is (#greater before it) + min(#equal before
//   it, k - n_gt), computed with wave ballots and one barrier per chunk, so the
//   output is already in column order with no sort.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN -> -inf
    if (u == 0x80000000u) u = 0u;                           // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Validity and plane row of column c.
__device__ __forceinline__ bool col_valid(const TopkParams& p, int r, int c, int64_t nv, int32_t& row) {
    if (p.n_blocks == 0) {
        row = c;
        return c < nv;
    }
    const int i = c / p.block_rows;
    const int t = c - i * p.block_rows;
    const int32_t b = p.cand[(int64_t)r * p.n_blocks + i];
    if (b < 0) return false;
    const int64_t jr = (int64_t)b * p.block_rows + t;
    row = (int32_t)jr;
    return jr < nv;
}

// Block-wide exclusive suffix sum: returns sum of v over threads with a larger index.
__device__ __forceinline__ uint32_t block_suffix_excl(uint32_t v, uint32_t* wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // inclusive suffix scan within the wave (lane l gets sum over lanes >= l)
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_down(x, o, 64);
        if (lane + o < 64) x += y;
    }
    if (lane == 0) wave_tot[wave] = x;
    __syncthreads();
    uint32_t later = 0;
    for (int w = wave + 1; w < kWaves; ++w) later += wave_tot[w];
    __syncthreads();
    return later + x - v;
}

// Finds the bin b (scanning bins from the top) where the running count first
// reaches `need`; each thread owns bins [nb_per*t, nb_per*t + nb_per).
// Returns through LDS: sel[0] = bin, sel[1] = count of keys in higher bins.
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nbins, uint32_t need, uint32_t* wave_tot,
                                         uint32_t* sel) {
    const int per = nbins / kThreads;  // 4 or (for 256 bins) 0 -> handled below
    const int t = threadIdx.x;
    uint32_t local = 0;
    int b0 = 0, b1 = 0;
    if (per > 0) {
        b0 = per * t;
        b1 = b0 + per;
    } else if (t < nbins) {
        b0 = t;
        b1 = t + 1;
    }
    for (int b = b0; b < b1; ++b) local += hist[b];
    uint32_t above = block_suffix_excl(local, wave_tot);
    for (int b = b1 - 1; b >= b0; --b) {
        const uint32_t h = hist[b];
        if (above < need && above + h >= need) {
            sel[0] = (uint32_t)b;
            sel[1] = above;
        }
        above += h;
    }
    __syncthreads();
}

}  // namespace

__global__ __launch_bounds__(kThreads) void topk_select_kernel(const TopkParams p) {
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t wave_tot[kWaves];
    __shared__ uint32_t sel[2];
    __shared__ uint32_t flags_cnt[2][2 * kWaves];

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t nv = (p.pos[r] + 1) / p.ratio;
    const float* srow = p.scores + (int64_t)r * p.width;
    int32_t* orow = p.out + (int64_t)r * p.k;
    const int ncols = (p.n_blocks == 0) ? (int)(nv < p.width ? nv : p.width) : (int)p.width;
    const uint32_t k = (uint32_t)p.k;

    // ---- pass 1: top 12 bits -------------------------------------------------
    for (int b = tid; b < 4096; b += kThreads) hist[b] = 0;
    __syncthreads();
    for (int c = tid; c < ncols; c += kThreads) {
        int32_t row;
        if (col_valid(p, r, c, nv, row)) atomicAdd(&hist[order_key(srow[c]) >> 20], 1u);
    }
    __syncthreads();
    // total valid columns
    {
        uint32_t local = hist[4 * tid] + hist[4 * tid + 1] + hist[4 * tid + 2] + hist[4 * tid + 3];
        uint32_t later = block_suffix_excl(local, wave_tot);
        if (tid == 0) sel[0] = later + local;
        __syncthreads();
    }
    const uint32_t total = sel[0];
    __syncthreads();

    bool select_all = total <= k;
    uint32_t T = 0, n_gt = 0;
    if (!select_all) {
        find_bin(hist, 4096, k, wave_tot, sel);
        const uint32_t b1 = sel[0];
        const uint32_t above1 = sel[1];
        __syncthreads();
        // ---- pass 2: bits [19:8] among keys with top bits b1 ----------------------
        for (int b = tid; b < 4096; b += kThreads) hist[b] = 0;
        __syncthreads();
        for (int c = tid; c < ncols; c += kThreads) {
            int32_t row;
            if (col_valid(p, r, c, nv, row)) {
                const uint32_t key = order_key(srow[c]);
                if ((key >> 20) == b1) atomicAdd(&hist[(key >> 8) & 0xfffu], 1u);
            }
        }
        __syncthreads();
        find_bin(hist, 4096, k - above1, wave_tot, sel);
        const uint32_t b2 = sel[0];
        const uint32_t above2 = sel[1];
        __syncthreads();
        // ---- pass 3: bits [7:0] among keys with prefix (b1, b2) -------------------
        const uint32_t pre = (b1 << 12) | b2;
        for (int b = tid; b < 256; b += kThreads) hist[b] = 0;
        __syncthreads();
        for (int c = tid; c < ncols; c += kThreads) {
            int32_t row;
            if (col_valid(p, r, c, nv, row)) {
                const uint32_t key = order_key(srow[c]);
                if ((key >> 8) == pre) atomicAdd(&hist[key & 0xffu], 1u);
            }
        }
        __syncthreads();
        find_bin(hist, 256, k - above1 - above2, wave_tot, sel);
        const uint32_t b3 = sel[0];
        const uint32_t above3 = sel[1];
        __syncthreads();
        T = (pre << 8) | b3;
        n_gt = above1 + above2 + above3;
    }
    const uint32_t need = select_all ? 0u : k - n_gt;  // equal keys to take, lowest columns first
    const uint32_t goal = select_all ? total : k;

    // ---- ordered compaction ---------------------------------------------------
    uint32_t gt_base = 0, eq_base = 0;
    int buf = 0;
    for (int cs = 0; cs < ncols; cs += kThreads) {
        const int c = cs + tid;
        int32_t row = -1;
        bool gt = false, eq = false;
        if (c < ncols && col_valid(p, r, c, nv, row)) {
            if (select_all) {
                gt = true;
            } else {
                const uint32_t key = order_key(srow[c]);
                gt = key > T;
                eq = key == T;
            }
        }
        const uint64_t mgt = __ballot(gt);
        const uint64_t meq = __ballot(eq);
        const uint32_t lo_mask_lo = (uint32_t)(mgt), lo_mask_hi = (uint32_t)(mgt >> 32);
        const uint32_t gt_lane = __builtin_amdgcn_mbcnt_hi(lo_mask_hi, __builtin_amdgcn_mbcnt_lo(lo_mask_lo, 0u));
        const uint32_t eq_lane =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(meq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)meq, 0u));
        if (lane == 0) {
            flags_cnt[buf][wave] = (uint32_t)__builtin_popcountll(mgt);
            flags_cnt[buf][kWaves + wave] = (uint32_t)__builtin_popcountll(meq);
        }
        __syncthreads();
        uint32_t gt_before = gt_base, eq_before = eq_base, gt_all = 0, eq_all = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t a = flags_cnt[buf][w], b = flags_cnt[buf][kWaves + w];
            if (w < wave) {
                gt_before += a;
                eq_before += b;
            }
            gt_all += a;
            eq_all += b;
        }
        gt_before += gt_lane;
        eq_before += eq_lane;
        if (gt || (eq && eq_before < need)) {
            const uint32_t slot = gt_before + (eq_before < need ? eq_before : need);
            orow[slot] = row;
        }
        gt_base += gt_all;
        eq_base += eq_all;
        buf ^= 1;
        const uint32_t done = gt_base + (eq_base < need ? eq_base : need);
        if (done >= goal) break;
    }
    for (int i = (int)goal + tid; i < p.k; i += kThreads) orow[i] = -1;
}

hipError_t launch_topk_select(const TopkParams& p, int rows, hipStream_t stream) {
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace csa2

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
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

namespace {

// ReLU as an integer max on the float's bits: every negative float and -0 has
// a negative signed pattern and becomes +0; +0, positive values and +inf are
// unchanged.  One instruction, where fmaxf would also canonicalise NaNs.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

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
        st.sc = p.scale;
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
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc_sum += wr[t][rr] * relu_bits(acc[rr]);
            }
            v[u] = acc_sum;
        }
        // Reduce over the 4 lane groups and scatter so that lane l ends with column cb + l.
        const bool hi = (lane & 32) != 0;
        const bool mid = (lane & 16) != 0;
        float k0 = hi ? v[2] : v[0];
        float k1 = hi ? v[3] : v[1];
        k0 += shfl_xor(hi ? v[0] : v[2], 32);
        k1 += shfl_xor(hi ? v[1] : v[3], 32);
        float kk = mid ? k1 : k0;
        kk += shfl_xor(mid ? k0 : k1, 16);
        const int64_t c_out = cb + lane;
        const float score = st.valid ? st.sc * kk : kNegInf;
        if (c_out < c_end) {
            srow[c_out] = score;
            if (HIST && st.valid) atomicAdd(&hist[order_key(score) >> 20], 1u);
        }
        if (BMAX) {
            // Block score over bm_rows consecutive columns = lanes (blocks never
            // straddle a 64-column step): NaN as -inf, infinities clipped, invalid
            // columns -inf; the block of the newest visible row is pinned to +inf.
            float bm = st.valid ? pool_value(score) : kNegInf;
            for (int o = 1; o < p.bm_rows; o <<= 1) bm = fmaxf(bm, shfl_xor(bm, o));
            if ((lane & (p.bm_rows - 1)) == 0 && c_out < c_end) {
                const int64_t blk = c_out / p.bm_rows;
                p.block_max[(int64_t)r * p.bm_blocks + blk] = (blk == (nv - 1) / p.bm_rows) ? kPosInf : bm;
            }
        }
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
    for (; cb < c_end; cb += 256) {  // nothing visible in these columns
        const int64_t c_out = cb + lane;
        if (c_out < c_end) srow[c_out] = kNegInf;
        if (BMAX && (lane & (p.bm_rows - 1)) == 0 && c_out < c_end)
            p.block_max[(int64_t)r * p.bm_blocks + c_out / p.bm_rows] = kNegInf;
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

hipError_t launch_indexer_score(const IndexParams& p, int rows, int heads, int dim, int dtype, bool reindex,
                                hipStream_t stream) {
    if (heads == 64 && dim == 128) {
        if (dtype == CSA2_BF16) return reindex ? launch_one<CSA2_BF16, 64, 128, true>(p, rows, stream)
                                               : launch_one<CSA2_BF16, 64, 128, false>(p, rows, stream);
        if (dtype == CSA2_FP8_E4M3) return reindex ? launch_one<CSA2_FP8_E4M3, 64, 128, true>(p, rows, stream)
                                                   : launch_one<CSA2_FP8_E4M3, 64, 128, false>(p, rows, stream);
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

bool indexer_supported(int heads, int dim, int dtype) {
    if (heads == 64 && dim == 128) return dtype == CSA2_BF16 || dtype == CSA2_FP8_E4M3 || dtype == CSA2_F32;
    if (heads == 4 && dim == 32) return dtype == CSA2_F32 || dtype == CSA2_BF16;
    return false;
}

}  // namespace csa2

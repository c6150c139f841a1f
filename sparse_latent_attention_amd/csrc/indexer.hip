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
template <bool HIST, bool BMAX>
__device__ __forceinline__ void store_step(const IndexParams& p, int r, int64_t nv, int64_t cb, int64_t c_end,
                                           int lane, const float (&v)[4], float sc, bool valid, float* srow,
                                           uint32_t* hist) {
    const bool hi = (lane & 32) != 0;
    const bool mid = (lane & 16) != 0;
    float k0 = hi ? v[2] : v[0];
    float k1 = hi ? v[3] : v[1];
    k0 += shfl_xor(hi ? v[0] : v[2], 32);
    k1 += shfl_xor(hi ? v[1] : v[3], 32);
    float kk = mid ? k1 : k0;
    kk += shfl_xor(mid ? k0 : k1, 16);
    const int64_t c_out = cb + lane;
    const float score = valid ? sc * kk : kNegInf;
    if (c_out < c_end) {
        srow[c_out] = score;
        if (HIST && valid) atomicAdd(&hist[order_key(score) >> 20], 1u);
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

// Columns of a workgroup beyond the visible prefix: -inf scores, -inf block scores.
template <bool BMAX>
__device__ __forceinline__ void store_invisible(const IndexParams& p, int r, int64_t cb, int64_t c_end, int lane,
                                                float* srow) {
    const int64_t c_out = cb + lane;
    if (c_out < c_end) srow[c_out] = kNegInf;
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

// Steps of key-row loads each wave keeps in flight in the FP8 FULL kernel, and
// the most 64-column steps one wave makes (a workgroup covers <= 4096 columns).
constexpr int kFp8Depth = 2;
constexpr int kFp8MaxSteps = 16;

// FP8 FULL scoring with coalesced, non-temporal key-row loads.
//
// A FULL row's key rows are contiguous in the plane, so a wave's 64-key step is
// one 8 KiB span.  Each lane loads 8 x 16 B of it (instruction j covers keys
// 8j..8j+7 completely: whole 128-byte lines, non-temporal, since each byte is
// read once), writes them to its wave's LDS slot and reads them back in the
// MFMA B-operand layout (lane (g, n) of tile u: key 16u + n, bytes 16g and
// 64 + 16g -- the k order of the query fragments).  Chunk c of key kk sits at
// position c ^ ((kk >> 1) & 7) of its 128-byte LDS row, which keeps both the
// writes and the reads free of bank conflicts.
//
// Loads go through buffer descriptors that cover exactly the workgroup's
// visible key rows (and their scales): a load past the visible prefix returns
// zeros instead of touching memory, so no address is clamped and no branch
// guards a load.  The per-lane offset is fixed for the whole launch and the
// step offset is a scalar.  DEPTH steps of loads are in flight per wave while
// the matrix cores work on the step in LDS.
template <bool HIST, bool BMAX, int DEPTH>
__global__ __launch_bounds__(256) void indexer_fp8_full_kernel(const IndexParams p) {
    __shared__ uint32_t hist[HIST ? kKeyBins : 1];
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][64 * 128];
    typedef IdxOps<CSA2_FP8_E4M3, 128> Ops;
    typedef Ops::Frag Frag;
    constexpr int HI = 64, HT = 4;
    constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9-family descriptor
    constexpr int kNT = 2;                  // non-temporal cache policy

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

    Frag qa[HT];
    float wr[HT][4];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        qa[t] = Ops::load(p.q, (int64_t)r * HI + 16 * t + li, 0, g);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) wr[t][rr] = p.w[(int64_t)r * HI + 16 * t + 4 * g + rr];
    }
    if (HIST) {
        for (int b = threadIdx.x; b < kKeyBins; b += 256) hist[b] = 0u;
        __syncthreads();
    }

    // Descriptors over this workgroup's visible rows [c_begin, c_live).
    const int n_live = c_live > c_begin ? (int)(c_live - c_begin) : 0;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.k) + (base + c_begin) * 128), (short)0, n_live * 128,
        kRsrcWord3);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.k_scale + base + c_begin), (short)0, n_live * 4, kRsrcWord3);
    const int ksub = lane >> 3, kchunk = lane & 7;
    const int voff = ksub * 128 + kchunk * 16;

    struct Buf {
        u32x4 v[8];
        float sc;
    };
    auto issue = [&](int64_t cb, Buf& b) {
        const int so = (int)(cb - c_begin) * 128;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            b.v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, voff, so + 1024 * j, kNT));
        b.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, lane * 4, (int)(cb - c_begin) * 4, 0));
    };
    auto step = [&](int64_t cb, Buf& b) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kk = 8 * j + ksub;
            *reinterpret_cast<u32x4*>(my + kk * 128 + 16 * (kchunk ^ ((kk >> 1) & 7))) = b.v[j];
        }
        const float sc = p.scale * b.sc;
        const bool valid = cb + lane < c_live;
        // Unconditional: past the visible rows the descriptor turns the loads into zeros
        // (a conditional issue would make the compiler drain every load at the join).
        issue(cb + 256 * DEPTH, b);
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kk = 16 * u + li;
            const int sw = (kk >> 1) & 7;
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(my + kk * 128 + 16 * (g ^ sw));
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(my + kk * 128 + 16 * ((g + 4) ^ sw));
            Frag kb;
            kb[0] = a0[0]; kb[1] = a0[1]; kb[2] = a0[2]; kb[3] = a0[3];
            kb[4] = a1[0]; kb[5] = a1[1]; kb[6] = a1[2]; kb[7] = a1[3];
            float acc_sum = 0.f;
#pragma unroll
            for (int t = 0; t < HT; ++t) {
                const f32x4 acc = Ops::mma(f32x4{0.f, 0.f, 0.f, 0.f}, qa[t], kb);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc_sum += wr[t][rr] * relu_bits(acc[rr]);
            }
            v[u] = acc_sum;
        }
        store_step<HIST, BMAX>(p, r, nv, cb, c_end, lane, v, sc, valid, srow, hist);
    };

    // At most kFp8MaxSteps steps per wave (cols_per_wg <= 256 * kFp8MaxSteps): the step
    // loop is unrolled completely, so the compiler's memory-counter waits see the
    // loads in flight exactly instead of draining them at a loop back edge.
    const int64_t cb0 = c_begin + 64 * wave;
    Buf bufs[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(cb0 + 256 * d, bufs[d]);
#pragma unroll
    for (int it = 0; it < kFp8MaxSteps; ++it) {
        const int64_t cb = cb0 + 256 * it;
        if (cb >= c_live) break;
        step(cb, bufs[it % DEPTH]);
    }
    int64_t cb = cb0;
    if (c_live > cb0) cb += 256 * ((c_live - cb0 + 255) / 256);
    for (; cb < c_end; cb += 256) store_invisible<BMAX>(p, r, cb, c_end, lane, srow);
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

static hipError_t launch_fp8_full(const IndexParams& p, int rows, hipStream_t stream) {
    if (p.cols_per_wg > 256 * kFp8MaxSteps || p.cols_per_wg % 256 != 0) return hipErrorInvalidValue;
    const int64_t chunks = (p.width + p.cols_per_wg - 1) / p.cols_per_wg;
    dim3 grid((unsigned)chunks, (unsigned)rows);
    const bool hist = p.key_hist != nullptr;
    if (hist) {
        const int64_t nh = (int64_t)rows * kKeyBins;
        hipLaunchKernelGGL(key_hist_zero_kernel, dim3((unsigned)((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024)),
                           dim3(256), 0, stream, p.key_hist, nh);
    }
    constexpr int D = kFp8Depth;
    if (p.block_max != nullptr) {
        if (hist) hipLaunchKernelGGL((indexer_fp8_full_kernel<true, true, D>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((indexer_fp8_full_kernel<false, true, D>), grid, dim3(256), 0, stream, p);
    } else {
        if (hist) hipLaunchKernelGGL((indexer_fp8_full_kernel<true, false, D>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((indexer_fp8_full_kernel<false, false, D>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_indexer_score(const IndexParams& p, int rows, int heads, int dim, int dtype, bool reindex,
                                hipStream_t stream) {
    if (heads == 64 && dim == 128) {
        if (dtype == CSA2_BF16) return reindex ? launch_one<CSA2_BF16, 64, 128, true>(p, rows, stream)
                                               : launch_one<CSA2_BF16, 64, 128, false>(p, rows, stream);
        if (dtype == CSA2_FP8_E4M3) return reindex ? launch_one<CSA2_FP8_E4M3, 64, 128, true>(p, rows, stream)
                                                   : launch_fp8_full(p, rows, stream);
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

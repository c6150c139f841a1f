// The FULL layer's write path for gfx950: compressor, main row and index key.
//
// For the token rows of one call ("万字长文解析DeekSeekV4.1flash" appendix
// A.15.1; "DeepSeek-V4.1-Flash 架构解剖", special modules "compressor" and
// "indexer", key side; "DeepSeek-V4.1-Flash 结构说明" §4):
//   kv = wkv . x, score = wgate . x (ratio 2)               [512] each, FP32
//   latent_j = RMSNorm(per-channel softmax(score) pooling of kv over the
//              group's ratio positions) * norm_w             (ratio 1: RMSNorm(kv))
//   main row j  = latent_j with its last 64 dims rotated at position j*ratio
//   index key j = RMSNorm(wk . latent_j) * knorm_w, last 64 dims rotated alike
// then both are quantised into their planes at row row_base + j.  A group whose
// second token is not in the call waits in the sequence's FP32 tail state.
//
// Three kernels:
//  * compress_project_kernel: the projections, a bf16 x bf16 -> f32 GEMM on
//    MFMA (16x16x32).  A workgroup owns a 64-row x 64-column output tile; each
//    wave one 16-column slice of it (four 16-row tiles).  Operands go straight
//    from memory into registers in the MFMA layout (lane (g, n) holds 8
//    consecutive k of row n: 16 contiguous bytes).  With few rows (decode) the
//    K range is split over workgroups so the weights, the dominant bytes, are
//    streamed by enough of them; partial tiles go to a workspace and are added
//    in a fixed order, so the result does not depend on scheduling.  At
//    prefill sizes (many rows, no split) compress_gemm_kernel takes the
//    projections instead: 128 x 128 output tiles with both operands staged
//    through LDS, so each fragment read feeds several MFMAs.
//  * compress_finish_kernel: one workgroup per token row: pooling with its
//    group partner (the previous row of the call, or the tail state), the two
//    RMSNorms, the 128 x 512 index-key projection (thread pairs split each
//    output's dot product), the rotations (angles in float64) and the
//    quantisation.  Every rounding decision is taken from float32 values with
//    correctly rounded operations (IEEE division), and the roundings
//    themselves are integer operations on the float32 bits written from the
//    format definitions.
//  * compress_tail_kernel (ratio 2): stores the pending first token of a group
//    that the call does not complete, after every row has read the tail state
//    the call started with.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

namespace {

constexpr int kLatent = 512;
constexpr int kKey = 128;
constexpr int kRope = 64;

// ---- format roundings (OCP 8-bit FP, OCP Microscaling v1.0) ----------------

// float32 -> E4M3-FN code: nearest, ties to the even code, saturating at +-448
// (infinities too); NaN -> 0x7F with its sign.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;
    if (a >= 0x43e00000u) return sign | 0x7eu;             // |y| >= 448 (464, the tie, goes to 448 too)
    if (a < 0x3c800000u) {                                  // |y| < 2^-6: multiples of 2^-9
        const float q = __uint_as_float(a) * 512.0f;        // exact
        return sign | (uint32_t)__builtin_rintf(q);         // 8 is 2^-6 = code 0x08
    }
    int e = (int)(a >> 23) - 127;                           // -6 .. 8
    uint32_t m = (a >> 20) & 7u;
    const uint32_t rem = a & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) {
        m = 0u;
        ++e;
    }
    uint32_t code = ((uint32_t)(e + 7) << 3) | m;
    if (code > 0x7eu) code = 0x7eu;
    return sign | code;
}

// E4M3-FN code (non-NaN, sign ignored) -> its magnitude.
__device__ __forceinline__ float e4m3_magnitude(uint32_t code) {
    const uint32_t e = (code >> 3) & 15u, m = code & 7u;
    if (e == 0u) return (float)m * 0.001953125f;            // m * 2^-9
    return __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) 2^(e-7)
}

// float32 -> E2M1 code: nearest magnitude, ties to the even code, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
    const float a = fabsf(y);
    uint32_t c;
    if (a <= 0.25f) c = 0u;
    else if (a < 0.75f) c = 1u;
    else if (a <= 1.25f) c = 2u;
    else if (a < 1.75f) c = 3u;
    else if (a <= 2.5f) c = 4u;
    else if (a < 3.5f) c = 5u;
    else if (a <= 5.0f) c = 6u;
    else c = 7u;
    return c | ((__float_as_uint(y) >> 28) & 8u);
}

// E8M0 exponent e = ceil(log2(amax / 6)) clamped to [-127, 127] (-127 for 0);
// returns the biased byte.
__device__ __forceinline__ uint32_t e8m0_for(float amax) {
    const float v = amax / 6.0f;
    const uint32_t b = __float_as_uint(v);
    int e;
    if (v <= 0.0f) e = -127;
    else if ((b >> 23) == 0u) e = -127;                     // subnormal: below 2^-126
    else e = (int)(b >> 23) - 127 + ((b & 0x7fffffu) ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    return (uint32_t)(e + 127);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ float group_max(float v, int lanes) {
    for (int o = 1; o < lanes; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Stores elements (a, b) = (2t, 2t+1) of a row of n elements held by thread t,
// in the plane's format.  A scale group's elements sit in 16 (groups of 32) or
// 8 (groups of 16) consecutive lanes, so its amax is a shuffle reduction; an
// FP8 row (n = 128) is one whole wave.
template <int DT>
__device__ __forceinline__ void store_pair(void* out, void* scale_out, int64_t row, int n, int t, float a, float b) {
    if (DT == CSA2_F32) {
        *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(out) + row * n + 2 * t) = f32x2{a, b};
    } else if (DT == CSA2_BF16) {
        reinterpret_cast<uint32_t*>(out)[row * (n / 2) + t] = pack_bf16x2(a, b);
    } else if (DT == CSA2_FP8_E4M3) {  // one float32 scale per row (a whole row is one wave: n = 128)
        const float amax = group_max(fmaxf(fabsf(a), fabsf(b)), n / 2);
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        const uint32_t c = e4m3_rne(a / sc) | (e4m3_rne(b / sc) << 8);
        reinterpret_cast<uint16_t*>(out)[row * (n / 2) + t] = (uint16_t)c;
        if (t == 0) reinterpret_cast<float*>(scale_out)[row] = sc;
    } else if (DT == CSA2_FP4_E2M1) {  // one E8M0 per 32 elements, planar
        const float amax = group_max(fmaxf(fabsf(a), fabsf(b)), 16);
        const uint32_t e = e8m0_for(amax);
        const float sc = e8m0_to_f32(e);
        reinterpret_cast<uint8_t*>(out)[row * (n / 2) + t] = (uint8_t)(e2m1_rne(a / sc) | (e2m1_rne(b / sc) << 4));
        if ((t & 15) == 0) reinterpret_cast<uint8_t*>(scale_out)[row * (n / 32) + t / 16] = (uint8_t)e;
    } else {  // CSA2_FP4_E2M1_E4M3G16: E2M1 bytes then one E4M3 scale per 16, inline
        const float amax = group_max(fmaxf(fabsf(a), fabsf(b)), 8);
        const float v = fminf(fmaxf(amax / 6.0f, 0.001953125f), 448.0f);
        const uint32_t sc_code = e4m3_rne(v);
        const float sc = e4m3_magnitude(sc_code);
        uint8_t* rp = reinterpret_cast<uint8_t*>(out) + row * (n / 2 + n / 16);
        rp[t] = (uint8_t)(e2m1_rne(a / sc) | (e2m1_rne(b / sc) << 4));
        if ((t & 7) == 0) rp[n / 2 + t / 8] = (uint8_t)sc_code;
    }
}

}  // namespace

// grid (nproj / 64, ceil(rows / 64), ksplit), 256 threads.  (Loading the next
// k step ahead of the matrix cores measured no faster at prefill sizes and
// slower at decode sizes.)
__global__ __launch_bounds__(256) void compress_project_kernel(const CompressParams p, int k_per_split) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int n0 = blockIdx.x * 64 + 16 * wave;
    const int m0 = blockIdx.y * 64;
    const int k0 = blockIdx.z * k_per_split;
    const uint16_t* wrow = (n0 < kLatent ? p.wkv + (int64_t)(n0 + li) * p.d_in
                                         : p.wgate + (int64_t)(n0 - kLatent + li) * p.d_in) + 8 * g;
    const uint16_t* xrow[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        int m = m0 + 16 * t + li;
        if (m >= p.rows) m = p.rows - 1;  // in bounds; the row's results are not stored
        xrow[t] = p.x + (int64_t)m * p.d_in + 8 * g;
    }
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = k0; k < k0 + k_per_split; k += 64) {  // k_per_split is a multiple of 64
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(wrow + k);
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(wrow + k + 32);
        bf16x8 a0[4], a1[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a0[t] = *reinterpret_cast<const bf16x8*>(xrow[t] + k);
            a1[t] = *reinterpret_cast<const bf16x8*>(xrow[t] + k + 32);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = Mma<__bf16>::k32(acc[t], a0[t], b0);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = Mma<__bf16>::k32(acc[t], a1[t], b1);
    }
    // D[4g + rr][li] of tile t: row m0 + 16t + 4g + rr, column n0 + li
    float* part = p.partial + (int64_t)blockIdx.z * p.rows * p.nproj;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = m0 + 16 * t + 4 * g + rr;
            if (m < p.rows) part[(int64_t)m * p.nproj + n0 + li] = acc[t][rr];
        }
}

namespace {

// Columns (col, col + 1) of one row's projections: the split-K partial tiles
// added in the order k = 0, 1, ... (eight loads in flight at a time).  The
// finish and tail kernels both use it, so a tail holds exactly the values
// the row's own group would have used.
__device__ __forceinline__ f32x2 proj2(const CompressParams& p, int row, int col) {
    const float* base = p.partial + (int64_t)row * p.nproj + col;
    if (p.ksplit == 1) return *reinterpret_cast<const f32x2*>(base);
    const int64_t stride = (int64_t)p.rows * p.nproj;
    f32x2 acc{0.f, 0.f};
    for (int k0 = 0; k0 < p.ksplit; k0 += 8) {
        f32x2 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = k0 + e < p.ksplit ? k0 + e : p.ksplit - 1;  // in bounds; not added below
            v[e] = *reinterpret_cast<const f32x2*>(base + k * stride);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (k0 + e < p.ksplit) acc += v[e];
    }
    return acc;
}

}  // namespace

// grid ceil(rows / RPB), 256 threads: RPB consecutive token rows per workgroup
// (the index-key weights are read once for all of them).  Thread t owns latent
// channels 2t, 2t+1 and (t < 64) key elements 2t, 2t+1.
template <int RATIO, int MT, int KT, int RPB>
__global__ __launch_bounds__(256) void compress_finish_kernel(const CompressParams p) {
    __shared__ float lat[RPB][kLatent];
    __shared__ float key[RPB][kKey];
    __shared__ float red[4];
    const int t = threadIdx.x;
    const int c = 2 * t;
    const int r0 = blockIdx.x * RPB;
    // Loads that depend on nothing are issued first, so their latency overlaps
    // the partial sums: the norm weights, the rotation frequencies and, with one
    // row per workgroup (the latency-bound decode shape), this thread's 512 bytes
    // of index-key weights.
    const int ki = t >> 1, kh = t & 1;
    const uint16_t* wr = p.wk + (int64_t)ki * kLatent + 256 * kh;
    constexpr int kPre = RPB == 1 ? 32 : 1;
    u32x4 wv[kPre];
    if constexpr (RPB == 1) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) wv[q] = *reinterpret_cast<const u32x4*>(wr + 8 * q);
    }
    // (with several rows per workgroup these stay at their uses: registers there buy occupancy)
    f32x2 nw_pre{0.f, 0.f}, knw_pre{0.f, 0.f};
    double fm_pre = 0.0, fk_pre = 0.0;
    if constexpr (RPB == 1) {
        nw_pre = *reinterpret_cast<const f32x2*>(p.norm_w + c);
        if (t < kKey / 2) knw_pre = *reinterpret_cast<const f32x2*>(p.knorm_w + 2 * t);
        if (c >= kLatent - kRope) fm_pre = p.inv_freq[(c - (kLatent - kRope)) / 2];
        if (t < kKey / 2 && 2 * t >= kKey - kRope) fk_pre = p.inv_freq[(2 * t - (kKey - kRope)) / 2];
    }
    auto nw = [&](int e) { return RPB == 1 ? nw_pre[e] : p.norm_w[c + e]; };
    auto knw = [&](int e) { return RPB == 1 ? knw_pre[e] : p.knorm_w[2 * t + e]; };
    auto fm = [&]() { return RPB == 1 ? fm_pre : p.inv_freq[(c - (kLatent - kRope)) / 2]; };
    auto fk = [&]() { return RPB == 1 ? fk_pre : p.inv_freq[(2 * t - (kKey - kRope)) / 2]; };
    float lv[RPB][2];
    bool emit[RPB];
    int64_t jj[RPB];
#pragma unroll
    for (int rr = 0; rr < RPB; ++rr) {
        const int r = r0 + rr;
        emit[rr] = false;
        jj[rr] = 0;
        lv[rr][0] = lv[rr][1] = 0.f;
        if (r >= p.rows) continue;  // uniform over the workgroup, as every condition on r below
        const int64_t pos = p.pos[r];
        if (RATIO == 2 && (pos & 1) == 0) continue;  // first token of its group: no row yet
        emit[rr] = true;
        float v0, v1;
        if (RATIO == 1) {
            const f32x2 kv = proj2(p, r, c);
            v0 = kv[0];
            v1 = kv[1];
            jj[rr] = pos;
        } else {
            const int s = p.slot[r];
            const f32x2 kv = proj2(p, r, c), sc = proj2(p, r, kLatent + c);
            f32x2 pk, ps;
            if (r > 0 && p.slot[r - 1] == s && p.pos[r - 1] == pos - 1) {
                pk = proj2(p, r - 1, c);
                ps = proj2(p, r - 1, kLatent + c);
            } else {
                pk = *reinterpret_cast<const f32x2*>(p.tail_kv + (int64_t)s * kLatent + c);
                ps = *reinterpret_cast<const f32x2*>(p.tail_score + (int64_t)s * kLatent + c);
            }
            // per channel, softmax over the group's two positions (first: partner)
            const float m0 = fmaxf(ps[0], sc[0]), m1 = fmaxf(ps[1], sc[1]);
            const float a0 = expf(ps[0] - m0), b0 = expf(sc[0] - m0);
            const float a1 = expf(ps[1] - m1), b1 = expf(sc[1] - m1);
            v0 = (a0 * pk[0] + b0 * kv[0]) / (a0 + b0);
            v1 = (a1 * pk[1] + b1 * kv[1]) / (a1 + b1);
            jj[rr] = pos / 2;
        }
        // RMSNorm of the latent
        const float ss = block_sum(v0 * v0 + v1 * v1, red);
        const float inv = 1.0f / sqrtf(ss / (float)kLatent + p.eps);
        lv[rr][0] = v0 * inv * nw(0);
        lv[rr][1] = v1 * inv * nw(1);
        lat[rr][c] = lv[rr][0];
        lat[rr][c + 1] = lv[rr][1];
    }
    __syncthreads();
    // index keys: output i = t / 2 over channels [256 h, 256 h + 256) of half h = t % 2
    {
        const int h = kh;
        float acc[RPB];
#pragma unroll
        for (int rr = 0; rr < RPB; ++rr) acc[rr] = 0.f;
        auto fma8 = [&](const u32x4& w, int q) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float w0 = bf16_bits_to_f32(w[e] & 0xffffu), w1 = bf16_bits_to_f32(w[e] >> 16);
#pragma unroll
                for (int rr = 0; rr < RPB; ++rr) {
                    if (!emit[rr]) continue;
                    acc[rr] = fmaf(w0, lat[rr][256 * h + q + 2 * e], acc[rr]);
                    acc[rr] = fmaf(w1, lat[rr][256 * h + q + 2 * e + 1], acc[rr]);
                }
            }
        };
        if constexpr (RPB == 1) {
#pragma unroll
            for (int q8 = 0; q8 < kPre; ++q8) fma8(wv[q8], 8 * q8);
        } else {
#pragma unroll 4
            for (int q = 0; q < 256; q += 8) fma8(*reinterpret_cast<const u32x4*>(wr + q), q);
        }
#pragma unroll
        for (int rr = 0; rr < RPB; ++rr) {
            acc[rr] += __shfl_xor(acc[rr], 1, 64);
            if (h == 0) key[rr][ki] = acc[rr];
        }
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RPB; ++rr) {
        if (!emit[rr]) continue;
        const int r = r0 + rr;
        float k0 = 0.f, k1 = 0.f;
        if (t < kKey / 2) {
            k0 = key[rr][2 * t];
            k1 = key[rr][2 * t + 1];
        }
        const float kss = block_sum(k0 * k0 + k1 * k1, red);
        const float kinv = 1.0f / sqrtf(kss / (float)kKey + p.k_eps);
        if (t < kKey / 2) {
            k0 = k0 * kinv * knw(0);
            k1 = k1 * kinv * knw(1);
        }
        // rotation of the last 64 dims at the group's first position
        const int64_t rp = jj[rr] * RATIO;
        float v0 = lv[rr][0], v1 = lv[rr][1];
        if (c >= kLatent - kRope) {
            float cs, sn;
            rope_angle(rp, fm(), cs, sn);
            const float x0 = v0, x1 = v1;
            v0 = x0 * cs - x1 * sn;
            v1 = x0 * sn + x1 * cs;
        }
        if (t < kKey / 2 && 2 * t >= kKey - kRope) {
            float cs, sn;
            rope_angle(rp, fk(), cs, sn);
            const float x0 = k0, x1 = k1;
            k0 = x0 * cs - x1 * sn;
            k1 = x0 * sn + x1 * cs;
        }
        const int64_t row = p.row_base[r] + jj[rr];
        store_pair<MT>(p.main_out, p.main_scale_out, row, kLatent, t, v0, v1);
        if (t < kKey / 2) store_pair<KT>(p.idx_out, p.idx_scale_out, row, kKey, t, k0, k1);
    }
}

// grid rows, 256 threads: the first token of a group that no later row of the
// call completes leaves its kv and score in the sequence's tail state.  A
// kernel of its own, after compress_finish_kernel: that kernel may still read
// the tail state the call started with.
__global__ __launch_bounds__(256) void compress_tail_kernel(const CompressParams p) {
    const int r = blockIdx.x;
    const int s = p.slot[r];
    if ((p.pos[r] & 1) != 0 || (r + 1 < p.rows && p.slot[r + 1] == s)) return;
    const int c = 2 * threadIdx.x;
    *reinterpret_cast<f32x2*>(p.tail_kv + (int64_t)s * kLatent + c) = proj2(p, r, c);
    *reinterpret_cast<f32x2*>(p.tail_score + (int64_t)s * kLatent + c) = proj2(p, r, kLatent + c);
}

bool compress_supported(int main_dtype, int idx_dtype) {
    const bool m = main_dtype == CSA2_F32 || main_dtype == CSA2_BF16 || main_dtype == CSA2_FP4_E2M1 ||
                   main_dtype == CSA2_FP4_E2M1_E4M3G16;
    const bool k = idx_dtype == CSA2_F32 || idx_dtype == CSA2_BF16 || idx_dtype == CSA2_FP8_E4M3 ||
                   idx_dtype == CSA2_FP4_E2M1;
    return m && k;
}

template <int RATIO, int MT, int RPB>
static void launch_finish_k(const CompressParams& p, int idx_dtype, hipStream_t st) {
    const dim3 grid((unsigned)((p.rows + RPB - 1) / RPB));
    switch (idx_dtype) {
        case CSA2_F32:
            hipLaunchKernelGGL((compress_finish_kernel<RATIO, MT, CSA2_F32, RPB>), grid, dim3(256), 0, st, p);
            break;
        case CSA2_BF16:
            hipLaunchKernelGGL((compress_finish_kernel<RATIO, MT, CSA2_BF16, RPB>), grid, dim3(256), 0, st, p);
            break;
        case CSA2_FP8_E4M3:
            hipLaunchKernelGGL((compress_finish_kernel<RATIO, MT, CSA2_FP8_E4M3, RPB>), grid, dim3(256), 0, st, p);
            break;
        default:
            hipLaunchKernelGGL((compress_finish_kernel<RATIO, MT, CSA2_FP4_E2M1, RPB>), grid, dim3(256), 0, st, p);
            break;
    }
}

template <int RATIO, int RPB>
static void launch_finish_m(const CompressParams& p, int main_dtype, int idx_dtype, hipStream_t st) {
    switch (main_dtype) {
        case CSA2_F32: launch_finish_k<RATIO, CSA2_F32, RPB>(p, idx_dtype, st); break;
        case CSA2_BF16: launch_finish_k<RATIO, CSA2_BF16, RPB>(p, idx_dtype, st); break;
        case CSA2_FP4_E2M1: launch_finish_k<RATIO, CSA2_FP4_E2M1, RPB>(p, idx_dtype, st); break;
        default: launch_finish_k<RATIO, CSA2_FP4_E2M1_E4M3G16, RPB>(p, idx_dtype, st); break;
    }
}

// Rows per finish workgroup: several when there are many rows (the index-key
// weights are then read once per group of rows), one otherwise.
template <int RATIO>
static void launch_finish(const CompressParams& p, int main_dtype, int idx_dtype, hipStream_t st) {
    if (p.rows >= 1024) launch_finish_m<RATIO, 4>(p, main_dtype, idx_dtype, st);
    else launch_finish_m<RATIO, 1>(p, main_dtype, idx_dtype, st);
}

// Projection for many rows (a prefill chunk): one workgroup per 128 x 128 tile
// of the [rows, nproj] product, its 4 waves 64 x 64 each.  The x and weight
// rows of a 128-column slice of the reduction are staged in LDS once per
// workgroup (double-buffered; 256-byte rows whose 16-byte chunks are XOR-ed
// with the row's low 4 bits, so the MFMA operand reads hit distinct banks) and
// each operand fragment read from LDS feeds 4 MFMAs; compress_project_kernel
// instead reads every fragment from memory for every wave.  One partial slice
// (no split of the reduction), in the layout the finish kernel reads.
constexpr int kGemmTile = 128;
__device__ __forceinline__ int gemm_off(int row, int c) { return 256 * row + 16 * (c ^ (row & 15)); }

__global__ __launch_bounds__(256) void compress_gemm_kernel(const CompressParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t sa[2][kGemmTile * 256];
    __shared__ __attribute__((aligned(16))) uint8_t sb[2][kGemmTile * 256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * kGemmTile, n0 = blockIdx.x * kGemmTile;

    // Staging: chunk i = tid + 256 j (j < 8) of a 128 x 128 operand slice is 16-byte chunk
    // i % 16 of row i / 16 (consecutive threads read consecutive bytes of a row).
    const uint16_t* arow[8];
    const uint16_t* brow[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int ci = tid + 256 * j, r = ci / 16, c = ci % 16;
        int m = m0 + r;
        if (m >= p.rows) m = p.rows - 1;  // in bounds; such rows' results are not stored
        const int n = n0 + r;
        arow[j] = p.x + (int64_t)m * p.d_in + 8 * c;
        brow[j] = (n < kLatent ? p.wkv + (int64_t)n * p.d_in : p.wgate + (int64_t)(n - kLatent) * p.d_in) + 8 * c;
    }
    auto fetch = [&](int k, u32x4 (&xa)[8], u32x4 (&xb)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            xa[j] = *reinterpret_cast<const u32x4*>(arow[j] + k);
            xb[j] = *reinterpret_cast<const u32x4*>(brow[j] + k);
        }
    };
    auto put = [&](int b, const u32x4 (&xa)[8], const u32x4 (&xb)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int ci = tid + 256 * j;
            *reinterpret_cast<u32x4*>(sa[b] + gemm_off(ci / 16, ci % 16)) = xa[j];
            *reinterpret_cast<u32x4*>(sb[b] + gemm_off(ci / 16, ci % 16)) = xb[j];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        u32x4 xa[8], xb[8];
        fetch(0, xa, xb);
        put(0, xa, xb);
    }
    __syncthreads();
    int b = 0;
    for (int k = 0; k < p.d_in; k += kGemmTile) {
        const bool more = k + kGemmTile < p.d_in;
        u32x4 xa[8], xb[8];
        if (more) fetch(k + kGemmTile, xa, xb);  // in flight during this slice's MFMAs
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                fa[t] = *reinterpret_cast<const bf16x8*>(sa[b] + gemm_off(64 * wm + 16 * t + li, 4 * s + g));
                fb[t] = *reinterpret_cast<const bf16x8*>(sb[b] + gemm_off(64 * wn + 16 * t + li, 4 * s + g));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = Mma<__bf16>::k32(acc[i][j], fa[i], fb[j]);
        }
        if (more) put(b ^ 1, xa, xb);
        __syncthreads();
        b ^= 1;
    }
    // D[4g + rr][li] of tile (i, j): row m0 + 64 wm + 16 i + 4g + rr, column n0 + 64 wn + 16 j + li
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = m0 + 64 * wm + 16 * i + 4 * g + rr;
            if (m < p.rows) {
#pragma unroll
                for (int j = 0; j < 4; ++j) p.partial[(int64_t)m * p.nproj + n0 + 64 * wn + 16 * j + li] = acc[i][j][rr];
            }
        }
}

hipError_t launch_compress(const CompressParams& p, int ratio, int main_dtype, int idx_dtype, hipStream_t stream) {
    if (p.rows <= 0) return hipSuccess;
    const int k_per_split = p.d_in / p.ksplit;
    if (k_per_split % 64 != 0 || p.nproj % 64 != 0) return hipErrorInvalidValue;
    if (p.ksplit == 1 && p.rows >= 1024 && p.d_in % kGemmTile == 0 && p.nproj % kGemmTile == 0) {
        const dim3 grid((unsigned)(p.nproj / kGemmTile), (unsigned)((p.rows + kGemmTile - 1) / kGemmTile));
        hipLaunchKernelGGL(compress_gemm_kernel, grid, dim3(256), 0, stream, p);
    } else {
        const dim3 grid((unsigned)(p.nproj / 64), (unsigned)((p.rows + 63) / 64), (unsigned)p.ksplit);
        hipLaunchKernelGGL(compress_project_kernel, grid, dim3(256), 0, stream, p, k_per_split);
    }
    if (ratio == 1) {
        launch_finish<1>(p, main_dtype, idx_dtype, stream);
    } else {
        launch_finish<2>(p, main_dtype, idx_dtype, stream);
        hipLaunchKernelGGL(compress_tail_kernel, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace csa2

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
//    in a fixed order, so the result does not depend on scheduling.
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

// grid (nproj / 64, ceil(rows / 64), ksplit), 256 threads.
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
        bf16x8 b0 = *reinterpret_cast<const bf16x8*>(wrow + k);
        bf16x8 b1 = *reinterpret_cast<const bf16x8*>(wrow + k + 32);
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

// grid rows, 256 threads: thread t owns latent channels 2t, 2t+1 and (t < 64)
// key elements 2t, 2t+1.
template <int RATIO, int MT, int KT>
__global__ __launch_bounds__(256) void compress_finish_kernel(const CompressParams p) {
    __shared__ float lat[kLatent];
    __shared__ float key[kKey];
    __shared__ float red[4];
    const int t = threadIdx.x;
    const int r = blockIdx.x;
    const int64_t pos = p.pos[r];
    const int s = p.slot[r];
    const int nk = p.ksplit;
    // projections: the split-K partial tiles added in a fixed order (the tail
    // kernel adds them the same way, so a tail holds exactly these values)
    auto proj = [&](int row, int col) {
        float v = 0.f;
        for (int k = 0; k < nk; ++k) v += p.partial[((int64_t)k * p.rows + row) * p.nproj + col];
        return v;
    };
    const int c = 2 * t;
    float v0, v1;
    int64_t j;
    if (RATIO == 1) {
        v0 = proj(r, c);
        v1 = proj(r, c + 1);
        j = pos;
    } else {
        const float kv0 = proj(r, c), kv1 = proj(r, c + 1);
        const float s0 = proj(r, kLatent + c), s1 = proj(r, kLatent + c + 1);
        if ((pos & 1) == 0) return;  // first token of its group (uniform over the workgroup)
        float pk0, pk1, ps0, ps1;
        if (r > 0 && p.slot[r - 1] == s && p.pos[r - 1] == pos - 1) {
            pk0 = proj(r - 1, c);
            pk1 = proj(r - 1, c + 1);
            ps0 = proj(r - 1, kLatent + c);
            ps1 = proj(r - 1, kLatent + c + 1);
        } else {
            const f32x2 tk = *reinterpret_cast<const f32x2*>(p.tail_kv + (int64_t)s * kLatent + c);
            const f32x2 ts = *reinterpret_cast<const f32x2*>(p.tail_score + (int64_t)s * kLatent + c);
            pk0 = tk[0];
            pk1 = tk[1];
            ps0 = ts[0];
            ps1 = ts[1];
        }
        // per channel, softmax over the group's two positions (first: partner)
        const float m0 = fmaxf(ps0, s0), m1 = fmaxf(ps1, s1);
        const float a0 = expf(ps0 - m0), b0 = expf(s0 - m0);
        const float a1 = expf(ps1 - m1), b1 = expf(s1 - m1);
        v0 = (a0 * pk0 + b0 * kv0) / (a0 + b0);
        v1 = (a1 * pk1 + b1 * kv1) / (a1 + b1);
        j = pos / 2;
    }
    // RMSNorm of the latent
    const float ss = block_sum(v0 * v0 + v1 * v1, red);
    const float inv = 1.0f / sqrtf(ss / (float)kLatent + p.eps);
    v0 = v0 * inv * p.norm_w[c];
    v1 = v1 * inv * p.norm_w[c + 1];
    lat[c] = v0;
    lat[c + 1] = v1;
    __syncthreads();
    // index key: output i = t / 2, channels [256 h, 256 h + 256) of half h = t % 2
    {
        const int i = t >> 1, h = t & 1;
        const uint16_t* wr = p.wk + (int64_t)i * kLatent + 256 * h;
        const float* lr = lat + 256 * h;
        float acc = 0.f;
#pragma unroll 4
        for (int q = 0; q < 256; q += 8) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(wr + q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = fmaf(bf16_bits_to_f32(w[e] & 0xffffu), lr[q + 2 * e], acc);
                acc = fmaf(bf16_bits_to_f32(w[e] >> 16), lr[q + 2 * e + 1], acc);
            }
        }
        acc += __shfl_xor(acc, 1, 64);
        if (h == 0) key[i] = acc;
    }
    __syncthreads();
    float k0 = 0.f, k1 = 0.f;
    if (t < kKey / 2) {
        k0 = key[2 * t];
        k1 = key[2 * t + 1];
    }
    const float kss = block_sum(k0 * k0 + k1 * k1, red);
    const float kinv = 1.0f / sqrtf(kss / (float)kKey + p.k_eps);
    if (t < kKey / 2) {
        k0 = k0 * kinv * p.knorm_w[2 * t];
        k1 = k1 * kinv * p.knorm_w[2 * t + 1];
    }
    // rotation of the last 64 dims at the group's first position
    const int64_t rp = j * RATIO;
    if (c >= kLatent - kRope) {
        float cs, sn;
        rope_angle(rp, p.inv_freq[(c - (kLatent - kRope)) / 2], cs, sn);
        const float x0 = v0, x1 = v1;
        v0 = x0 * cs - x1 * sn;
        v1 = x0 * sn + x1 * cs;
    }
    if (t < kKey / 2 && 2 * t >= kKey - kRope) {
        float cs, sn;
        rope_angle(rp, p.inv_freq[(2 * t - (kKey - kRope)) / 2], cs, sn);
        const float x0 = k0, x1 = k1;
        k0 = x0 * cs - x1 * sn;
        k1 = x0 * sn + x1 * cs;
    }
    const int64_t row = p.row_base[r] + j;
    store_pair<MT>(p.main_out, p.main_scale_out, row, kLatent, t, v0, v1);
    if (t < kKey / 2) store_pair<KT>(p.idx_out, p.idx_scale_out, row, kKey, t, k0, k1);
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
    f32x2 kv{0.f, 0.f}, sc{0.f, 0.f};
    for (int k = 0; k < p.ksplit; ++k) {
        const float* pr = p.partial + ((int64_t)k * p.rows + r) * p.nproj;
        kv += *reinterpret_cast<const f32x2*>(pr + c);
        sc += *reinterpret_cast<const f32x2*>(pr + kLatent + c);
    }
    *reinterpret_cast<f32x2*>(p.tail_kv + (int64_t)s * kLatent + c) = kv;
    *reinterpret_cast<f32x2*>(p.tail_score + (int64_t)s * kLatent + c) = sc;
}

bool compress_supported(int main_dtype, int idx_dtype) {
    const bool m = main_dtype == CSA2_F32 || main_dtype == CSA2_BF16 || main_dtype == CSA2_FP4_E2M1 ||
                   main_dtype == CSA2_FP4_E2M1_E4M3G16;
    const bool k = idx_dtype == CSA2_F32 || idx_dtype == CSA2_BF16 || idx_dtype == CSA2_FP8_E4M3 ||
                   idx_dtype == CSA2_FP4_E2M1;
    return m && k;
}

template <int RATIO, int MT>
static void launch_finish_k(const CompressParams& p, int idx_dtype, hipStream_t st) {
    const dim3 grid((unsigned)p.rows);
    switch (idx_dtype) {
        case CSA2_F32: hipLaunchKernelGGL((compress_finish_kernel<RATIO, MT, CSA2_F32>), grid, dim3(256), 0, st, p); break;
        case CSA2_BF16: hipLaunchKernelGGL((compress_finish_kernel<RATIO, MT, CSA2_BF16>), grid, dim3(256), 0, st, p); break;
        case CSA2_FP8_E4M3:
            hipLaunchKernelGGL((compress_finish_kernel<RATIO, MT, CSA2_FP8_E4M3>), grid, dim3(256), 0, st, p);
            break;
        default:
            hipLaunchKernelGGL((compress_finish_kernel<RATIO, MT, CSA2_FP4_E2M1>), grid, dim3(256), 0, st, p);
            break;
    }
}

template <int RATIO>
static void launch_finish_m(const CompressParams& p, int main_dtype, int idx_dtype, hipStream_t st) {
    switch (main_dtype) {
        case CSA2_F32: launch_finish_k<RATIO, CSA2_F32>(p, idx_dtype, st); break;
        case CSA2_BF16: launch_finish_k<RATIO, CSA2_BF16>(p, idx_dtype, st); break;
        case CSA2_FP4_E2M1: launch_finish_k<RATIO, CSA2_FP4_E2M1>(p, idx_dtype, st); break;
        default: launch_finish_k<RATIO, CSA2_FP4_E2M1_E4M3G16>(p, idx_dtype, st); break;
    }
}

hipError_t launch_compress(const CompressParams& p, int ratio, int main_dtype, int idx_dtype, hipStream_t stream) {
    if (p.rows <= 0) return hipSuccess;
    const int k_per_split = p.d_in / p.ksplit;
    if (k_per_split % 64 != 0 || p.nproj % 64 != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(p.nproj / 64), (unsigned)((p.rows + 63) / 64), (unsigned)p.ksplit);
    hipLaunchKernelGGL(compress_project_kernel, grid, dim3(256), 0, stream, p, k_per_split);
    if (ratio == 1) {
        launch_finish_m<1>(p, main_dtype, idx_dtype, stream);
    } else {
        launch_finish_m<2>(p, main_dtype, idx_dtype, stream);
        hipLaunchKernelGGL(compress_tail_kernel, dim3((unsigned)p.rows), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace csa2

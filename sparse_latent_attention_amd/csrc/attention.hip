// Sparse sink attention over SWA + selected compressed rows, for gfx950.
//
//   s_j = scale * <q_h, v_j>,  o_h = sum_j e^{s_j} v_j / (e^{sink_h} + sum_j e^{s_j}),
//   then the rope tail of o_h is rotated back by -pos * inv_freq.
//
// ("DeepSeek-V4-Pro 架构解剖", attention merge fig. 2d formula; "DeepSeek-V4.1-
// Flash 架构解剖", shared attention path, "四种层合并出来的是什么形状" and
// "出来之后"; "DeepSeek-V4.1-Flash 结构说明", sections 4.1 and 6.1.)
//
// Design.  One workgroup handles one query row (and, in decode, one slice of
// its entry list).  The entry list is W SWA entries followed by topk selected
// rows, walked in tiles of 16 entries; W and topk are multiples of 16, so a
// tile comes from one source.  Per tile:
//   1. gather: each thread fetches 8 contiguous elements of 4 rows (one load
//      instruction of a wave covers a whole row), decodes FP4/FP8 in
//      registers, and stores the tile twice into LDS: row-major Kt[j][d] (the
//      QK^T operand) and Vt[j/4][d][j%4] (the PV operand, 4 entries of one
//      column contiguous).  K == V, so both copies come from one HBM read.
//   2. each wave owns 16 heads: S^T[16 entries x 16 heads] = Kt . q^T with
//      16x16x32 MFMAs (q stays in registers), an online-softmax update with
//      the running max/sum per head, then out^T[d][h] += Vt^T . P^T with
//      16x16x16 MFMAs.  The S^T result layout is exactly the P^T operand
//      layout, so P never leaves registers.
// The sink enters as the initial softmax state (max = sink, sum = 1).  Invalid
// entries (absent SWA slots, -1 or out-of-range indices, rows the group-causal
// mask hides) are zero-filled in LDS and get probability 0.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

namespace {

// Eight consecutive elements of one row, in the compute type.
template <class CT>
struct Pack8;
template <>
struct Pack8<__bf16> {
    uint32_t w[4];  // bf16 pairs, element 2q in the low half of w[q]
};
template <>
struct Pack8<float> {
    float v[8];
};

template <class CT>
__device__ __forceinline__ void pack_from_floats(const float* f, Pack8<CT>& o);
template <>
__device__ __forceinline__ void pack_from_floats<__bf16>(const float* f, Pack8<__bf16>& o) {
#pragma unroll
    for (int q = 0; q < 4; ++q) o.w[q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
}
template <>
__device__ __forceinline__ void pack_from_floats<float>(const float* f, Pack8<float>& o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = f[e];
}

template <class CT>
__device__ __forceinline__ void pack_zero(Pack8<CT>& o);
template <>
__device__ __forceinline__ void pack_zero<__bf16>(Pack8<__bf16>& o) {
    o.w[0] = o.w[1] = o.w[2] = o.w[3] = 0u;
}
template <>
__device__ __forceinline__ void pack_zero<float>(Pack8<float>& o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = 0.f;
}

// Loads elements [8*x8, 8*x8+8) of stored row `row` and converts them.
//   F32/BF16: dense rows of D elements.  FP8: D codes per row times fscale[row].
//   FP4: D/2 packed bytes per row times 2^(e8[row*D/32 + blk] - 127).
template <int DT, int D, class CT>
struct RowLoad;

template <int D>
struct RowLoad<CSA2_BF16, D, __bf16> {
    static __device__ __forceinline__ void run(const void* base, const float*, const uint8_t*, int64_t row, int x8,
                                               Pack8<__bf16>& o) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + row * D + 8 * x8);
        o.w[0] = v[0]; o.w[1] = v[1]; o.w[2] = v[2]; o.w[3] = v[3];
    }
};

template <int D>
struct RowLoad<CSA2_F32, D, float> {
    static __device__ __forceinline__ void run(const void* base, const float*, const uint8_t*, int64_t row, int x8,
                                               Pack8<float>& o) {
        const float* p = reinterpret_cast<const float*>(base) + row * D + 8 * x8;
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
        o.v[0] = a[0]; o.v[1] = a[1]; o.v[2] = a[2]; o.v[3] = a[3];
        o.v[4] = b[0]; o.v[5] = b[1]; o.v[6] = b[2]; o.v[7] = b[3];
    }
};

template <int D>
struct RowLoad<CSA2_FP8_E4M3, D, __bf16> {
    static __device__ __forceinline__ void run(const void* base, const float* fscale, const uint8_t*, int64_t row,
                                               int x8, Pack8<__bf16>& o) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(base) + row * D + 8 * x8);
        const float s = fscale[row];
        float f[8];
        f32x2 a = fp8x2_to_f32<false>(v[0]), b = fp8x2_to_f32<true>(v[0]);
        f32x2 c = fp8x2_to_f32<false>(v[1]), d = fp8x2_to_f32<true>(v[1]);
        f[0] = a[0] * s; f[1] = a[1] * s; f[2] = b[0] * s; f[3] = b[1] * s;
        f[4] = c[0] * s; f[5] = c[1] * s; f[6] = d[0] * s; f[7] = d[1] * s;
        pack_from_floats<__bf16>(f, o);
    }
};

template <int D>
struct RowLoad<CSA2_FP4_E2M1, D, __bf16> {
    static __device__ __forceinline__ void run(const void* base, const float*, const uint8_t* e8, int64_t row, int x8,
                                               Pack8<__bf16>& o) {
        const uint32_t v =
            *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(base) + row * (D / 2) + 4 * x8);
        const float s = e8m0_to_f32(e8[row * (D / 32) + (8 * x8) / 32]);
        float f[8];
        f32x2 a = fp4x2_to_f32<0>(v), b = fp4x2_to_f32<1>(v), c = fp4x2_to_f32<2>(v), d = fp4x2_to_f32<3>(v);
        f[0] = a[0] * s; f[1] = a[1] * s; f[2] = b[0] * s; f[3] = b[1] * s;
        f[4] = c[0] * s; f[5] = c[1] * s; f[6] = d[0] * s; f[7] = d[1] * s;
        pack_from_floats<__bf16>(f, o);
    }
};

// LDS tile writers.
template <class CT, int D, int KS>
__device__ __forceinline__ void store_k(CT* Kt, int j, int x8, const Pack8<CT>& v);
template <class CT, int D, int VS>
__device__ __forceinline__ void store_v4(CT* Vt, int jb, int x8, const Pack8<CT> (&v)[4]);

template <>
__device__ __forceinline__ void store_k<__bf16, 512, 520>(__bf16* Kt, int j, int x8, const Pack8<__bf16>& v) {
    *reinterpret_cast<u32x4*>(Kt + j * 520 + 8 * x8) = u32x4{v.w[0], v.w[1], v.w[2], v.w[3]};
}
template <>
__device__ __forceinline__ void store_k<float, 64, 68>(float* Kt, int j, int x8, const Pack8<float>& v) {
    float* p = Kt + j * 68 + 8 * x8;
    *reinterpret_cast<f32x4*>(p) = f32x4{v.v[0], v.v[1], v.v[2], v.v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v.v[4], v.v[5], v.v[6], v.v[7]};
}

// Vt layout: Vt[jb * VS + d * 4 + i] holds entry 4*jb + i, element d.
template <>
__device__ __forceinline__ void store_v4<__bf16, 512, 512 * 4 + 64>(__bf16* Vt, int jb, int x8,
                                                                   const Pack8<__bf16> (&v)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // elements 2q (low halves) and 2q+1 (high halves) of the four rows
        const uint32_t lo01 = (v[0].w[q] & 0xffffu) | (v[1].w[q] << 16);
        const uint32_t lo23 = (v[2].w[q] & 0xffffu) | (v[3].w[q] << 16);
        const uint32_t hi01 = (v[0].w[q] >> 16) | (v[1].w[q] & 0xffff0000u);
        const uint32_t hi23 = (v[2].w[q] >> 16) | (v[3].w[q] & 0xffff0000u);
        const int d = 8 * x8 + 2 * q;
        *reinterpret_cast<u32x2*>(Vt + jb * (512 * 4 + 64) + d * 4) = u32x2{lo01, lo23};
        *reinterpret_cast<u32x2*>(Vt + jb * (512 * 4 + 64) + (d + 1) * 4) = u32x2{hi01, hi23};
    }
}
template <>
__device__ __forceinline__ void store_v4<float, 64, 64 * 4 + 16>(float* Vt, int jb, int x8,
                                                                const Pack8<float> (&v)[4]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = 8 * x8 + e;
        *reinterpret_cast<f32x4*>(Vt + jb * (64 * 4 + 16) + d * 4) = f32x4{v[0].v[e], v[1].v[e], v[2].v[e], v[3].v[e]};
    }
}

// MFMA operand reads from LDS.
template <class CT>
__device__ __forceinline__ typename Mma<CT>::Frag8 lds_frag8(const CT* p);
template <>
__device__ __forceinline__ bf16x8 lds_frag8<__bf16>(const __bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
template <>
__device__ __forceinline__ F32x8 lds_frag8<float>(const float* p) {
    F32x8 f;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
    return f;
}
template <class CT>
__device__ __forceinline__ typename Mma<CT>::Frag4 lds_frag4(const CT* p);
template <>
__device__ __forceinline__ s16x4 lds_frag4<__bf16>(const __bf16* p) {
    return __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(p));
}
template <>
__device__ __forceinline__ F32x4 lds_frag4<float>(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    F32x4 f;
    f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
    return f;
}

// Query fragment (B operand of S^T = K q^T): q[h][32s + 8g .. +8].
template <int QT, class CT, int D>
__device__ __forceinline__ typename Mma<CT>::Frag8 load_q_frag(const void* q, int64_t qrow_elem, int s, int g);
template <>
__device__ __forceinline__ bf16x8 load_q_frag<CSA2_BF16, __bf16, 512>(const void* q, int64_t off, int s, int g) {
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(q) + off + 32 * s + 8 * g));
}
template <>
__device__ __forceinline__ F32x8 load_q_frag<CSA2_F32, float, 64>(const void* q, int64_t off, int s, int g) {
    return lds_frag8<float>(reinterpret_cast<const float*>(q) + off + 32 * s + 8 * g);
}

template <class CT>
__device__ __forceinline__ typename Mma<CT>::Frag8 zero_frag8();
template <>
__device__ __forceinline__ bf16x8 zero_frag8<__bf16>() {
    return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
}
template <>
__device__ __forceinline__ F32x8 zero_frag8<float>() {
    F32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = 0.f;
    return f;
}

// P^T operand (B of out^T = Vt^T P^T) from the 4 probabilities a lane holds.
template <class CT>
__device__ __forceinline__ typename Mma<CT>::Frag4 p_frag(const float (&p)[4]);
template <>
__device__ __forceinline__ s16x4 p_frag<__bf16>(const float (&p)[4]) {
    return __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
}
template <>
__device__ __forceinline__ F32x4 p_frag<float>(const float (&p)[4]) {
    F32x4 f;
    f.v[0] = p[0]; f.v[1] = p[1]; f.v[2] = p[2]; f.v[3] = p[3];
    return f;
}

template <int OT>
__device__ __forceinline__ void store_out4(void* out, int64_t off, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store_out4<CSA2_BF16>(void* out, int64_t off, float a, float b, float c, float d) {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + off) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
template <>
__device__ __forceinline__ void store_out4<CSA2_F32>(void* out, int64_t off, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off) = f32x4{a, b, c, d};
}

// cos/sin of pos * inv_freq[i] in float64, returned as float.
__device__ __forceinline__ void rope_angle(int64_t pos, double f, float& c, float& s) {
    double sd, cd;
    sincos((double)pos * f, &sd, &cd);
    c = (float)cd;
    s = (float)sd;
}

}  // namespace

template <int H, int D, int R, class CT, int QT, int KVT, int SWT, int OT, bool DECODE>
__global__ __launch_bounds__(64 * ((H + 15) / 16)) void sparse_attn_kernel(const AttnParams p) {
    constexpr int NW = (H + 15) / 16;
    constexpr int NT = 64 * NW;
    constexpr int KS = (D == 512) ? 520 : 68;               // Kt row stride (elements)
    constexpr int VS = (D == 512) ? 512 * 4 + 64 : 64 * 4 + 16;  // Vt block stride (elements)
    constexpr int NDT = D / 16;                              // 16-wide output tiles per head
    constexpr int NS = D / 32;                               // k-steps of QK^T
    constexpr int PAIRS = 4 * (D / 8);                       // (row-block, 8-element chunk) pairs per tile
    typedef Mma<CT> M;

    __shared__ __attribute__((aligned(16))) CT Kt[16 * KS];
    __shared__ __attribute__((aligned(16))) CT Vt[4 * VS];
    __shared__ float rope_cs[R];  // [i] cos at 2i, sin at 2i+1
    __shared__ uint32_t vmask;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int r = blockIdx.x;
    const int split = DECODE ? (int)blockIdx.y : 0;

    const int64_t pos = p.pos[r];
    const int64_t nv = (pos + 1) / p.ratio;
    const int W = p.window;
    const int n_tiles = (W + p.topk) / 16;
    const int t_begin = split * p.tiles_per_split;
    const int t_end = (t_begin + p.tiles_per_split < n_tiles) ? t_begin + p.tiles_per_split : n_tiles;

    if (tid < R / 2) {
        float c, s;
        rope_angle(pos, p.inv_freq[tid], c, s);
        rope_cs[2 * tid] = c;
        rope_cs[2 * tid + 1] = s;
    }
    __syncthreads();  // rope_cs complete before any epilogue reads it

    // Query fragments for this wave's 16 heads.
    const int h = 16 * wave + li;
    typename M::Frag8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
        qf[s] = (h < H) ? load_q_frag<QT, CT, D>(p.q, ((int64_t)r * H + h) * D, s, g) : zero_frag8<CT>();

    // Softmax state (log2 units).  Split 0 starts from the sink: max = sink, sum = 1.
    float m = kNegInf, l = 0.f;
    if (split == 0 && h < H) {
        m = p.sink[h] * kLog2e;
        l = (g == 0) ? 1.f : 0.f;
    }
    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t kv_base = p.kv_row_base[r];

    for (int tile = t_begin; tile < t_end; ++tile) {
        const bool swa_tile = tile * 16 < W;
        // ---- gather 16 entries into Kt / Vt -------------------------------------
        if (tid == 0) vmask = 0u;
        __syncthreads();
        for (int pr = tid; pr < PAIRS; pr += NT) {
            const int jb = pr / (D / 8);
            const int x8 = pr - jb * (D / 8);
            Pack8<CT> v[4];
            uint32_t vbits = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = tile * 16 + 4 * jb + i;
                bool valid;
                if (swa_tile) {
                    int64_t srow;
                    if (DECODE) {
                        const int64_t a = pos - ((pos - e) % W + W) % W;
                        valid = a >= 0;
                        srow = (int64_t)r * W + e;
                    } else {
                        const int64_t a = pos - (W - 1) + e;
                        srow = a - p.swa_pos0;
                        valid = a >= 0 && srow >= 0 && srow < p.swa_rows;
                    }
                    if (valid) RowLoad<SWT, D, CT>::run(p.swa, p.swa_scale, nullptr, srow, x8, v[i]);
                    else pack_zero<CT>(v[i]);
                } else {
                    const int32_t id = p.idx[(int64_t)r * p.topk + (e - W)];
                    valid = id >= 0 && (int64_t)id < nv;
                    if (valid) RowLoad<KVT, D, CT>::run(p.kv, nullptr, p.kv_scale, kv_base + id, x8, v[i]);
                    else pack_zero<CT>(v[i]);
                }
                vbits |= (valid ? 1u : 0u) << (4 * jb + i);
                store_k<CT, D, KS>(Kt, 4 * jb + i, x8, v[i]);
            }
            store_v4<CT, D, VS>(Vt, jb, x8, v);
            if (x8 == 0) atomicOr(&vmask, vbits);
        }
        __syncthreads();

        // ---- scores S^T[j = 4g + rr][h] ------------------------------------------
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) st = M::k32(st, lds_frag8<CT>(Kt + li * KS + 32 * s + 8 * g), qf[s]);
        const uint32_t vm = vmask;
        float x[4];
        float tmax = kNegInf;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            x[rr] = ((vm >> (4 * g + rr)) & 1u) ? st[rr] * p.scale_log2 : kNegInf;
            tmax = fmaxf(tmax, x[rr]);
        }
        tmax = fmaxf(tmax, shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2f(m - m_use);
        float pr4[4];
        float psum = 0.f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            pr4[rr] = exp2f(x[rr] - m_use);
            psum += pr4[rr];
        }
        l = l * alpha + psum;
        m = m_new;
        const typename M::Frag4 pb = p_frag<CT>(pr4);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            acc[dt] *= alpha;
            acc[dt] = M::k16(acc[dt], lds_frag4<CT>(Vt + g * VS + (16 * dt + li) * 4), pb);
        }
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------------
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (h >= H) return;
    if (DECODE && p.splits > 1) {
        const int64_t prow = ((int64_t)r * p.splits + split) * H + h;
        float* wa = p.ws_acc + prow * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            *reinterpret_cast<f32x4*>(wa + 16 * dt + 4 * g) = acc[dt];
        if (g == 0) {
            p.ws_ml[2 * prow] = m;
            p.ws_ml[2 * prow + 1] = l;
        }
        return;
    }
    const float inv = 1.f / l;
    const int64_t obase = ((int64_t)r * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int d0 = 16 * dt + 4 * g;
        float o0 = acc[dt][0] * inv, o1 = acc[dt][1] * inv, o2 = acc[dt][2] * inv, o3 = acc[dt][3] * inv;
        if (d0 >= D - R) {
            const int i0 = (d0 - (D - R)) / 2;
            const float c0 = rope_cs[2 * i0], s0 = rope_cs[2 * i0 + 1];
            const float c1 = rope_cs[2 * i0 + 2], s1 = rope_cs[2 * i0 + 3];
            const float a0 = o0 * c0 + o1 * s0, a1 = o1 * c0 - o0 * s0;
            const float a2 = o2 * c1 + o3 * s1, a3 = o3 * c1 - o2 * s1;
            o0 = a0; o1 = a1; o2 = a2; o3 = a3;
        }
        store_out4<OT>(p.out, obase + d0, o0, o1, o2, o3);
    }
}

// Combines the per-split partial states of one (row, head) and applies the
// inverse rotation.  One workgroup of D/4 threads per (row, head).
template <int D, int R, int OT>
__global__ __launch_bounds__(D / 4) void attn_merge_kernel(const AttnParams p, int heads) {
    const int rh = blockIdx.x;  // row * heads + head
    const int r = rh / heads;
    const int t = threadIdx.x;
    const int d0 = 4 * t;
    float mx = kNegInf;
    for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.ws_ml[2 * ((int64_t)(r * p.splits + s) * heads + (rh - r * heads))]);
    const float mu = (mx == kNegInf) ? 0.f : mx;
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.splits; ++s) {
        const int64_t prow = (int64_t)(r * p.splits + s) * heads + (rh - r * heads);
        const float wgt = exp2f(p.ws_ml[2 * prow] - mu);
        L += wgt * p.ws_ml[2 * prow + 1];
        o += wgt * *reinterpret_cast<const f32x4*>(p.ws_acc + prow * D + d0);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float o0 = o[0] * inv, o1 = o[1] * inv, o2 = o[2] * inv, o3 = o[3] * inv;
    if (d0 >= D - R) {
        const int i0 = (d0 - (D - R)) / 2;
        float c0, s0, c1, s1;
        rope_angle(p.pos[r], p.inv_freq[i0], c0, s0);
        rope_angle(p.pos[r], p.inv_freq[i0 + 1], c1, s1);
        const float a0 = o0 * c0 + o1 * s0, a1 = o1 * c0 - o0 * s0;
        const float a2 = o2 * c1 + o3 * s1, a3 = o3 * c1 - o2 * s1;
        o0 = a0; o1 = a1; o2 = a2; o3 = a3;
    }
    store_out4<OT>(p.out, (int64_t)rh * D + d0, o0, o1, o2, o3);
}

// ---------------------------------------------------------------------------
template <int H, int D, int R, class CT, int QT, int KVT, int SWT, int OT>
static hipError_t launch_attn(const AttnParams& p, bool decode, hipStream_t stream) {
    constexpr int NT = 64 * ((H + 15) / 16);
    if (decode) {
        dim3 grid((unsigned)p.rows, (unsigned)p.splits);
        hipLaunchKernelGGL((sparse_attn_kernel<H, D, R, CT, QT, KVT, SWT, OT, true>), grid, dim3(NT), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.splits <= 1) return e;
        hipLaunchKernelGGL((attn_merge_kernel<D, R, OT>), dim3((unsigned)(p.rows * H)), dim3(D / 4), 0, stream, p, H);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((sparse_attn_kernel<H, D, R, CT, QT, KVT, SWT, OT, false>), dim3((unsigned)p.rows), dim3(NT), 0,
                       stream, p);
    return hipGetLastError();
}

bool attn_supported(const AttnShape& s) {
    if (s.heads == 4 && s.dim == 64 && s.rope_dim == 16)
        return s.q_dtype == CSA2_F32 && s.kv_dtype == CSA2_F32 && s.swa_dtype == CSA2_F32 && s.out_dtype == CSA2_F32;
    if (s.heads == 64 && s.dim == 512 && s.rope_dim == 64)
        return s.q_dtype == CSA2_BF16 && s.out_dtype == CSA2_BF16 &&
               (s.kv_dtype == CSA2_BF16 || s.kv_dtype == CSA2_FP4_E2M1) &&
               (s.swa_dtype == CSA2_BF16 || s.swa_dtype == CSA2_FP8_E4M3);
    return false;
}

hipError_t launch_sparse_attn(const AttnParams& p, const AttnShape& s, bool decode, hipStream_t stream) {
    if (s.heads == 4 && s.dim == 64 && s.rope_dim == 16)
        return launch_attn<4, 64, 16, float, CSA2_F32, CSA2_F32, CSA2_F32, CSA2_F32>(p, decode, stream);
    if (s.heads == 64 && s.dim == 512 && s.rope_dim == 64) {
        if (s.kv_dtype == CSA2_BF16 && s.swa_dtype == CSA2_BF16)
            return launch_attn<64, 512, 64, __bf16, CSA2_BF16, CSA2_BF16, CSA2_BF16, CSA2_BF16>(p, decode, stream);
        if (s.kv_dtype == CSA2_FP4_E2M1 && s.swa_dtype == CSA2_FP8_E4M3)
            return launch_attn<64, 512, 64, __bf16, CSA2_BF16, CSA2_FP4_E2M1, CSA2_FP8_E4M3, CSA2_BF16>(p, decode, stream);
        if (s.kv_dtype == CSA2_FP4_E2M1 && s.swa_dtype == CSA2_BF16)
            return launch_attn<64, 512, 64, __bf16, CSA2_BF16, CSA2_FP4_E2M1, CSA2_BF16, CSA2_BF16>(p, decode, stream);
        if (s.kv_dtype == CSA2_BF16 && s.swa_dtype == CSA2_FP8_E4M3)
            return launch_attn<64, 512, 64, __bf16, CSA2_BF16, CSA2_BF16, CSA2_FP8_E4M3, CSA2_BF16>(p, decode, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace csa2

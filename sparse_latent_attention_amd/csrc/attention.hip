// Sparse sink attention over SWA + selected compressed rows, for gfx950.
//
//   s_j = scale * <q_h, v_j>,  o_h = sum_j e^{s_j} v_j / (e^{sink_h} + sum_j e^{s_j}),
//   then the rope tail of o_h is rotated back by -pos * inv_freq.
//
// ("DeepSeek-V4-Pro 架构解剖", attention merge fig. 2d formula; "DeepSeek-V4.1-
// Flash 架构解剖", shared attention path, "四种层合并出来的是什么形状" and
// "出来之后"; "DeepSeek-V4.1-Flash 结构说明", sections 4.1 and 6.1.)
//
// Shared design.  A query row's entry list is W SWA entries followed by topk
// selected rows, walked in tiles of 16 entries (W and topk are multiples of 16,
// so a tile comes from one source).  A tile is gathered once from HBM (an
// absent row is read from a zero row, so no load needs a branch), FP4/FP8 rows
// are decoded in registers, and the tile is stored once into LDS, row-major
// with XOR-swizzled 16-byte chunks.  QK^T reads it as the MFMA operand; PV
// reads it through the gfx950 transposing LDS read, so no transposed copy is
// written (K == V).  The score result layout of the QK MFMA is the probability
// operand of the PV MFMA, so probabilities never leave registers.  The sink is
// the initial softmax state (max = sink, sum = 1); invalid entries (absent SWA
// slots, -1 or out-of-range indices, rows the group-causal mask hides) get
// probability 0.
//
// attn_rows_kernel (16x16 MFMAs; 16-head groups of two waves) serves decode
// rows, whose entries are also split over S workgroups (each leaves its softmax
// state; attn_merge_kernel combines them), and prefill rows outside the next
// kernel's shape.  attn_prefill_kernel (32x32x16 MFMAs; four waves of 32 heads
// per row, one per SIMD) serves prefill rows over BF16 planes: one workgroup per
// CU streams a contiguous run of rows.
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

// LDS tile writers.
template <class CT, int D, int KS>
__device__ __forceinline__ void store_k(CT* Kt, int j, int x8, const Pack8<CT>& v);
template <class CT, int D, int VS>
__device__ __forceinline__ void store_v4(CT* Vt, int jb, int x8, const Pack8<CT> (&v)[4]);

// Tile layouts in LDS (element offsets).  D = 512 (BF16): Kt rows of 512
// elements whose 8-element (16-byte) chunks are XOR-ed with the row's low 4
// bits, and the PV copy's column d at 4 (d ^ ((d >> 3) & 7)): both measured
// free of bank conflicts for the MFMA operand reads with rocprofv3
// (SQ_LDS_BANK_CONFLICT), where rows padded by 16 bytes (2.7 conflict cycles
// per LDS cycle) and columns with a gap after every 8 (1.3) were not.
// D = 64 (F32): rows padded to 68 elements, column d at 4d + 4(d/8).
template <int D>
__device__ __forceinline__ int kpos(int j, int c8) {
    return D == 512 ? j * 512 + 8 * (c8 ^ (j & 15)) : j * 68 + 8 * c8;
}
template <int D>
__device__ __forceinline__ int vcol(int d) {
    return D == 512 ? 4 * (d ^ ((d >> 3) & 7)) : 4 * d + 4 * (d >> 3);
}

template <>
__device__ __forceinline__ void store_k<__bf16, 512, 512>(__bf16* Kt, int j, int x8, const Pack8<__bf16>& v) {
    *reinterpret_cast<u32x4*>(Kt + kpos<512>(j, x8)) = u32x4{v.w[0], v.w[1], v.w[2], v.w[3]};
}
template <>
__device__ __forceinline__ void store_k<float, 64, 68>(float* Kt, int j, int x8, const Pack8<float>& v) {
    float* p = Kt + kpos<64>(j, x8);
    *reinterpret_cast<f32x4*>(p) = f32x4{v.v[0], v.v[1], v.v[2], v.v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v.v[4], v.v[5], v.v[6], v.v[7]};
}

// Vt layout: Vt[jb * VS + vcol<D>(d) + i] holds entry 4*jb + i, element d.
template <>
__device__ __forceinline__ void store_v4<__bf16, 512, 2368>(__bf16* Vt, int jb, int x8,
                                                                   const Pack8<__bf16> (&v)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // elements 2q (low halves) and 2q+1 (high halves) of the four rows
        const uint32_t lo01 = (v[0].w[q] & 0xffffu) | (v[1].w[q] << 16);
        const uint32_t lo23 = (v[2].w[q] & 0xffffu) | (v[3].w[q] << 16);
        const uint32_t hi01 = (v[0].w[q] >> 16) | (v[1].w[q] & 0xffff0000u);
        const uint32_t hi23 = (v[2].w[q] >> 16) | (v[3].w[q] & 0xffff0000u);
        const int d = 8 * x8 + 2 * q;
        *reinterpret_cast<u32x2*>(Vt + jb * 2368 + vcol<512>(d)) = u32x2{lo01, lo23};
        *reinterpret_cast<u32x2*>(Vt + jb * 2368 + vcol<512>(d + 1)) = u32x2{hi01, hi23};
    }
}
template <>
__device__ __forceinline__ void store_v4<float, 64, 304>(float* Vt, int jb, int x8,
                                                                const Pack8<float> (&v)[4]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = 8 * x8 + e;
        *reinterpret_cast<f32x4*>(Vt + jb * 304 + vcol<64>(d)) = f32x4{v[0].v[e], v[1].v[e], v[2].v[e], v[3].v[e]};
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



// Raw bytes of one pair (4 rows x 8 elements) of a tile, as loaded from HBM.
struct RawPair {
    u32x4 v[4];    // BF16: 16 B per row; F32: elements 0..3; FP8: .x .y; FP4: .x
    u32x4 v2[4];   // F32: elements 4..7
    float s[4];    // FP8 row scale
    uint32_t sb[4];  // FP4: E8M0 block-scale byte (decoded at conversion, so no load waits on it)
    uint32_t valid;  // bit i: row i of the pair exists and is visible
};

// Byte offsets within a stored row of D elements: the 8 elements of chunk x8, and (formats with
// inline scales) the scale byte that covers them.
template <int DT, int D>
__device__ __forceinline__ int chunk_off(int x8) {
    return DT == CSA2_F32 ? 32 * x8 : DT == CSA2_BF16 ? 16 * x8
         : (DT == CSA2_FP8_E4M3 || DT == CSA2_FP8_E4M3_E8M0G32) ? 8 * x8 : 4 * x8;
}
template <int DT, int D>
__device__ __forceinline__ int inline_scale_off(int x8) {
    return DT == CSA2_FP4_E2M1_E4M3G16 ? D / 2 + (8 * x8) / 16 : DT == CSA2_FP8_E4M3_E8M0G32 ? D + (8 * x8) / 32 : 0;
}

// Loads the 8 elements of one row's chunk: `dp` points at them (chunk_off already added; an
// invalid row points into the zero row, so the loads need no branch and decode to zeros), `fsc` at
// the row's FP8 scale, `e8` at its E8M0 byte (planar FP4 scales); inline scale bytes sit at
// dp + sdelta.
template <int DT, int D>
__device__ __forceinline__ void raw_load_row(const uint8_t* dp, const float* fsc, const uint8_t* e8, int sdelta,
                                             RawPair& raw, int i) {
    if (DT == CSA2_BF16) {
        raw.v[i] = *reinterpret_cast<const u32x4*>(dp);
    } else if (DT == CSA2_F32) {
        raw.v[i] = *reinterpret_cast<const u32x4*>(dp);
        raw.v2[i] = *reinterpret_cast<const u32x4*>(dp + 16);
    } else if (DT == CSA2_FP8_E4M3) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(dp);
        raw.v[i].x = w.x;
        raw.v[i].y = w.y;
        raw.s[i] = *fsc;
    } else if (DT == CSA2_FP4_E2M1) {  // FP4-E2M1 with one E8M0 per 32 (planar scales)
        raw.v[i].x = *reinterpret_cast<const uint32_t*>(dp);
        raw.sb[i] = *e8;
    } else if (DT == CSA2_FP4_E2M1_E4M3G16) {  // FP4-E2M1, then one E4M3 scale per 16, inline
        raw.v[i].x = *reinterpret_cast<const uint32_t*>(dp);
        raw.sb[i] = dp[sdelta];
    } else {  // CSA2_FP8_E4M3_E8M0G32: FP8-E4M3, then one E8M0 scale per 32, inline
        const u32x2 w = *reinterpret_cast<const u32x2*>(dp);
        raw.v[i].x = w.x;
        raw.v[i].y = w.y;
        raw.sb[i] = dp[sdelta];
    }
}

template <int DT>
constexpr int row_bytes(int d) {
    return DT == CSA2_F32 ? 4 * d : DT == CSA2_BF16 ? 2 * d : DT == CSA2_FP8_E4M3 ? d
         : DT == CSA2_FP4_E2M1_E4M3G16 ? d / 2 + d / 16 : DT == CSA2_FP8_E4M3_E8M0G32 ? d + d / 32 : d / 2;
}

// (Rows that are not there were loaded from the zero row: zero values and zero scale bytes, which
// decode to zeros, so no validity select is needed here.)
template <int DT, class CT>
__device__ __forceinline__ void raw_convert(const RawPair& raw, int i, Pack8<CT>& o) {
    if constexpr (DT == CSA2_BF16) {
        o.w[0] = raw.v[i].x;
        o.w[1] = raw.v[i].y;
        o.w[2] = raw.v[i].z;
        o.w[3] = raw.v[i].w;
    } else if constexpr (DT == CSA2_F32) {
        const uint32_t u[8] = {raw.v[i].x, raw.v[i].y, raw.v[i].z, raw.v[i].w,
                               raw.v2[i].x, raw.v2[i].y, raw.v2[i].z, raw.v2[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = __uint_as_float(u[e]);
    } else if constexpr (DT == CSA2_FP4_E2M1 && sizeof(CT) == 2) {
        // E2M1 pairs straight to bf16 pairs, multiplied by the power-of-two block scale (exact).
        // E8M0 byte 255 is NaN: every element of its block decodes to NaN (0 x NaN included),
        // set explicitly rather than left to the convert's handling of a NaN scale.
        const uint32_t w = raw.v[i].x;
        const float sc = e8m0_to_f32(raw.sb[i]);
        const bool nan_blk = raw.sb[i] == 255u;
        constexpr uint32_t kNanPair = 0x7fc07fc0u;
        const uint32_t b0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
        const uint32_t b1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
        const uint32_t b2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
        const uint32_t b3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
        o.w[0] = nan_blk ? kNanPair : b0;
        o.w[1] = nan_blk ? kNanPair : b1;
        o.w[2] = nan_blk ? kNanPair : b2;
        o.w[3] = nan_blk ? kNanPair : b3;
    } else {
        // Exact in every case: an FP8 or FP4 value times a power of two, or an E2M1 value
        // (<= 2 significant bits) times an E4M3 scale (<= 4), fits bf16's 8 bits.
        float f[8];
        float sc;
        if constexpr (DT == CSA2_FP4_E2M1 || DT == CSA2_FP8_E4M3_E8M0G32) sc = e8m0_to_f32(raw.sb[i]);
        else if constexpr (DT == CSA2_FP4_E2M1_E4M3G16) sc = fp8x2_to_f32<false>(raw.sb[i])[0];
        else sc = raw.s[i];
        if constexpr (DT == CSA2_FP8_E4M3 || DT == CSA2_FP8_E4M3_E8M0G32) {
            const f32x2 a = fp8x2_to_f32<false>(raw.v[i].x), b = fp8x2_to_f32<true>(raw.v[i].x);
            const f32x2 c = fp8x2_to_f32<false>(raw.v[i].y), d = fp8x2_to_f32<true>(raw.v[i].y);
            f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1]; f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
        } else {
            const uint32_t w = raw.v[i].x;
            const f32x2 a = fp4x2_to_f32<0>(w), b = fp4x2_to_f32<1>(w), c = fp4x2_to_f32<2>(w), d = fp4x2_to_f32<3>(w);
            f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1]; f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f[e] * sc;
        pack_from_floats<CT>(f, o);
    }
}

constexpr int kMaxTiles = 192;  // (window + topk) / 16 at most (window <= 1024, topk <= 2048)
constexpr int kMaxSplits = 8;   // decode workgroups per (row, head group) at most
// Rounds of tile loads in flight in attn_rows_kernel: two for prefill (measured 7 % faster than one
// on the 4096-row chunk), one for decode (two were 1 us slower: a decode workgroup has few rounds).
// Workgroups per row (head slices) of the 64-head shape: two (32 heads each, two workgroups per CU)
// for decode over BF16 rows, measured 2.8 us faster than one at 32 rows x 1M; one otherwise -- for
// prefill and for FP4 / FP8 rows the second slice's repeated gather and decode cost more than the
// overlap of two independent workgroups gains (prefill 3.92 -> 4.28 ms, FP4 decode 39 -> 43 us).
#ifndef CSA2_ATTN_BF16_DECODE_SLICES
#define CSA2_ATTN_BF16_DECODE_SLICES 2
#endif
#ifndef CSA2_ATTN_PREFILL_PF
#define CSA2_ATTN_PREFILL_PF 2
#endif
// Prefill rows of the 64-head shape on attn_prefill_kernel (32x32x16 MFMAs, 32 heads per wave).
#ifndef CSA2_ATTN_PREFILL_WIDE
#define CSA2_ATTN_PREFILL_WIDE 1
#endif
#ifndef CSA2_ATTN_WIDE_PF
#define CSA2_ATTN_WIDE_PF 1
#endif
#ifndef CSA2_ATTN_DECODE_PF
#define CSA2_ATTN_DECODE_PF 1
#endif

// Rows that are not there (absent SWA slots, -1 or out-of-range indices, rows the group-causal mask
// hides) are read from here instead: zeros, which decode to zeros in every stored format.  Never
// written; 1 KiB covers the largest stored row (512 BF16 elements).
__device__ __attribute__((aligned(64))) uint8_t g_zero_row[1024];

// Per-row geometry the gather needs.
struct RowCtx {
    int64_t pos, nv;
    int r;
    const uint8_t* swa0;   // window slot e's stored row at swa0 + e * (SWA row bytes)
    const float* swas0;    // FP8 SWA rows: slot e's scale at swas0[e]
    const uint8_t* kv0;    // selected row id at kv0 + id * (main row bytes)
    const uint8_t* kvs0;   // planar E8M0 scales: row id's at kvs0 + id * (D / 32)
    int win_lo, win_hi;    // window slots e with win_lo <= e < win_hi are there
    uint32_t nv32;         // ids below this are visible (-1 is not: it wraps to the top)
};

template <int D, int KVT, int SWT, bool DECODE>
__device__ __forceinline__ void row_ctx_init(const AttnParams& p, RowCtx& c, int r) {
    c.r = r;
    c.pos = p.pos[r];
    c.nv = (c.pos + 1) / p.ratio;
    c.nv32 = (uint32_t)(c.nv < 0x7fffffff ? (c.nv > 0 ? c.nv : 0) : 0x7fffffff);
    const int64_t kv_base = p.kv_row_base[r];
    c.kv0 = reinterpret_cast<const uint8_t*>(p.kv) + kv_base * row_bytes<KVT>(D);
    c.kvs0 = KVT == CSA2_FP4_E2M1 ? p.kv_scale + kv_base * (D / 32) : nullptr;
    const int W = p.window;
    int64_t s0, lo, hi;  // stored SWA row of slot 0, and the slots that are there
    if (DECODE) {
        // Ring slot e holds position pos - ((pos - e) mod W); that position is negative (the slot
        // was never written) exactly when e > pos.
        s0 = (int64_t)r * W;
        lo = 0;
        hi = c.pos + 1;
    } else {
        // slot e is linear window position a = pos - (W - 1) + e, stored row a - swa_pos0
        s0 = c.pos - (W - 1) - p.swa_pos0;
        lo = (W - 1) - c.pos;                         // a >= 0
        if (lo < -s0) lo = -s0;                       // stored row >= 0
        hi = p.swa_rows - s0;                         // stored row < swa_rows
    }
    if (lo < 0) lo = 0;
    if (hi > W) hi = W;
    if (hi < lo) hi = lo;
    c.win_lo = (int)lo;
    c.win_hi = (int)hi;
    c.swa0 = reinterpret_cast<const uint8_t*>(p.swa) + s0 * row_bytes<SWT>(D);
    c.swas0 = SWT == CSA2_FP8_E4M3 ? p.swa_scale + s0 : nullptr;
}

// Loads the raw bytes of pair (jb, x8) of tile `tile`: chunk x8 of 4 consecutive entries.
// `sel` is the row's selected-index list, staged in LDS.  Each row address is one 32 x 32 -> 64
// multiply-add on a per-row base and a select against the zero row.
template <int D, int KVT, int SWT, bool DECODE>
__device__ __forceinline__ void load_pair(const AttnParams& p, const RowCtx& c, const int32_t* sel, int tile, int jb,
                                          int x8, RawPair& raw) {
    const int W = p.window;
    raw.valid = 0u;
    if (tile * 16 < W) {
        constexpr int RB = row_bytes<SWT>(D);
        const int xo = chunk_off<SWT, D>(x8);
        const int sd = inline_scale_off<SWT, D>(x8) - xo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tile * 16 + 4 * jb + i;
            const bool valid = (uint32_t)(e - c.win_lo) < (uint32_t)(c.win_hi - c.win_lo);
            const uint8_t* dp = valid ? c.swa0 + ((uint64_t)(uint32_t)e * RB + xo) : g_zero_row + xo;
            const float* fs = SWT == CSA2_FP8_E4M3 ? (valid ? c.swas0 + e : reinterpret_cast<const float*>(g_zero_row))
                                                   : nullptr;
            raw_load_row<SWT, D>(dp, fs, nullptr, sd, raw, i);
            raw.valid |= (valid ? 1u : 0u) << i;
        }
    } else {
        constexpr int RB = row_bytes<KVT>(D);
        const int xo = chunk_off<KVT, D>(x8);
        const int sd = inline_scale_off<KVT, D>(x8) - xo;
        // the pair's 4 selected indices with one 16-byte LDS read (W and 16 * tile are multiples of 16)
        const i32x4 ids = *reinterpret_cast<const i32x4*>(sel + tile * 16 + 4 * jb - W);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t id = (uint32_t)ids[i];
            const bool valid = id < c.nv32;  // group-causal mask; -1 wraps to the top
            const uint8_t* dp = valid ? c.kv0 + ((uint64_t)id * RB + xo) : g_zero_row + xo;
            const uint8_t* e8 = KVT == CSA2_FP4_E2M1
                                    ? (valid ? c.kvs0 + ((uint64_t)id * (D / 32) + (8 * x8) / 32) : g_zero_row)
                                    : nullptr;
            raw_load_row<KVT, D>(dp, nullptr, e8, sd, raw, i);
            raw.valid |= (valid ? 1u : 0u) << i;
        }
    }
}

// Decodes a loaded pair and writes it into the tile buffers.
template <int D, class CT, int KS, int VS, int KVT, int SWT>
__device__ __forceinline__ void store_pair(const RawPair& raw, bool swa_tile, CT* Kt, CT* Vt, int jb, int x8) {
    Pack8<CT> v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (swa_tile) raw_convert<SWT, CT>(raw, i, v[i]);
        else raw_convert<KVT, CT>(raw, i, v[i]);
        store_k<CT, D, KS>(Kt, 4 * jb + i, x8, v[i]);
    }
    store_v4<CT, D, VS>(Vt, jb, x8, v);
}

// Tile pairs (BF16, D = 512): only the row-major K tiles live in LDS.  The PV
// operand (8 entries of one column: 4 of each tile of the pair) is read from
// them with the gfx950 transposing LDS read (ds_read_b64_tr_b16, see
// lds_col4), so no transposed copy is written.
template <int KVT, int SWT>
__device__ __forceinline__ void store_pair_k(const RawPair& raw, bool swa_tile, __bf16* Kt, int jb, int x8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        Pack8<__bf16> v;
        if (swa_tile) raw_convert<SWT, __bf16>(raw, i, v);
        else raw_convert<KVT, __bf16>(raw, i, v);
        store_k<__bf16, 512, 512>(Kt, 4 * jb + i, x8, v);
    }
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j names 4 consecutive bf16 at its address; lane i then receives
// element i % 4 of lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 (checked on
// the device with a lane-layout probe).  So if lane j of group g points at
// entry 4 g + j / 4, columns c0 + 4 (j % 4) .. + 3, lane i of that group gets
// column c0 + i of entries 4 g .. 4 g + 3: the A-operand slots 8 g .. 8 g + 3
// of a 16x16x32 MFMA whose rows are the 16 columns c0 ...
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_col4(const __bf16* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<__bf16*>(p)));
    return __builtin_bit_cast(u32x2, r);
}

template <class CT, int D>
struct TileGeom {
    static constexpr int KS = (D == 512) ? 512 : 68;                // Kt row stride (elements)
    static constexpr int VS = (D == 512) ? 2368 : 304;  // Vt block stride (elements): 4D + D/2 + padding
    static constexpr int K_ELEMS = 16 * KS;
    static constexpr int V_ELEMS = 4 * VS;
    static constexpr int BYTES = (K_ELEMS + V_ELEMS) * (int)sizeof(CT);
};

// Scores S^T of one tile for the wave's 16 heads over NSQ of the D / 32 k-steps,
// starting koff elements into each row (all of them by default).
template <int D, class CT, int KS, int NSQ = D / 32>
__device__ __forceinline__ f32x4 tile_scores(const CT* Kt, const typename Mma<CT>::Frag8* qf, int g, int li,
                                             int koff = 0) {
    typedef Mma<CT> M;
    constexpr int NS = NSQ;
    // Four independent accumulation chains keep the matrix cores busy.
    constexpr int NC = NS >= 4 ? 4 : NS;
    f32x4 part[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) part[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Operand addresses.  With the D = 512 layout the lane-dependent part of
    // kpos(li, 4s + g) takes 4 values (by s mod 4); the rest is a compile-time offset.
    int ko[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        ko[b] = (D == 512) ? li * 512 + 32 * (b ^ (li >> 2)) + 8 * (g ^ (li & 3)) + koff : kpos<D>(li, 4 * b + g);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int k_off = (D == 512) ? ko[s & 3] + 128 * (s >> 2) : kpos<D>(li, 4 * s + g);
        part[s % NC] = M::k32(part[s % NC], lds_frag8<CT>(Kt + k_off), qf[s]);
    }
    if constexpr (sizeof(CT) == 2) {
        // keep 4 operand reads in flight ahead of the matrix instructions
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < NS - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    f32x4 st = part[0];
#pragma unroll
    for (int k = 1; k < NC; ++k) st += part[k];
    return st;
}

// The online-softmax update and PV of one tile, given its full scores st.
template <int D, class CT, int VS, int NACC = D / 16>
__device__ __forceinline__ void tile_update(f32x4 st, const CT* Vt, uint32_t vm, float scale_log2, int g, int li,
                                            float& m, float& l, f32x4* acc, int dt0 = 0) {
    typedef Mma<CT> M;
    int vo[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        vo[b] = (D == 512) ? g * VS + 64 * dt0 + 4 * (16 * b + (li & 8) + ((li & 7) ^ ((2 * b + (li >> 3)) & 7)))
                           : g * VS + vcol<D>(16 * (dt0 + b) + li);
    float x[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) x[rr] = st[rr] * scale_log2;
    if (vm != 0xffffu) {  // the same for the whole wave: most tiles have 16 valid entries
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) x[rr] = ((vm >> (4 * g + rr)) & 1u) ? x[rr] : kNegInf;
    }
    const float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    float tmax_all = tmax;
    tmax_all = fmaxf(tmax_all, shfl_xor(tmax_all, 16));
    tmax_all = fmaxf(tmax_all, shfl_xor(tmax_all, 32));
    // Lazy rescaling: m is only a reference point (the result is the same for any
    // m), so it moves -- and acc and l are rescaled -- only when some head's scores
    // exceed it by more than 2^8; the probabilities then stay below 256.
    const uint64_t need_rescale = __ballot(tmax_all > m + 8.f);
    if (__builtin_expect(__builtin_amdgcn_readfirstlane((uint32_t)(need_rescale | (need_rescale >> 32))) != 0u, 0)) {
        const float m_new = fmaxf(m, tmax_all);
        const float alpha = exp2f(m - m_new);  // 0 when m was -inf
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NACC; ++dt) acc[dt] *= alpha;
        m = m_new;
        __builtin_amdgcn_sched_barrier(0);
    }
    const float m_use = (m == kNegInf) ? 0.f : m;
    float pr4[4];
    float psum = 0.f;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        // x - m_use <= 8 (lazy rescaling) and -inf for masked entries: the hardware exp2 (v_exp_f32,
        // -inf -> 0) needs none of exp2f's range handling
        pr4[rr] = __builtin_amdgcn_exp2f(x[rr] - m_use);
        psum += pr4[rr];
    }
    l += psum;
    const typename M::Frag4 pb = p_frag<CT>(pr4);
#pragma unroll
    for (int dt = 0; dt < NACC; ++dt) {
        const int v_off = (D == 512) ? vo[dt & 3] + 256 * (dt >> 2) : g * VS + vcol<D>(16 * (dt0 + dt) + li);
        acc[dt] = M::k16(acc[dt], lds_frag4<CT>(Vt + v_off), pb);
    }
}

// One wave's work on one tile for its 16 heads: scores, online softmax, PV.
// The wave accumulates output columns 16 dt0 .. 16 (dt0 + NACC) - 1 (all of D
// by default); the scores and the softmax state always cover the whole row.
template <int D, class CT, int KS, int VS, int NACC = D / 16>
__device__ __forceinline__ void tile_compute(const CT* Kt, const CT* Vt, uint32_t vm, const typename Mma<CT>::Frag8* qf,
                                             float scale_log2, int g, int li, float& m, float& l, f32x4* acc,
                                             int dt0 = 0) {
    tile_update<D, CT, VS, NACC>(tile_scores<D, CT, KS>(Kt, qf, g, li), Vt, vm, scale_log2, g, li, m, l, acc, dt0);
}

// Two tiles at once (BF16, D = 512): the scores of both, one softmax update
// over their 32 entries, and PV as 16x16x32 MFMAs.  Slot 8g + i of such an
// MFMA's 32-long reduction is entry 4g + i of tile 0 for i < 4 and entry
// 4g + i - 4 of tile 1 otherwise, in both operands: a lane's P^T fragment is
// then its 4 probabilities of each tile side by side, and its V^T fragment the
// same 4 entries' column from each tile's PV copy.  On gfx950 a 16x16x32 MFMA
// takes about as long as a 16x16x16 one (measured: 1.44 against 0.81 PFLOP/s
// sustained), so this halves the PV matrix time.  Two score chains per tile.
template <int NACC>
__device__ __forceinline__ void tile_pair_compute(const __bf16* Kt0, const __bf16* Kt1,
                                                  uint32_t vm0, uint32_t vm1, const bf16x8* qf, int half,
                                                  f32x4* xch_mine, const f32x4* xch_partner, float scale_log2,
                                                  int g, int li, int lane, float& m, float& l, f32x4* acc, int dt0) {
    constexpr int NS = 512 / 32, NH = NS / 2;
    // K operand offsets: the lane-dependent part takes 4 values (by s mod 4); the rest is constant.
    // This wave's half of the reduction is k-steps NH * half .. NH * half + NH - 1 (256 elements on).
    int ko[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) ko[b] = li * 512 + 32 * (b ^ (li >> 2)) + 8 * (g ^ (li & 3)) + 256 * half;
    // PV operand (lds_col4): lane (g, li) names entry e = 4 g + li / 4, columns c0 + 4 (li % 4) .. + 3
    // with c0 = 16 (dt0 + dt), i.e. half (li % 2) of 16-byte chunk c0 / 8 + (li % 4) / 2, stored at
    // chunk index ^ (e & 15).  dt0 is a multiple of 16, so the chunk is 2 dt0 + 16 (dt / 8) +
    // ((2 (dt % 8) + (li % 4) / 2) ^ (e & 15)): the lane's part takes 8 values (by dt mod 8).
    const int e = 4 * g + (li >> 2);
    const int vrow = e * 512 + 4 * (li & 1) + 16 * dt0;
    const int vx = ((li >> 1) & 1) ^ (e & 15);
    f32x4 part[4];  // chains 0, 1: tile 0; chains 2, 3: tile 1
#pragma unroll
    for (int k = 0; k < 4; ++k) part[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NH; ++s) {
        const int k_off = ko[s & 3] + 128 * (s >> 2);
        part[s & 1] = Mma<__bf16>::k32(part[s & 1], lds_frag8<__bf16>(Kt0 + k_off), qf[s]);
        part[2 + (s & 1)] = Mma<__bf16>::k32(part[2 + (s & 1)], lds_frag8<__bf16>(Kt1 + k_off), qf[s]);
    }
    // Keep QK_AHEAD operand reads in flight ahead of the matrix instructions.
    constexpr int QK_AHEAD = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, QK_AHEAD, 0);
#pragma unroll
    for (int i = 0; i < 2 * NH - QK_AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, QK_AHEAD, 0);
    // The two waves of a head group exchange their halves through LDS; a + b == b + a exactly,
    // so both form bit-identical scores and softmax states.
    f32x4 st0 = part[0] + part[1], st1 = part[2] + part[3];
    xch_mine[lane] = st0;
    xch_mine[64 + lane] = st1;
    __syncthreads();
    st0 = st0 + xch_partner[lane];
    st1 = st1 + xch_partner[64 + lane];
    float x[8];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        x[rr] = st0[rr] * scale_log2;
        x[4 + rr] = st1[rr] * scale_log2;
    }
    if ((vm0 & vm1) != 0xffffu) {  // the same for the whole wave
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            x[rr] = ((vm0 >> (4 * g + rr)) & 1u) ? x[rr] : kNegInf;
            x[4 + rr] = ((vm1 >> (4 * g + rr)) & 1u) ? x[4 + rr] : kNegInf;
        }
    }
    float tmax_all = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    tmax_all = fmaxf(tmax_all, shfl_xor(tmax_all, 16));
    tmax_all = fmaxf(tmax_all, shfl_xor(tmax_all, 32));
    // lazy rescaling, as in tile_compute
    const uint64_t need_rescale = __ballot(tmax_all > m + 8.f);
    if (__builtin_expect(__builtin_amdgcn_readfirstlane((uint32_t)(need_rescale | (need_rescale >> 32))) != 0u, 0)) {
        const float m_new = fmaxf(m, tmax_all);
        const float alpha = exp2f(m - m_new);  // 0 when m was -inf
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NACC; ++dt) acc[dt] *= alpha;
        m = m_new;
        __builtin_amdgcn_sched_barrier(0);
    }
    const float m_use = (m == kNegInf) ? 0.f : m;
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        pr[e] = __builtin_amdgcn_exp2f(x[e] - m_use);  // x - m_use <= 8; -inf -> 0
        psum += pr[e];
    }
    l += psum;
    const bf16x8 pb = __builtin_bit_cast(
        bf16x8, u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]), pack_bf16x2(pr[4], pr[5]),
                      pack_bf16x2(pr[6], pr[7])});
#pragma unroll
    for (int dt = 0; dt < NACC; ++dt) {
        const int v_off = vrow + 8 * (16 * (dt >> 3) + ((2 * (dt & 7)) ^ vx));
        const u32x2 a0 = lds_col4(Kt0 + v_off), a1 = lds_col4(Kt1 + v_off);
        acc[dt] = Mma<__bf16>::k32(acc[dt], __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y}), pb);
    }
}

// Normalises 4 consecutive elements (columns d0 .. d0 + 3) and rotates the rope tail back.
template <int D, int R>
__device__ __forceinline__ f32x4 finish4(int d0, f32x4 a, float inv, const float* rope_cs) {
    float o0 = a[0] * inv, o1 = a[1] * inv, o2 = a[2] * inv, o3 = a[3] * inv;
    if (d0 >= D - R) {
        const int i0 = (d0 - (D - R)) / 2;
        const float c0 = rope_cs[2 * i0], s0 = rope_cs[2 * i0 + 1];
        const float c1 = rope_cs[2 * i0 + 2], s1 = rope_cs[2 * i0 + 3];
        const float b0 = o0 * c0 + o1 * s0, b1 = o1 * c0 - o0 * s0;
        const float b2 = o2 * c1 + o3 * s1, b3 = o3 * c1 - o2 * s1;
        o0 = b0; o1 = b1; o2 = b2; o3 = b3;
    }
    return f32x4{o0, o1, o2, o3};
}

// ... and stores them.
template <int D, int R, int OT>
__device__ __forceinline__ void emit4(void* out, int64_t off, int d0, f32x4 a, float inv, const float* rope_cs) {
    const f32x4 o = finish4<D, R>(d0, a, inv, rope_cs);
    store_out4<OT>(out, off, o[0], o[1], o[2], o[3]);
}

}  // namespace

// ---------------------------------------------------------------------------
// One workgroup per query row, all waves on the same tiles.  Each 16-head
// group has DS waves: each computes the group's scores and softmax state over
// the whole row (identical in all DS waves) and accumulates 1/DS of the output
// columns.  DS = 2 halves the accumulator registers, so two waves fit on each
// SIMD and one wave's LDS reads and waits overlap the other's matrix work.
template <int H, int D, int R, class CT, int QT, int KVT, int SWT, int OT, bool DECODE, int DS, int HS>
__global__ __launch_bounds__(64 * ((H + 15) / 16 / HS) * DS, 2) void attn_rows_kernel(const AttnParams p) {
    constexpr int NHG = (H + 15) / 16;  // 16-head groups of a row
    constexpr int NHGW = NHG / HS;      // of which this workgroup's head slice holds
    static_assert(NHG % HS == 0, "head slices of whole 16-head groups");
    constexpr int NW = NHGW * DS;
    constexpr int NT = 64 * NW;
    typedef TileGeom<CT, D> G;
    constexpr int NS = D / 32, NDT = D / 16 / DS;
    constexpr int PAIRS = 4 * (D / 8);
    // DS tiles per round: thread group ts (NT / DS threads) gathers tile DS*round + ts, so every
    // thread takes part in the gather; each wave then computes the round's DS tiles.
    constexpr int TPR = DS;
    constexpr int TT = NT / TPR;                // threads per tile
    constexpr int PPT = (PAIRS + TT - 1) / TT;  // pairs per thread

    // Tile pairs (see store_pair_k) for the BF16 512-wide shape with two tiles per round.
    constexpr bool PAIRED = TPR == 2 && D == 512 && sizeof(CT) == 2;
    // One buffer set per round parity: TPR tiles (paired: two K tiles, also read as the PV operand).
    constexpr int SET_ELEMS = PAIRED ? 2 * G::K_ELEMS : TPR * (G::K_ELEMS + G::V_ELEMS);
    __shared__ __attribute__((aligned(16))) CT tiles[2][SET_ELEMS];
    // Paired: per wave, the partial scores of its half of the reduction (2 tiles x 64 lanes).
    __shared__ f32x4 xch[PAIRED ? 128 * NW : 1];
    __shared__ float rope_cs[R];
    __shared__ uint32_t vmask[kMaxTiles + 1];  // validity bits of each tile's 16 entries, written once
    // this row's selected indices (topk entries; sized at launch, so that two workgroups of the
    // 64-head shape share a CU when topk is small)
    extern __shared__ __attribute__((aligned(16))) int32_t sel[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int ts = tid / TT, tl = tid % TT;  // this thread's tile of a round, and its index there
    // Unit u is a row, or (decode) one of the S splits of a row's tiles: each split takes an
    // even-length run of tiles and leaves its softmax state for attn_merge_kernel.  A unit's HS head
    // slices are separate workgroups; their ids follow each other on one XCD (workgroup ids go
    // round-robin over the 8 XCDs), so the slices gather the unit's rows through the same L2.
    const int S = DECODE ? p.splits : 1;
    int u, hs;
    if constexpr (HS == 1) {
        u = (int)blockIdx.x;
        hs = 0;
    } else {
        const int s8 = (int)(blockIdx.x >> 3);
        hs = s8 % HS;
        u = ((s8 / HS) << 3) | (int)(blockIdx.x & 7);
        if (u >= (DECODE ? p.rows * S : p.rows)) return;  // padding workgroup (before any barrier)
    }
    const int split = DECODE ? u % S : 0;
    RowCtx c;
    row_ctx_init<D, KVT, SWT, DECODE>(p, c, DECODE ? u / S : u);
    const int n_all = (p.window + p.topk) / 16;
    const int per = S > 1 ? ((n_all + S - 1) / S + 1) & ~1 : n_all;
    const int tb = split * per;  // first tile of this workgroup
    const int n_tiles = tb < n_all ? (n_all - tb < per ? n_all - tb : per) : 0;  // its tiles: tb ..

    // The first selected index of each thread is loaded before the float64 rope angles are
    // computed, so that latency and the angles overlap.
    const int32_t idx0 = tid < p.topk ? p.idx[(int64_t)c.r * p.topk + tid] : 0;
    if (tid < R / 2) {
        float cs, sn;
        rope_angle(c.pos, p.inv_freq[tid], cs, sn);
        rope_cs[2 * tid] = cs;
        rope_cs[2 * tid + 1] = sn;
    }
    for (int i = tid; i < n_tiles; i += NT) vmask[tb + i] = 0u;
    if (tid < p.topk) sel[tid] = idx0;
    for (int i = tid + NT; i < p.topk; i += NT) sel[i] = p.idx[(int64_t)c.r * p.topk + i];

    const int hg = NHGW * hs + wave / DS;  // this wave's 16-head group of the row
    const int h = 16 * hg + li;
    const int dt0 = (wave % DS) * NDT;  // this wave's first 16-column output block
    // Paired: the two waves of a head group each hold and reduce over half of the query.
    constexpr int NQ = PAIRED ? NS / 2 : NS;
    const int s0 = PAIRED ? (wave % 2) * NQ : 0;
    typename Mma<CT>::Frag8 qf[NQ];
#pragma unroll
    for (int s = 0; s < NQ; ++s)
        qf[s] = (H % 16 == 0 || h < H) ? load_q_frag<QT, CT, D>(p.q, ((int64_t)c.r * H + h) * D, s0 + s, g)
                                       : zero_frag8<CT>();
    float m = kNegInf, l = 0.f;
    if ((H % 16 == 0 || h < H) && split == 0) {
        m = p.sink[h] * kLog2e;  // the sink is the initial state: max = sink, sum = 1
        l = (g == 0) ? 1.f : 0.f;
    }
    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The raw bytes of the next PF rounds' tiles are in flight in registers (slot q % PF holds round
    // q's); the loop is unrolled by PF so every slot index is a constant.
    constexpr int PF = (DECODE || HS > 1) ? CSA2_ATTN_DECODE_PF : CSA2_ATTN_PREFILL_PF;
    RawPair raw[PF][PPT];
    auto load_tile = [&](int tile, RawPair* rw) {
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int pr = tl + k * TT;
            if (pr < PAIRS) load_pair<D, KVT, SWT, DECODE>(p, c, sel, tile, pr / (D / 8), pr % (D / 8), rw[k]);
        }
    };
    // Tile buffer b = TPR * set + i: its K tile, and (not paired) its PV copy.
    auto kbuf = [&](int b) -> CT* {
        return tiles[b / TPR] + (b % TPR) * (PAIRED ? G::K_ELEMS : G::K_ELEMS + G::V_ELEMS);
    };
    auto vbuf = [&](int b) -> CT* { return kbuf(b) + G::K_ELEMS; };
    auto store_tile = [&](int tile, int b, const RawPair* raw) {  // tile into buffer b
        CT* Kt = kbuf(b);
        uint32_t bits = 0;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int pr = tl + k * TT;
            if (pr < PAIRS) {
                const int jb = pr / (D / 8), x8 = pr % (D / 8);
                if constexpr (PAIRED)
                    store_pair_k<KVT, SWT>(raw[k], tile * 16 < p.window, Kt, jb, x8);
                else
                    store_pair<D, CT, G::KS, G::VS, KVT, SWT>(raw[k], tile * 16 < p.window, Kt, vbuf(b), jb, x8);
                if (x8 == 0) bits |= raw[k].valid << (4 * jb);
            }
        }
        if (bits) atomicOr(&vmask[tile], bits);
    };
    // With tile pairs, an odd tile count leaves the last pair's second buffer without a tile:
    // it is zero-filled (its mask is empty, so it adds exactly nothing).
    auto zero_tile = [&](int b) {
        if constexpr (PAIRED) {
            RawPair z = {};  // every row invalid (valid == 0): the stores write zeros
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                const int pr = tl + k * TT;
                if (pr < PAIRS) store_pair_k<KVT, SWT>(z, false, kbuf(b), pr / 64, pr % 64);
            }
        }
    };

    __syncthreads();  // rope table and vmask reset visible
    const int n_rounds = (n_tiles + TPR - 1) / TPR;
    if (ts < n_tiles) {
        load_tile(tb + ts, raw[0]);
        store_tile(tb + ts, ts, raw[0]);
    } else if (PAIRED && ts == n_tiles) {
        zero_tile(ts);
    }
#pragma unroll
    for (int j = 1; j <= PF; ++j)
        if (TPR * j + ts < n_tiles) load_tile(tb + TPR * j + ts, raw[j % PF]);
    __syncthreads();
    for (int rd0 = 0; rd0 < n_rounds; rd0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        const int rd = rd0 + j;
        if (rd >= n_rounds) break;  // the same in every wave
        const int bs = (rd & 1) * TPR;
        if constexpr (PAIRED) {
            // (an odd last tile is paired with the zero-filled buffer, under an empty mask)
            const int t = 2 * rd;
            tile_pair_compute<NDT>(kbuf(bs), kbuf(bs + 1), vmask[tb + t], t + 1 < n_tiles ? vmask[tb + t + 1] : 0u,
                                   qf, wave % 2, xch + 128 * wave, xch + 128 * (wave ^ 1), p.scale_log2, g, li,
                                   lane, m, l, acc, dt0);
        } else {
#pragma unroll
            for (int jt = 0; jt < TPR; ++jt) {
                const int t = rd * TPR + jt;
                if (t < n_tiles)
                    tile_compute<D, CT, G::KS, G::VS, NDT>(kbuf(bs + jt), vbuf(bs + jt), vmask[tb + t], qf, p.scale_log2,
                                                           g, li, m, l, acc, dt0);
            }
        }
        // the next round's tiles go into the other buffer set; their loads were issued PF rounds ago,
        // and the slot they free takes the tiles PF rounds after them
        const int tn = (rd + 1) * TPR + ts;
        if (tn < n_tiles) {
            store_tile(tb + tn, (bs ^ TPR) + ts, raw[(j + 1) % PF]);
            if (tn + PF * TPR < n_tiles) load_tile(tb + tn + PF * TPR, raw[(j + 1) % PF]);
        } else if (PAIRED && tn == n_tiles && (n_tiles & 1)) {
            zero_tile((bs ^ TPR) + ts);
        }
        __syncthreads();
    }
    }

    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (h >= H) return;
    if (S > 1) {  // this split's state (max in log2 units, sum and values relative to it) for the merge
        float* part = p.part + (((int64_t)c.r * NHG + hg) * S + split) * (16 * (2 + D));
        if (wave % DS == 0 && g == 0) {
            part[li] = m;
            part[16 + li] = l;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            *reinterpret_cast<f32x4*>(part + 32 + li * D + 16 * (dt0 + dt) + 4 * g) = acc[dt];
        return;
    }
    const float inv = 1.f / l;
    const int64_t obase = ((int64_t)c.r * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int d0 = 16 * (dt0 + dt) + 4 * g;
        emit4<D, R, OT>(p.out, obase + d0, d0, acc[dt], inv, rope_cs);
    }
}

// ---------------------------------------------------------------------------
// Prefill rows of the 64-head, 512-wide shape over BF16 rows, on 32x32x16
// MFMAs: one workgroup of four waves per query row, one wave per SIMD (its
// 128 accumulator registers in AGPRs).  Wave w owns the 32 heads 32 (w / 2) ..
// + 31; the two waves of a 32-head block split the QK reduction (256
// dimensions each; partial scores exchanged through LDS, and a + b == b + a, so
// both form bit-identical scores and softmax states) and the output columns
// (256 each).  A round takes the two tiles of 16 entries that one 32-row MFMA
// operand spans:
//   S^T (32 entries x 32 heads) = K . q^T   (A: K rows from LDS, B: q in registers)
//   out^T (32 columns x 32 heads) += V^T . P^T
// The result layout of the first (lane l: head l % 32; register i: entry
// 8 (i / 4) + 4 (l / 32) + i % 4) is the P^T operand of the second once the
// reduction slots are relabelled -- slot 8 (l / 32) + e of k-step t is entry
// 16 t + 8 (e / 4) + 4 (l / 32) + e % 4 in both operands -- so probabilities
// stay in registers, and the V^T operand is two transposing LDS reads
// (lds_col4) of the row-major K tile.  Each K element read from LDS feeds 32
// heads (16 with the 16x16 shape), and a lane's accumulator is one head's.
//
// One wave per SIMD has no second wave to hide its latencies, so the rounds are
// software-pipelined over three tile sets, with the work of different rounds
// side by side in straight-line code the compiler can interleave:
//   (1) QK of round r (its accumulator starts at the entries' score bias), the
//       stores of round r + 1's tiles (loaded PF rounds before) and the loads
//       of round r + 1 + PF, the probabilities of round r - 1 and its PV;
//   (2) the exchange of partial scores: the round's one barrier;
//   (3) the running max of round r and, rarely, the lazy rescale.
// One barrier per round suffices: a tile set's last reader is the PV of its
// round, in the next round's phase (1), and the set is rewritten in the phase
// (1) after that, past that round's barrier; the exchange buffer alternates
// with the round's parity.  Every row address is
// prepared once per workgroup (absent rows and the rounds past the end point at
// the zero row and carry a -inf score bias), so the gather has no branch.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
// global-memory view of a row address held as an integer (a flat load would also count against the
// LDS wait counter)
typedef __attribute__((address_space(1))) u32x4 gu32x4;

__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// a *= s for an accumulator that lives in AGPRs.  Written as explicit AGPR reads and writes: a
// plain vector multiply inside the loop made the compiler keep all 128 accumulator registers in
// VGPRs (copying them to AGPRs around every MFMA) and spill.
__device__ __forceinline__ void acc_scale(f32x16& a, float s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float t, u;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(a[i]));
        t *= s;
        asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(u) : "v"(t));
        a[i] = u;
    }
}

// The larger of v over the wave's two 32-lane halves, in every lane (v_permlane32_swap: no LDS).
__device__ __forceinline__ float max_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Entries (window + topk) a row of attn_prefill_kernel may have (longer rows go to attn_rows_kernel),
// and a row's tables: every entry, then one round of zero rows.  Two rows' tables are kept: the
// current row's and the next one's, built while the current row is computed.
constexpr int kWideMaxSel = 1024;
constexpr int kWideEntries = kWideMaxSel + 32;

// A row's geometry for the wide kernel's tables.
__device__ __forceinline__ void wide_row_setup(const AttnParams& p, int r, RowCtx& c) {
    row_ctx_init<512, CSA2_BF16, CSA2_BF16, false>(p, c, r);
}

// Workgroup b takes the contiguous rows [row0, row0 + nk) (consecutive rows share most of their
// window rows, which then stay in this CU's caches).  The rounds of all its rows form one stream:
// the gather runs PF + 1 rounds ahead across row boundaries, and at a boundary the finished row's
// output is normalised and stored while the next row's first rounds are computed.  A row's tables
// and rope angles are built during the row before it; its query is loaded at the end of that row.
__global__ __launch_bounds__(256, 1) void attn_prefill_kernel(const AttnParams p, int rows_per_wg) {
    constexpr int H = 64, D = 512, R = 64, NT = 256;
    constexpr int TE = 16 * 512;  // elements of one K tile
    constexpr int RB = 2 * D;     // bytes of one stored row
    constexpr int PF = CSA2_ATTN_WIDE_PF;
    constexpr int KE = (kWideEntries + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) __bf16 tiles[3][2 * TE];
    __shared__ f32x4 xch[2][4][4][64];  // by round parity, per wave: its partial S^T, register quad q of every lane
    __shared__ __attribute__((aligned(16))) uint64_t eaddr[2][kWideEntries];  // by row parity: entry e's row
    __shared__ __attribute__((aligned(16))) float ebias[2][kWideEntries];     // 0, or -inf: not there
    __shared__ float rope_cs[2][R];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gk = lane >> 5, li = lane & 15, a16 = (lane >> 4) & 1;
    const int hb = wave >> 1, half = wave & 1;
    const int h = 32 * hb + (lane & 31);
    const int row0 = (int)blockIdx.x * rows_per_wg;
    const int nk = p.rows - row0 < rows_per_wg ? p.rows - row0 : rows_per_wg;  // rows of this workgroup (>= 1)
    const int W = p.window;
    const int n_sel = W + p.topk;
    const int n = (n_sel + 31) / 32;  // rounds per row

    // Table of row slot k: entry e's row address (the zero row where there is none) and score bias.
    uint32_t ids[KE];
    auto load_ids = [&](int r) {
        if (p.topk > 0) {
            const int32_t* idr = p.idx + (int64_t)r * p.topk;
#pragma unroll
            for (int k = 0; k < KE; ++k) {
                const int j = tid + NT * k - W;
                ids[k] = (uint32_t)idr[j < 0 ? 0 : (j < p.topk ? j : p.topk - 1)];
            }
        }
    };
    auto build_tables = [&](const RowCtx& rc, int buf) {
#pragma unroll
        for (int k = 0; k < KE; ++k) {
            const int e = tid + NT * k;
            if (e < 32 * (n + 1)) {
                const uint8_t* a = g_zero_row;
                bool valid = false;
                if (e < W) {
                    valid = (uint32_t)(e - rc.win_lo) < (uint32_t)(rc.win_hi - rc.win_lo);
                    if (valid) a = rc.swa0 + (uint64_t)e * RB;
                } else if (e < n_sel) {
                    valid = ids[k] < rc.nv32;  // group-causal mask; -1 wraps to the top
                    if (valid) a = rc.kv0 + (uint64_t)ids[k] * RB;
                }
                eaddr[buf][e] = reinterpret_cast<uint64_t>(a);
                ebias[buf][e] = valid ? 0.f : kNegInf;
            }
        }
        if (tid < R / 2) {
            float cs, sn;
            rope_angle(rc.pos, p.inv_freq[tid], cs, sn);
            rope_cs[buf][2 * tid] = cs;
            rope_cs[buf][2 * tid + 1] = sn;
        }
    };

    RowCtx c;
    wide_row_setup(p, row0, c);
    load_ids(row0);
    build_tables(c, 0);
    // round 2's set is read (as round -1, under zero probabilities) before anything is stored there
    {
        u32x4* z = reinterpret_cast<u32x4*>(tiles[2]) + tid;
#pragma unroll
        for (int k = 0; k < 8; ++k) z[NT * k] = u32x4{0u, 0u, 0u, 0u};
    }

    // q^T operand of k-step s: head h, dimensions 256 half + 16 s + 8 gk .. + 7
    bf16x8 qf[16];
    auto load_q = [&](int r) {
        const uint16_t* q16 = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)r * H + h) * D + 256 * half + 8 * gk;
#pragma unroll
        for (int s = 0; s < 16; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q16 + 16 * s));
    };
    load_q(row0);
    const float sink_m = p.sink[h] * kLog2e;  // the sink is each row's initial state: max = sink, sum = 1
    float m = sink_m;
    float l = gk == 0 ? 1.f : 0.f;
    f32x16 acc[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;

    // Tile layout: row j of a K tile holds its 64 16-byte chunks with chunk c at c ^ sw(j), sw(j)
    // the row's two 2-bit halves swapped.  The QK read (16 rows, one chunk) and the transposing PV
    // read (4 consecutive rows x 4 consecutive chunks) then both touch 16 distinct chunk slots of
    // the 64 banks; with c ^ j the PV read put its 4 rows on the same 4 slots.
    auto sw = [](int j) { return ((j & 3) << 2) | (j >> 2); };
    // K operand (QK): lane l reads entry l % 32 of the round (tile (l % 32) / 16, row jr), chunk
    // 32 half + 2 s + gk; the lane-dependent part takes 8 values (s mod 8).
    const int jr = lane & 15;
    int ko[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) ko[b] = a16 * TE + jr * 512 + 256 * half + 8 * ((2 * b + gk) ^ sw(jr));
    // V^T operand (PV, lds_col4): lane j of a 16-lane group names row 4 gk + j / 4 (+ 8 for the second
    // read) of tile t, columns 256 half + 32 cb + 16 a16 + 4 (j % 4) .. + 3: chunk 32 half + 4 cb +
    // 2 a16 + (j % 4) / 2, element 4 (j % 2) of it.
    const int vr0 = 4 * gk + (li >> 2), vr1 = vr0 + 8;
    const int vcb = 2 * a16 + ((li & 3) >> 1);
    int vo0[4], vo1[4];  // by cb mod 4 (cb / 4 adds 16 chunks, beyond the XOR's 4 bits)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        vo0[b] = vr0 * 512 + 256 * half + 8 * ((4 * b + vcb) ^ sw(vr0)) + 4 * (li & 1);
        vo1[b] = vr1 * 512 + 256 * half + 8 * ((4 * b + vcb) ^ sw(vr1)) + 4 * (li & 1);
    }
    // Gather: thread t takes tile t / 128 of a round, rows 4 ((t % 128) / 64 + 2 k) .. + 3 (k = 0, 1),
    // 16-byte chunk t % 64 of each: one load instruction covers whole rows.
    const int gt = tid >> 7, gx = tid & 63, gj = (tid >> 6) & 1;
    const int xo = 16 * gx;
    u32x4 raw[PF][2][4];
    // the round (lk, lrd) of row slot lk; past the last row: the last row's round of zero rows
    auto load_round = [&](int lk, int lrd, u32x4(&rw)[2][4]) {
        const int base = lk < nk ? (lk & 1) * kWideEntries + 32 * lrd : ((nk - 1) & 1) * kWideEntries + 32 * n;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const u64x2* ea = reinterpret_cast<const u64x2*>(&eaddr[0][0] + base + 16 * gt + 4 * (gj + 2 * k));
            const u64x2 a01 = ea[0], a23 = ea[1];
            rw[k][0] = *reinterpret_cast<const gu32x4*>(a01[0] + xo);
            rw[k][1] = *reinterpret_cast<const gu32x4*>(a01[1] + xo);
            rw[k][2] = *reinterpret_cast<const gu32x4*>(a23[0] + xo);
            rw[k][3] = *reinterpret_cast<const gu32x4*>(a23[1] + xo);
        }
    };
    auto store_round = [&](int set, const u32x4(&rw)[2][4]) {
        __bf16* Kt = tiles[set] + gt * TE;
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * (gj + 2 * k) + i;
                *reinterpret_cast<u32x4*>(Kt + j * 512 + 8 * (gx ^ sw(j))) = rw[k][i];
            }
    };
    // Normalises, rotates back and stores the finished row of slot k (its output rows leave as 8-byte
    // pieces; done once per row, in the middle of the stream).
    auto emit_row = [&](int k, float lsum) {
        const float inv = 1.f / lsum;
        const int64_t obase = ((int64_t)(row0 + k) * H + h) * D;
        const float* rcs = rope_cs[k & 1];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int d0 = 256 * half + 32 * cb + 8 * q + 4 * gk;
                emit4<D, R, CSA2_BF16>(p.out, obase + d0, d0,
                                       f32x4{acc[cb][4 * q], acc[cb][4 * q + 1], acc[cb][4 * q + 2], acc[cb][4 * q + 3]},
                                       inv, rcs);
            }
        }
    };

    __syncthreads();  // row 0's tables and rope angles, and the zeroed set, visible
    int lk = 0, lrd = 0;  // the gather's next round
    auto advance = [&](int& kk, int& rr) {
        if (++rr == n) {
            rr = 0;
            ++kk;
        }
    };
    load_round(lk, lrd, raw[0]);
    advance(lk, lrd);
    store_round(0, raw[0]);
#pragma unroll
    for (int j = 1; j <= PF; ++j) {
        load_round(lk, lrd, raw[j % PF]);
        advance(lk, lrd);
    }
    float xp[16];  // the previous round's scores (scaled by scale_log2 when used): none yet
#pragma unroll
    for (int i = 0; i < 16; ++i) xp[i] = kNegInf;
    int s_cur = 0, s_next = 1, s_prev = 2;
    RowCtx cn;  // the next row's geometry, while its tables are built
    __syncthreads();
    const int total = nk * n;
    int k = 0, rd = 0;  // this round: row slot k, round rd of that row
    for (int g0 = 0; g0 < total; g0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        const int g = g0 + j;
        if (g >= total) break;  // the same in every wave
        const __bf16* set = tiles[s_cur];
        // (1) QK of this round over the wave's 256 dimensions (one accumulation chain, started at the
        // entries' bias: 0, or -inf for entries that are not there -- both waves of the pair add it, and
        // -inf + -inf = -inf) ...
        f32x16 sc;
        {
            const f32x4* eb = reinterpret_cast<const f32x4*>(&ebias[k & 1][32 * rd + 4 * gk]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 b = eb[2 * q];
#pragma unroll
                for (int e = 0; e < 4; ++e) sc[4 * q + e] = b[e];
            }
        }
#pragma unroll
        for (int s = 0; s < 16; ++s)
            sc = mma32(lds_frag8<__bf16>(set + ko[s & 7] + 128 * (s >> 3)), qf[s], sc);
        // ... the next round's tiles into their set, and loads PF rounds ahead ...
        store_round(s_next, raw[(j + 1) % PF]);
        load_round(lk, lrd, raw[(j + 1) % PF]);
        advance(lk, lrd);
        // ... and the previous round's probabilities (x - m_use <= 8; -inf -> 0) and PV (its tiles and
        // probabilities are ready, so it needs no exchange; at a row boundary they are the last round
        // of the row before, with its softmax state)
        const float m_use = (m == kNegInf) ? 0.f : m;
        float pr[16];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xp[i], p.scale_log2, -m_use));
            psum += pr[i];
        }
        l += psum;
        bf16x8 pb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
            pb[t] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(pr[8 * t], pr[8 * t + 1]),
                                                     pack_bf16x2(pr[8 * t + 2], pr[8 * t + 3]),
                                                     pack_bf16x2(pr[8 * t + 4], pr[8 * t + 5]),
                                                     pack_bf16x2(pr[8 * t + 6], pr[8 * t + 7])});
        {
            const __bf16* pset = tiles[s_prev];
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const __bf16* Kt = pset + t * TE + 128 * (cb >> 2);
                    const u32x2 v0 = lds_col4(Kt + vo0[cb & 3]), v1 = lds_col4(Kt + vo1[cb & 3]);
                    acc[cb] = mma32(__builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y}), pb[t], acc[cb]);
                }
            }
        }
        // (2) the exchange of partial scores
        f32x16 st = sc;
#pragma unroll
        for (int q = 0; q < 4; ++q) xch[g & 1][wave][q][lane] = f32x4{st[4 * q], st[4 * q + 1], st[4 * q + 2], st[4 * q + 3]};
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 o = xch[g & 1][wave ^ 1][q][lane];
            st[4 * q] += o[0];
            st[4 * q + 1] += o[1];
            st[4 * q + 2] += o[2];
            st[4 * q + 3] += o[3];
        }
        // (3) at a row boundary, the finished row leaves and the softmax state restarts at the sink
        if (rd == 0 && k > 0) {
            emit_row(k - 1, l + shfl_xor(l, 32));
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;
            m = sink_m;
            l = gk == 0 ? 1.f : 0.f;
        }
        // The next row's tables: its indices are loaded in its predecessor's first round and written
        // in the second, after that round's barrier (the buffer's last readers are two rounds back);
        // the gather first reads them at least two barriers later.
        if (k + 1 < nk) {
            if (rd == 0) {
                wide_row_setup(p, row0 + k + 1, cn);
                load_ids(row0 + k + 1);
            } else if (rd == 1) {
                build_tables(cn, (k + 1) & 1);
            }
        }
        // the running max of this round's scores (register i: entry 32 rd + 8 (i / 4) + 4 gk + i % 4)
        // over both halves of the wave, in log2 units (scale_log2 > 0, so scaling commutes with the max)
        float tmax = fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]));
#pragma unroll
        for (int i = 4; i < 16; i += 4) tmax = fmaxf(tmax, fmaxf(fmaxf(st[i], st[i + 1]), fmaxf(st[i + 2], st[i + 3])));
        tmax = max_halves(tmax) * p.scale_log2;
        // Lazy rescaling: m is only a reference point, moved (with acc and l rescaled) only when a
        // head's scores exceed it by more than 2^8; the probabilities then stay below 256.  acc
        // here holds every round of the row up to the previous one, whose probabilities used the old m.
        const uint64_t need_rescale = __ballot(tmax > m + 8.f);
        if (__builtin_expect(__builtin_amdgcn_readfirstlane((uint32_t)(need_rescale | (need_rescale >> 32))) != 0u, 0)) {
            const float m_new = fmaxf(m, tmax);
            const float alpha = exp2f(m - m_new);  // 0 when m was -inf
            l *= alpha;
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) acc_scale(acc[cb], alpha);
            m = m_new;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) xp[i] = st[i];
        // the next row's query, once this row's last QK has used the current one
        if (rd == n - 1 && k + 1 < nk) load_q(row0 + k + 1);
        const int s_old = s_prev;
        s_prev = s_cur;
        s_cur = s_next;
        s_next = s_old;
        if (++rd == n) {
            rd = 0;
            ++k;
        }
    }
    }
    // the last round's probabilities and PV, and the last row's output
    {
        const float m_use = (m == kNegInf) ? 0.f : m;
        float pr[16];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xp[i], p.scale_log2, -m_use));
            psum += pr[i];
        }
        l += psum;
        bf16x8 pb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
            pb[t] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(pr[8 * t], pr[8 * t + 1]),
                                                     pack_bf16x2(pr[8 * t + 2], pr[8 * t + 3]),
                                                     pack_bf16x2(pr[8 * t + 4], pr[8 * t + 5]),
                                                     pack_bf16x2(pr[8 * t + 6], pr[8 * t + 7])});
        const __bf16* pset = tiles[s_prev];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const __bf16* Kt = pset + t * TE + 128 * (cb >> 2);
                const u32x2 v0 = lds_col4(Kt + vo0[cb & 3]), v1 = lds_col4(Kt + vo1[cb & 3]);
                acc[cb] = mma32(__builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y}), pb[t], acc[cb]);
            }
        }
    }
    emit_row(nk - 1, l + shfl_xor(l, 32));
}

// Merge of the splits' partial states of one (row, 16-head group): the largest max, each state's
// sum and values weighted by 2^(its max - that max), then normalisation, the inverse rotation of
// the rope tail and the store.
// One workgroup per (row, head group, quarter of the D columns): 64 threads per head... every thread
// owns 4 consecutive columns of one head; the splits' states are read once each, all loads issued
// before any is used.
template <int H, int D, int R, int OT>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnParams p) {
    constexpr int NHG = (H + 15) / 16;
    constexpr int DQ = D / 4;             // columns per workgroup
    constexpr int TPH = DQ / 4;           // threads per head (4 columns each)
    constexpr int HPW = 256 / TPH;        // heads per pass
    constexpr int PART = 16 * (2 + D);
    static_assert(R <= DQ && TPH <= 256 && 256 % TPH == 0, "the rope tail lies in the last quarter");
    __shared__ float rope_cs[R];
    const int S = p.splits;
    const int q4 = blockIdx.x % 4, rh = blockIdx.x / 4;
    const int r = rh / NHG, hg = rh % NHG;
    const int tid = threadIdx.x;
    if (q4 == 3 && tid < R / 2) {  // the rope tail lies in the last quarter (R <= D / 4)
        float cs, sn;
        rope_angle(p.pos[r], p.inv_freq[tid], cs, sn);
        rope_cs[2 * tid] = cs;
        rope_cs[2 * tid + 1] = sn;
    }
    __syncthreads();
    const float* part = p.part + (int64_t)rh * S * PART;
    for (int hh = tid / TPH; hh < 16; hh += HPW) {
        const int h = 16 * hg + hh;
        const int d0 = q4 * DQ + 4 * (tid % TPH);
        float ms[kMaxSplits], ls[kMaxSplits];
        f32x4 vs[kMaxSplits];
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s) {
            if (s < S) {
                ms[s] = part[s * PART + hh];
                ls[s] = part[s * PART + 16 + hh];
                vs[s] = *reinterpret_cast<const f32x4*>(part + s * PART + 32 + hh * D + d0);
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s)
            if (s < S) mx = fmaxf(mx, ms[s]);
        float L = 0.f;
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s) {
            if (s < S) {
                const float w = ms[s] == kNegInf ? 0.f : exp2f(ms[s] - mx);
                L += ls[s] * w;
                sum += vs[s] * w;
            }
        }
        if (h < H) emit4<D, R, OT>(p.out, ((int64_t)r * H + h) * D + d0, d0, sum, L > 0.f ? 1.f / L : 0.f, rope_cs);
    }
}

// Compute units of the current device (cached per device).
static int device_cu_count() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cached[dev] = v;
    }
    return cached[dev];
}

// ---------------------------------------------------------------------------
template <int H, int D, int R, class CT, int QT, int KVT, int SWT, int OT>
static hipError_t launch_attn(const AttnParams& p, bool decode, hipStream_t stream) {
    constexpr int NHG = (H + 15) / 16;
    // the 64-head shapes split each head group's output columns over two waves, and a row's heads
    // over HS workgroups
    constexpr int DS = (H == 64 && D == 512) ? 2 : 1;
    constexpr int HS = (H == 64 && D == 512 && KVT == CSA2_BF16 && SWT == CSA2_BF16) ? CSA2_ATTN_BF16_DECODE_SLICES : 1;
    const size_t sel_bytes = (size_t)(p.topk > 4 ? p.topk : 4) * sizeof(int32_t);
    if (decode) {
        constexpr int NT = 64 * (NHG / HS) * DS;
        const int units = p.rows * p.splits;
        const unsigned grid = HS == 1 ? (unsigned)units : (unsigned)(8 * HS * ((units + 7) / 8));
        hipLaunchKernelGGL((attn_rows_kernel<H, D, R, CT, QT, KVT, SWT, OT, true, DS, HS>), dim3(grid), dim3(NT),
                           sel_bytes, stream, p);
        if (p.splits > 1)
            hipLaunchKernelGGL((attn_merge_kernel<H, D, R, OT>), dim3((unsigned)(p.rows * NHG * 4)), dim3(256), 0,
                               stream, p);
    } else if (H == 64 && D == 512 && KVT == CSA2_BF16 && SWT == CSA2_BF16 && CSA2_ATTN_PREFILL_WIDE &&
               p.window + p.topk <= kWideMaxSel) {
        // one workgroup per CU, each over a contiguous run of rows (the stream needs rows of at least
        // PF + 4 rounds for its next-row tables; shorter rows get one workgroup each)
        if (p.rows <= 0) return hipSuccess;
        const int n_rounds = (p.window + p.topk + 31) / 32;
        int per = 1;
        if (n_rounds >= CSA2_ATTN_WIDE_PF + 4) {
            const int cus = device_cu_count();
            per = (p.rows + cus - 1) / cus;
        }
        const int grid = (p.rows + per - 1) / per;
        hipLaunchKernelGGL(attn_prefill_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p, per);
    } else {
        constexpr int NT = 64 * NHG * DS;
        hipLaunchKernelGGL((attn_rows_kernel<H, D, R, CT, QT, KVT, SWT, OT, false, DS, 1>), dim3((unsigned)p.rows),
                           dim3(NT), sel_bytes, stream, p);
    }
    return hipGetLastError();
}

// Splits of a decode row's entries: enough workgroups (one per CU: 158 KB of LDS each) to fill the
// 256 CUs, at most 4 from 32 rows on, each split keeping at least one pair of tiles; the caller may
// ask for a count (1..8).
int attn_decode_splits(int rows, int heads, int dim, int window, int topk, int requested) {
    (void)heads;
    (void)dim;
    if (rows <= 0) return 1;
    if (requested > 0) return requested < kMaxSplits ? requested : kMaxSplits;
    int s = 256 / rows;
    // From 32 rows on, 4 splits measured faster than more (the merge reads every split's state)
    if (rows >= 32 && s > 4) s = 4;
    const int by_tiles = (window + topk) / 32;  // each split keeps at least one pair of tiles
    if (s > by_tiles) s = by_tiles;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : s;
}

size_t attn_decode_workspace(int rows, int heads, int dim, int splits) {
    if (splits <= 1 || rows <= 0) return 0;
    return (size_t)rows * ((heads + 15) / 16) * splits * 16 * (2 + dim) * sizeof(float);
}

bool attn_supported(const AttnShape& s) {
    if (s.heads == 4 && s.dim == 64 && s.rope_dim == 16)
        return s.q_dtype == CSA2_F32 && s.kv_dtype == CSA2_F32 && s.swa_dtype == CSA2_F32 && s.out_dtype == CSA2_F32;
    if (s.heads == 64 && s.dim == 512 && s.rope_dim == 64)
        return s.q_dtype == CSA2_BF16 && s.out_dtype == CSA2_BF16 &&
               (((s.kv_dtype == CSA2_BF16 || s.kv_dtype == CSA2_FP4_E2M1) &&
                 (s.swa_dtype == CSA2_BF16 || s.swa_dtype == CSA2_FP8_E4M3)) ||
                (s.kv_dtype == CSA2_FP4_E2M1_E4M3G16 && s.swa_dtype == CSA2_FP8_E4M3_E8M0G32));
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
        if (s.kv_dtype == CSA2_FP4_E2M1_E4M3G16 && s.swa_dtype == CSA2_FP8_E4M3_E8M0G32)
            return launch_attn<64, 512, 64, __bf16, CSA2_BF16, CSA2_FP4_E2M1_E4M3G16, CSA2_FP8_E4M3_E8M0G32, CSA2_BF16>(
                p, decode, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace csa2

// Device helpers shared by the CSA2 kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand layouts used throughout (verified on gfx950):
//   16x16x32 bf16 : lane l holds A[i = l%16][k = 8*(l/16) + e], B[k = 8*(l/16) + e][j = l%16], e < 8
//   16x16x16 bf16 : lane l holds A[i = l%16][k = 4*(l/16) + e], B[k = 4*(l/16) + e][j = l%16], e < 4
//   16x16x4  f32  : lane l holds A[i = l%16][k = l/16],         B[k = l/16][j = l%16]
//   16x16x128 fp8 : lane l holds 32 bytes of row/column l%16, k-group l/16
//   result        : lane l holds D[i = 4*(l/16) + r][j = l%16], r < 4
// The order of k inside a lane's operand is free as long as A and B use the
// same one (the product sums over k), which the loaders exploit to keep global
// reads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();
constexpr float kFltMax = 3.40282346638528859812e+38f;

// A score as the candidate pool ranks it: NaN as -inf, +-inf clipped to +-FLT_MAX.
__device__ __forceinline__ float pool_value(float x) {
    return __builtin_isnan(x) ? kNegInf : fminf(fmaxf(x, -kFltMax), kFltMax);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// float -> bfloat16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, b);
}

// Two floats -> a bf16 pair (lo in the low half), one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// cos/sin of pos * inv_freq in float64 (an fp32 angle at positions near 10^6
// would be off by up to ~0.06 rad), returned as float.
__device__ __forceinline__ void rope_angle(int64_t pos, double f, float& c, float& s) {
    double sd, cd;
    sincos((double)pos * f, &sd, &cd);
    c = (float)cd;
    s = (float)sd;
}

// Value of an E8M0 scale byte: 2^(e-127), e = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    if (e == 255u) return __builtin_nanf("");
    if (e == 0u) return __uint_as_float(0x00400000u);  // 2^-127 (subnormal)
    return __uint_as_float(e << 23);
}

// Two FP8-E4M3 codes of `w` (bytes 0,1 or 2,3) -> float (exact).
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// Two FP4-E2M1 codes of byte SEL of `w` (low nibble first) -> float (exact).
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Order-preserving 32-bit key of a score: NaN ranks as -inf and -0 as +0, and
// key(a) < key(b) exactly when a < b otherwise.  Its top 12 bits are the bin
// of the top-k histogram.
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN -> -inf
    if (u == 0x80000000u) u = 0u;                           // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr int kKeyBins = 4096;  // bins of the top 12 key bits

// Wave-level lane exchange (ds_bpermute based).
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ uint32_t shfl_xor(uint32_t v, int m) { return (uint32_t)__shfl_xor((int)v, m, 64); }

// Columns per entry of the block-key summary the scoring pass can write
// instead of the scores (the largest block key of each 8 consecutive columns).
constexpr int kKeyBlock = 8;

// Block key of a score: its order key, except that a NaN gets 0x007FFFFE, just
// below key(-inf) = 0x007FFFFF and in the same histogram bin (no other score
// has this key).  Block keys thus still tell an all-NaN block (pool score
// -inf) from one holding -inf (pool score -FLT_MAX).  0 = no valid column.
constexpr uint32_t kNanBlockKey = 0x007ffffeu;
__device__ __forceinline__ uint32_t block_key(float s) {
    return __builtin_isnan(s) ? kNanBlockKey : order_key(s);
}

// The candidate pool's block score from a block key (before pinning).
__device__ __forceinline__ float pool_value_of_block_key(uint32_t bk) {
    if (bk == kNanBlockKey) return kNegInf;
    const uint32_t bits = (bk & 0x80000000u) ? (bk & 0x7fffffffu) : ~bk;
    return pool_value(__uint_as_float(bits));
}

// ---------------------------------------------------------------------------
// MFMA wrappers.  Compute element type CT is __bf16 or float.
template <class CT>
struct Mma;

template <>
struct Mma<__bf16> {
    typedef bf16x8 Frag8;  // 8 elements of one k-group
    typedef s16x4 Frag4;   // 4 elements of one k-group
    static __device__ __forceinline__ f32x4 k32(f32x4 c, Frag8 a, Frag8 b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 k16(f32x4 c, Frag4 a, Frag4 b) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};

struct F32x8 { float v[8]; };
struct F32x4 { float v[4]; };

template <>
struct Mma<float> {
    typedef F32x8 Frag8;
    typedef F32x4 Frag4;
    // 16x16x32 as eight 16x16x4 steps: step e takes element e of every lane
    static __device__ __forceinline__ f32x4 k32(f32x4 c, const Frag8& a, const Frag8& b) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f32x4 k16(f32x4 c, const Frag4& a, const Frag4& b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
        return c;
    }
};

// 16x16x128 FP8-E4M3 x FP8-E4M3 (both operands format 0, unit E8M0 scales = 127).
__device__ __forceinline__ f32x4 mma_fp8_k128(f32x4 c, i32x8 a, i32x8 b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// s_waitcnt vmcnt(0): every vector-memory load of this wave has returned.
// Issued after loads made before a loop that loads again, it keeps the
// compiler's wait insertion -- which cannot order conditional loads across
// the loop's back edge -- from making the first use of those earlier values
// inside the loop wait for the loop's own loads still in flight.
__device__ __forceinline__ void wait_vmem_all() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0; expcnt 7 and lgkmcnt 15: no wait
}

// Waits until at most N of this wave's vector memory loads are outstanding (expcnt, lgkmcnt: no
// wait).  After it the compiler's own wait insertion knows that every older load has completed.
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Keeps the compiler from moving LDS accesses of one wave across this point.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

}  // namespace csa2

// Block scores of the hierarchical candidate pool, from FULL score rows, for gfx950.
//
// Block b of row r covers columns [b*B, (b+1)*B); its score is the largest
// visible score in it with NaN read as -inf and infinities clipped to the
// largest finite float, and the block holding the newest visible row is
// pinned to +inf ("DeepSeek-V4.1-Flash 架构解剖", special module "indexer",
// fig. 3b second level).  The ranking of those scores into the kept blocks is
// the top-k select with block-granular visibility (topk.hip).
//
// The pass is a pure HBM stream (4 B read per visible column, 4 B written per
// block).  Each lane reads 4 consecutive columns with one 16-byte load, so a
// wave covers 256 contiguous columns; the B/4 lanes of a block combine their
// maxima with xor shuffles and the first of them writes the block.  Columns at
// or beyond the row's visible prefix are not read.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

template <bool VEC>
__global__ __launch_bounds__(256) void block_max_kernel(const float* __restrict__ scores,
                                                        const int64_t* __restrict__ pos, int ratio, int64_t width,
                                                        int B, int64_t nb, float* __restrict__ out) {
    const int r = blockIdx.y;
    int64_t nv = (pos[r] + 1) / ratio;
    if (nv > width) nv = width;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4-column group
    const int64_t c0 = 4 * t;
    const float* srow = scores + (int64_t)r * width;
    float m = kNegInf;
    if (c0 < nv) {
        float v[4];
        if (VEC) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(srow + c0);
            v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (c0 + e < nv) ? srow[c0 + e] : kNegInf;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c0 + e < nv) m = fmaxf(m, pool_value(v[e]));
    }
    // B is a power of two in 4..64: a block is B/4 lanes of one wave.
    for (int o = 1; o < B / 4; o <<= 1) m = fmaxf(m, shfl_xor(m, o));
    if ((t & (B / 4 - 1)) == 0 && c0 < width) {
        const int64_t blk = c0 / B;
        const int64_t newest = nv > 0 ? (nv - 1) / B : -1;
        out[(int64_t)r * nb + blk] = (blk == newest) ? kPosInf : m;
    }
}

hipError_t launch_block_max(const float* scores, const int64_t* pos, int ratio, int64_t width, int block_rows,
                            int rows, float* out, hipStream_t stream) {
    const int64_t nb = (width + block_rows - 1) / block_rows;
    const int64_t groups = (width + 3) / 4;
    dim3 grid((unsigned)((groups + 255) / 256), (unsigned)rows);
    const bool vec = (width % 4) == 0 && (reinterpret_cast<uintptr_t>(scores) % 16) == 0;
    if (vec) hipLaunchKernelGGL(block_max_kernel<true>, grid, dim3(256), 0, stream, scores, pos, ratio, width,
                                block_rows, nb, out);
    else hipLaunchKernelGGL(block_max_kernel<false>, grid, dim3(256), 0, stream, scores, pos, ratio, width,
                            block_rows, nb, out);
    return hipGetLastError();
}

}  // namespace csa2

// gemm_f16_sparse.hip -- the 2:4 structured-sparse product and the
// compression that produces its operand.
#include "gemm_f16_tile.h"

namespace gemm_f16_impl {

// ---- 2:4 compression -------------------------------------------------------------
// One thread per 16 consecutive k of a row of A (M x K, K % 16 == 0): in
// each group of 4 it keeps the 2 entries of largest magnitude (compared as
// binary16 bit patterns without the sign; ties: lower position), writes
// them in position order to vals (M x K/2) and their positions, 2 bits per
// kept value, to one word of meta, stored slice-major (sp_meta_index).  VEC:
// A and vals 16-byte aligned (16-byte loads and stores).
template <bool VEC>
__global__ void __launch_bounds__(256) sp_compress_kernel(const half_t *__restrict__ A, half_t *__restrict__ vals,
                                                          unsigned short *__restrict__ meta, int64_t words,
                                                          int64_t M, int64_t kw)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x; w < words; w += stride) {
        unsigned short x[16];
        if constexpr (VEC) {
            const int4v lo = reinterpret_cast<const int4v *>(A)[2 * w];
            const int4v hi = reinterpret_cast<const int4v *>(A)[2 * w + 1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = (unsigned short)((unsigned)lo[e] & 0xffffu);
                x[2 * e + 1] = (unsigned short)((unsigned)lo[e] >> 16);
                x[8 + 2 * e] = (unsigned short)((unsigned)hi[e] & 0xffffu);
                x[8 + 2 * e + 1] = (unsigned short)((unsigned)hi[e] >> 16);
            }
        } else {
            const unsigned short *a = reinterpret_cast<const unsigned short *>(A) + 16 * w;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                x[e] = a[e];
        }
        unsigned short kept[8];
        unsigned word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned short *g = x + 4 * q;
            int best = 0;
#pragma unroll
            for (int p = 1; p < 4; ++p)
                if ((g[p] & 0x7fffu) > (g[best] & 0x7fffu))
                    best = p;
            int next = best == 0 ? 1 : 0;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                if (p != best && (g[p] & 0x7fffu) > (g[next] & 0x7fffu))
                    next = p;
            const int lo = best < next ? best : next, hi = best < next ? next : best;
            kept[2 * q] = g[lo];
            kept[2 * q + 1] = g[hi];
            word |= (unsigned)lo << (4 * q);
            word |= (unsigned)hi << (4 * q + 2);
        }
        if constexpr (VEC) {
            int4v out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = (int)((unsigned)kept[2 * e] | ((unsigned)kept[2 * e + 1] << 16));
            reinterpret_cast<int4v *>(vals)[w] = out;
        } else {
            unsigned short *v = reinterpret_cast<unsigned short *>(vals) + 8 * w;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = kept[e];
        }
        meta[sp_meta_index(w / kw, w % kw, M, kw)] = (unsigned short)word;
    }
}

hipError_t launch_sp_compress(const _Float16 *A, _Float16 *vals, uint16_t *meta, int64_t M, int64_t K, bool vec,
                              hipStream_t s)
{
    const int64_t words = M * (K / 16);
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((words + 255) / 256, 256 * 16));
    if (vec)
        hipLaunchKernelGGL(sp_compress_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, A, vals,
                           (unsigned short *)meta, words, M, K / 16);
    else
        hipLaunchKernelGGL(sp_compress_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, A, vals,
                           (unsigned short *)meta, words, M, K / 16);
    return hipGetLastError();
}


// Sparse configurations (A compressed 2:4; B as K x N, or given as N x K
// when BR; 16-byte loads).
template <bool BR>
static hipError_t launch_sparse_layout(int config, const KernelArgs &a, int64_t grid, hipStream_t s)
{
    switch (config) {
    case 0: return launch_one<256, 256, 64, 2, 4, 3, true, 8, 8, true, BR, 1, true>(a, grid, s);
    case 1: return launch_one<128, 128, 64, 2, 2, 3, true, 8, 8, true, BR, 1, true>(a, grid, s);
    case 2: return launch_one<256, 256, 64, 2, 2, 3, true, 8, 8, true, BR, 1, true>(a, grid, s);
    case 3: return launch_one<256, 256, 64, 2, 2, 3, true, 8, 8, true, BR, 2, true>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sparse(int config, const KernelArgs &a, bool trans_b, int64_t grid, hipStream_t s)
{
    return trans_b ? launch_sparse_layout<true>(config, a, grid, s) : launch_sparse_layout<false>(config, a, grid, s);
}

} // namespace gemm_f16_impl

// gemm_f16_kernels.hip -- the split-K reduction kernel and the dispatch of
// a planned call to the kernel of its layout (the tile kernel itself is in
// gemm_f16_tile.h).
#include <mutex>

#include "gemm_f16_tile.h"

namespace gemm_f16_impl {

// ---- static split-K scratch -------------------------------------------------------
// Device memory for the split-K partial sums of gemm_f16_split_static, for
// callers that cannot allocate: one array per GPU, held from module load
// until the process ends.  Host code never uses this name as an address
// (there it is only a host-side stand-in): static_scratch() looks up each
// device's own copy once and every kernel argument, copy or fill uses that.
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

hipError_t static_scratch(void **ptr)
{
    static std::mutex mutex;
    static void *addr[kMaxScratchDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mutex);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---- split-K reduction ---------------------------------------------------------
// C = rne16(epi(alpha * sum over s of W[s])) elementwise, the splits added in index
// order in fp32 (so the result does not depend on scheduling).  W holds
// `splits` slices of M x N fp32 one after another, C is M x N fp16, both
// with row pitch N: the flattened index e addresses the same element in
// both.  VEC4: four consecutive elements per step (M N % 4 == 0, C 8-byte
// aligned, W 16-byte aligned).  An HBM-bound stream: 4 splits + 2 bytes
// moved per output element.
template <bool VEC4>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *__restrict__ W, half_t *__restrict__ C,
                                                            int64_t mn, int splits, float alpha, int relu)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    if constexpr (VEC4) {
        const int64_t n4 = mn / 4;
        for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += stride) {
            float4v acc = __builtin_nontemporal_load(reinterpret_cast<const float4v *>(W) + q);
            for (int s = 1; s < splits; ++s) {
                const float4v v = __builtin_nontemporal_load(reinterpret_cast<const float4v *>(W + s * mn) + q);
                acc[0] += v[0];
                acc[1] += v[1];
                acc[2] += v[2];
                acc[3] += v[3];
            }
            acc[0] *= alpha;
            acc[1] *= alpha;
            acc[2] *= alpha;
            acc[3] *= alpha;
            if (relu) {
                acc[0] = __builtin_fmaxf(acc[0], 0.0f);
                acc[1] = __builtin_fmaxf(acc[1], 0.0f);
                acc[2] = __builtin_fmaxf(acc[2], 0.0f);
                acc[3] = __builtin_fmaxf(acc[3], 0.0f);
            }
            const half_t h0 = (half_t)acc[0], h1 = (half_t)acc[1], h2 = (half_t)acc[2], h3 = (half_t)acc[3];
            __builtin_nontemporal_store(half4{h0, h1, h2, h3}, reinterpret_cast<half4 *>(C) + q);   // C streams out
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < mn; e += stride) {
            float acc = W[e];
            for (int s = 1; s < splits; ++s)
                acc += W[s * mn + e];
            acc *= alpha;
            if (relu)
                acc = __builtin_fmaxf(acc, 0.0f);
            __builtin_nontemporal_store((half_t)acc, C + e);
        }
    }
}

hipError_t launch_reduce(const float *W, _Float16 *C, int64_t M, int64_t N, int splits, float alpha, int relu,
                         bool vec4, hipStream_t s)
{
    const int64_t mn = M * N;
    const int64_t items = vec4 ? mn / 4 : mn;
    // enough workgroups to keep every CU streaming, each thread a few items
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, 256 * 16));
    if (vec4)
        hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, W, C, mn, splits,
                           alpha, relu);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, W, C, mn,
                           splits, alpha, relu);
    return hipGetLastError();
}


hipError_t launch(int config, const KernelArgs &a, int va, int vb, bool trans_a, bool trans_b, int64_t grid,
                  hipStream_t s)
{
    if (trans_a && trans_b)
        return launch_tt(config, a, va, vb, grid, s);
    if (trans_a)
        return launch_tn(config, a, va, vb, grid, s);
    if (trans_b)
        return launch_nt(config, a, va, vb, grid, s);
    return launch_nn(config, a, va, vb, grid, s);
}

} // namespace gemm_f16_impl

// mfma_probe.hip -- measurement probe: sustained v_mfma_f32_32x32x16_f16
// throughput with no memory traffic, for operands of a chosen kind.
//
// The GEMM kernels are bound by the matrix cores.  Their nominal dense FP16
// peak (256 CUs x 2.4 GHz x 4096 flop/clk) assumes the top clock, but the
// clock the chip sustains under MFMA load depends on how much the operand
// bits toggle.  This probe runs the GEMM's own instruction mix (a 4 x 4 block
// of 32x32x16 MFMAs per wave, one wave per SIMD, 16 fp32 accumulator tiles)
// with nothing but register operands, so its throughput is the practical
// ceiling of the inner loop for that kind of data.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_f16_probe.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_probe_kernel(const half8 *__restrict__ operands, float *__restrict__ out, int iters)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    half8 x[2][4], y[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (MODE == GEMM_F16_PROBE_CONSTANT) {
                for (int e = 0; e < 8; ++e) {
                    x[s][i][e] = (_Float16)(0.001f * lane);
                    y[s][i][e] = (_Float16)(0.01f * e);
                }
            } else {
                // 2 x 8 distinct fragments per lane from the caller's random halves
                x[s][i] = operands[((s * 8 + i) * 64 + lane) % GEMM_F16_PROBE_OPERAND_VECTORS];
                y[s][i] = operands[((s * 8 + 4 + i) * 64 + lane) % GEMM_F16_PROBE_OPERAND_VECTORS];
            }
        }
    if (MODE == GEMM_F16_PROBE_RANDOM_FIXED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[1][i] = x[0][i];
            y[1][i] = y[0][i];
        }
    }
    float16v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = float16v{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x[s][j], y[s][i], acc[i][j], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sum += acc[i][j][v];
    out[t] = sum;
}

// The same work with v_mfma_f32_16x16x32_f16: per wave an 8 x 8 block of
// 16x16 accumulator tiles (the same 128 x 128 outputs), 8 + 8 fragments per
// 32-deep k step, two fragment sets alternating.
template <int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma16_probe_kernel(const half8 *__restrict__ operands, float *__restrict__ out, int iters)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    half8 x[2][8], y[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (MODE == GEMM_F16_PROBE_CONSTANT) {
                for (int e = 0; e < 8; ++e) {
                    x[s][i][e] = (_Float16)(0.001f * lane);
                    y[s][i][e] = (_Float16)(0.01f * e);
                }
            } else {
                x[s][i] = operands[((s * 16 + i) * 64 + lane) % GEMM_F16_PROBE_OPERAND_VECTORS];
                y[s][i] = operands[((s * 16 + 8 + i) * 64 + lane) % GEMM_F16_PROBE_OPERAND_VECTORS];
            }
        }
    if (MODE == GEMM_F16_PROBE_RANDOM_FIXED) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[1][i] = x[0][i];
            y[1][i] = y[0][i];
        }
    }
    float4v acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = float4v{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x[s][j], y[s][i], acc[i][j], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                sum += acc[i][j][v];
    out[t] = sum;
}

} // namespace

extern "C" int gemm_f16_probe_mfma(int mode, int iters, int64_t blocks, const void *operands, void *out,
                                   void *stream, double *flops)
{
    const int kind = mode % GEMM_F16_PROBE_MFMA16;
    if (iters < 0 || blocks <= 0 || blocks > 0x7fffffff || !out || mode < 0 ||
        mode >= 2 * GEMM_F16_PROBE_MFMA16 || (kind != GEMM_F16_PROBE_CONSTANT && !operands))
        return 1;
    hipStream_t s = (hipStream_t)stream;
    dim3 grid((unsigned)blocks), block(256);
    const bool m16 = mode >= GEMM_F16_PROBE_MFMA16;
    if (m16)
        mode -= GEMM_F16_PROBE_MFMA16;
    if (m16) {
        switch (mode) {
        case GEMM_F16_PROBE_CONSTANT:
            hipLaunchKernelGGL(mfma16_probe_kernel<GEMM_F16_PROBE_CONSTANT>, grid, block, 0, s,
                               (const half8 *)operands, (float *)out, iters);
            break;
        case GEMM_F16_PROBE_RANDOM_FIXED:
            hipLaunchKernelGGL(mfma16_probe_kernel<GEMM_F16_PROBE_RANDOM_FIXED>, grid, block, 0, s,
                               (const half8 *)operands, (float *)out, iters);
            break;
        case GEMM_F16_PROBE_RANDOM_CHANGING:
            hipLaunchKernelGGL(mfma16_probe_kernel<GEMM_F16_PROBE_RANDOM_CHANGING>, grid, block, 0, s,
                               (const half8 *)operands, (float *)out, iters);
            break;
        default:
            return 1;
        }
        if (hipGetLastError() != hipSuccess)
            return 2;
        if (flops)
            *flops = (double)blocks * 4.0 * (double)iters * 128.0 /* MFMAs */ * 16384.0;
        return 0;
    }
    switch (mode) {
    case GEMM_F16_PROBE_CONSTANT:
        hipLaunchKernelGGL(mfma_probe_kernel<GEMM_F16_PROBE_CONSTANT>, grid, block, 0, s, (const half8 *)operands,
                           (float *)out, iters);
        break;
    case GEMM_F16_PROBE_RANDOM_FIXED:
        hipLaunchKernelGGL(mfma_probe_kernel<GEMM_F16_PROBE_RANDOM_FIXED>, grid, block, 0, s,
                           (const half8 *)operands, (float *)out, iters);
        break;
    case GEMM_F16_PROBE_RANDOM_CHANGING:
        hipLaunchKernelGGL(mfma_probe_kernel<GEMM_F16_PROBE_RANDOM_CHANGING>, grid, block, 0, s,
                           (const half8 *)operands, (float *)out, iters);
        break;
    default:
        return 1;
    }
    if (hipGetLastError() != hipSuccess)
        return 2;
    if (flops)
        *flops = (double)blocks * 4.0 /* waves */ * (double)iters * 32.0 /* MFMAs */ * 32768.0;
    return 0;
}

// ---- lane-layout probe ---------------------------------------------------------
// One wave runs one MFMA on operands the caller lays out per lane and writes
// back every lane's accumulators, so that a test can check the lane layouts
// the GEMM kernels rely on (and that subnormal binary16 inputs are kept).
namespace {

typedef _Float16 half16v __attribute__((ext_vector_type(16)));

template <int INSTR>
__global__ void __launch_bounds__(64) mfma_layout_kernel(const half8 *__restrict__ src0,
                                                         const _Float16 *__restrict__ src1,
                                                         const int *__restrict__ index, float *__restrict__ out)
{
    const int lane = threadIdx.x;
    const half8 a = src0[lane];
    if constexpr (INSTR == GEMM_F16_PROBE_LAYOUT_32X32X16) {
        const half8 b = reinterpret_cast<const half8 *>(src1)[lane];
        const float16v d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, float16v{}, 0, 0, 0);
        for (int e = 0; e < 16; ++e)
            out[lane * 16 + e] = d[e];
    } else if constexpr (INSTR == GEMM_F16_PROBE_LAYOUT_16X16X32) {
        const half8 b = reinterpret_cast<const half8 *>(src1)[lane];
        const float4v d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, float4v{}, 0, 0, 0);
        for (int e = 0; e < 4; ++e)
            out[lane * 4 + e] = d[e];
    } else {
        const half16v b = reinterpret_cast<const half16v *>(src1)[lane];
        const float16v d = __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, float16v{}, index[lane], 0, 0);
        for (int e = 0; e < 16; ++e)
            out[lane * 16 + e] = d[e];
    }
}

}  // namespace

extern "C" int gemm_f16_probe_mfma_layout(int instr, const void *src0, const void *src1, const void *index,
                                          void *out, void *stream)
{
    if (!src0 || !src1 || !out || (instr == GEMM_F16_PROBE_LAYOUT_SMFMAC_32X32X32 && !index))
        return 1;
    hipStream_t s = (hipStream_t)stream;
    const half8 *a = (const half8 *)src0;
    const _Float16 *b = (const _Float16 *)src1;
    const int *idx = (const int *)index;
    float *o = (float *)out;
    switch (instr) {
    case GEMM_F16_PROBE_LAYOUT_32X32X16:
        hipLaunchKernelGGL(mfma_layout_kernel<GEMM_F16_PROBE_LAYOUT_32X32X16>, dim3(1), dim3(64), 0, s, a, b, idx, o);
        break;
    case GEMM_F16_PROBE_LAYOUT_16X16X32:
        hipLaunchKernelGGL(mfma_layout_kernel<GEMM_F16_PROBE_LAYOUT_16X16X32>, dim3(1), dim3(64), 0, s, a, b, idx, o);
        break;
    case GEMM_F16_PROBE_LAYOUT_SMFMAC_32X32X32:
        hipLaunchKernelGGL(mfma_layout_kernel<GEMM_F16_PROBE_LAYOUT_SMFMAC_32X32X32>, dim3(1), dim3(64), 0, s, a, b,
                           idx, o);
        break;
    default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

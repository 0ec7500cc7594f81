// gemm_f16_internal.h -- shared between the host API (gemm_f16_api.cpp) and
// the gfx950 kernels (gemm_f16_tile.h and the gemm_f16_*.hip files that
// instantiate it).  Not part of the public ABI.
#ifndef GEMM_F16_INTERNAL_H
#define GEMM_F16_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm_f16_impl {

// Kernel arguments, passed by value.  All dimensions fit in int32 (the public
// API limits M, N, K to 2^31 - 1 and K, N to 2^22).
struct KernelArgs {
    const _Float16 *A;   // M x K, row-major
    const _Float16 *B;   // K x N, row-major
    _Float16 *C;         // M x N, row-major
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;         // tile rows walked together by the tile remap
    int relu;            // 1: max(alpha acc, 0) before the fp16 conversion
    float alpha;         // the result block is scaled by alpha first (1: the plain product)
    int vec_c;           // 8: 16-byte stores of C are aligned (LDS-staged write-back);
                         // 4: 8-byte stores; 1: 2-byte stores
    int k_split;         // K elements per workgroup (a multiple of the tile depth); >= K unless split
    float *W;            // split-K: splits x M x N fp32 partial sums (written instead of C); else null
    const uint16_t *meta;  // sparse A: M x K/16 position words (A then holds the M x K/2 kept values)
};

// Static description of one compiled kernel configuration.
struct ConfigDesc {
    const char *name;
    int block_m, block_n, block_k;
    int stages;
    int waves;            // wave64s per workgroup (4: one per SIMD, 8: two)
    bool direct;          // operands move global -> LDS with buffer_load ... lds
    int min_vec;          // alignment of A's rows it needs, in elements: direct kernels (always
                          // 16-byte loads) 8 or 2, register-staged ones their narrowest vector
    int min_vec_b;        // ... of B's rows
    int layouts;          // layouts compiled, bit 2 trans_a + trans_b: 1 = A . B only, 15 = all four
    int occupancy;        // workgroups resident per CU (LDS and register limits)
    bool persistent;      // one resident workgroup per CU loops over the tiles
};

constexpr int kNumConfigs = 18;
extern const ConfigDesc kConfigs[kNumConfigs];

// Launch configuration `config` with `grid` workgroups on `s`.
// va / vb: elements per global load of A / B (8, 4, 2 or 1; direct configs
// load 8, or A 2 where the configuration's min_vec is 2; transposed layouts
// of register-staged configs 8 or 1).
// trans_a: A is stored K x M; trans_b: B is stored N x K.  Returns the
// launch status.
hipError_t launch(int config, const KernelArgs &a, int va, int vb, bool trans_a, bool trans_b, int64_t grid,
                  hipStream_t s);
// ... per layout: A . B, A . B^T, A^T . B, A^T . B^T (one source file each)
hipError_t launch_nn(int config, const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s);
hipError_t launch_nt(int config, const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s);
hipError_t launch_tn(int config, const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s);
hipError_t launch_tt(int config, const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s);

// 2:4 sparse A: compress M x K (K % 16 == 0) to vals (M x K/2) and meta
// (M x K/16 words); vec: A and vals 16-byte aligned.
hipError_t launch_sp_compress(const _Float16 *A, _Float16 *vals, uint16_t *meta, int64_t M, int64_t K, bool vec,
                              hipStream_t s);

// Sparse GEMM, configuration `config` of kSpConfigs (A = vals, a.meta set;
// trans_b: B stored N x K).
constexpr int kNumSpConfigs = 4;
extern const ConfigDesc kSpConfigs[kNumSpConfigs];
hipError_t launch_sparse(int config, const KernelArgs &a, bool trans_b, int64_t grid, hipStream_t s);

// Static split-K scratch (gemm_f16_split_static): kStaticScratchBytes of
// device memory per GPU.  static_scratch() returns the current device's copy
// (looked up once per device; no allocation).
constexpr int64_t kStaticScratchBytes = (int64_t)32 << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t static_scratch(void **ptr);

// Split-K reduction: C = rne16(epi(alpha (W[0] + ... + W[splits-1]))) over M x N
// elements (relu: 1 for the ReLU epilogue).  vec4: N % 4 == 0, C 8-byte and
// W 16-byte aligned.
hipError_t launch_reduce(const float *W, _Float16 *C, int64_t M, int64_t N, int splits, float alpha, int relu,
                         bool vec4, hipStream_t s);

} // namespace gemm_f16_impl

#endif

// plan_fuzz.cpp -- host-only driver for the C ABI's validation and planning,
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitized.py.  The HIP runtime calls and the kernel
// launchers are replaced by stubs that record what would have been
// launched, so every entry point runs to completion on a machine without a
// GPU; the checks are that nothing reads or writes out of bounds, no
// undefined behaviour occurs, invalid arguments never reach a launch, and
// every valid call launches exactly the plan's grid.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gemm_f16.h"
#include "gemm_f16_internal.h"

namespace {
int g_launches = 0;
int64_t g_last_grid = -1;
int g_reductions = 0;
alignas(256) unsigned char g_fake_scratch[256];
}  // namespace

extern "C" {
hipError_t hipGetDevice(int *device)
{
    *device = 0;
    return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *prop, int)
{
    memset(prop, 0, sizeof(*prop));
    strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
    prop->multiProcessorCount = 256;
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
}

namespace gemm_f16_impl {
hipError_t launch(int config, const KernelArgs &a, int, int, bool, bool, int64_t grid, hipStream_t)
{
    if (config < 0 || config >= kNumConfigs || grid <= 0 || a.M <= 0 || a.N <= 0)
        return hipErrorInvalidValue;
    ++g_launches;
    g_last_grid = grid;
    return hipSuccess;
}
hipError_t launch_reduce(const float *W, _Float16 *, int64_t M, int64_t N, int splits, float, int, bool, hipStream_t)
{
    if (!W || M <= 0 || N <= 0 || splits < 2)
        return hipErrorInvalidValue;
    ++g_reductions;
    return hipSuccess;
}
hipError_t launch_sparse(int config, const KernelArgs &, bool, int64_t grid, hipStream_t)
{
    if (config < 0 || config >= kNumSpConfigs || grid <= 0)
        return hipErrorInvalidValue;
    ++g_launches;
    g_last_grid = grid;
    return hipSuccess;
}
hipError_t launch_sp_compress(const _Float16 *, _Float16 *, uint16_t *, int64_t M, int64_t K, bool, hipStream_t)
{
    if (M <= 0 || K <= 0)
        return hipErrorInvalidValue;
    ++g_launches;
    return hipSuccess;
}
hipError_t static_scratch(void **ptr)
{
    *ptr = g_fake_scratch;
    return hipSuccess;
}
}  // namespace gemm_f16_impl

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t next()
{
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return g_rng;
}

// A dimension drawn from small, tile-edge, large and out-of-range values.
static int64_t dim()
{
    static const int64_t edges[] = {0, 1, 2, 7, 8, 15, 16, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 1024,
                                    4100, 8192, 28672, (int64_t)1 << 22, ((int64_t)1 << 22) + 1, (int64_t)1 << 24,
                                    ((int64_t)1 << 24) + 1, (int64_t)1 << 31, -1};
    if (next() % 4 == 0)
        return edges[next() % (sizeof(edges) / sizeof(edges[0]))];
    return (int64_t)(next() % 5000);
}

static int fails = 0;
#define CHECK(cond)                                                                 \
    do {                                                                            \
        if (!(cond)) {                                                              \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);     \
            ++fails;                                                                \
        }                                                                           \
    } while (0)

using gemm_f16_impl::kNumConfigs;
using gemm_f16_impl::kNumSpConfigs;

// Earlier planning calls and their results: replayed later, after other
// shapes have gone through the planner's per-thread cache, they must give
// the same status and the same plan.
struct Planned {
    int64_t M, N, K;
    int ta, tb;
    uintptr_t A, B, C;
    int config, splits;
    gemm_f16_status_t status;
    gemm_f16_plan_t plan;
};
static Planned g_history[512];

int main()
{
    const int iterations = 200000;
    for (int it = 0; it < iterations; ++it) {
        const int64_t M = dim(), N = dim(), K = dim();
        const int ta = (int)(next() % 2), tb = (int)(next() % 2);
        // aligned or deliberately misaligned stand-in addresses, far apart
        const uintptr_t base = (uintptr_t)1 << 40;
        const uintptr_t A = base + (next() % 8 == 0 ? 2 * (next() % 8) : 0);
        const uintptr_t B = base + ((uintptr_t)1 << 38) + (next() % 8 == 0 ? 2 * (next() % 8) : 0);
        const uintptr_t C = base + ((uintptr_t)2 << 38) + (next() % 8 == 0 ? 2 * (next() % 8) : 0);
        const int config = (int)(next() % (kNumConfigs + 2)) - 1;   // -1 .. kNumConfigs
        const int splits = (int)(next() % 70) - 2;                    // -2 .. 67
        gemm_f16_plan_t plan;
        memset(&plan, 0xAB, sizeof(plan));
        const gemm_f16_status_t ps = gemm_f16_plan_split(M, N, K, (const void *)A, ta, (const void *)B, tb,
                                                         (const void *)C, config, splits, &plan);
        if (ps == GEMM_F16_SUCCESS) {
            CHECK(plan.config >= 0 && plan.config < kNumConfigs);
            CHECK(plan.splits >= 1 && plan.splits <= GEMM_F16_MAX_SPLITS);
            CHECK(plan.grid >= 0 && plan.grid <= 0x7fffffff);
            CHECK(plan.lds_bytes > 0 && plan.lds_bytes <= 163840);
            CHECK(plan.workspace_bytes == (plan.splits > 1 ? (int64_t)plan.splits * M * N * 4 : 0));
            CHECK(plan.k_split >= 0);
            CHECK(!(ta && M > GEMM_F16_MAX_M_TRANS_A));
        }
        // planning again (from the cache) gives the same answer, now and later
        {
            gemm_f16_plan_t again;
            memset(&again, 0xCD, sizeof(again));
            CHECK(gemm_f16_plan_split(M, N, K, (const void *)A, ta, (const void *)B, tb, (const void *)C, config,
                                      splits, &again) == ps);
            if (ps == GEMM_F16_SUCCESS)
                CHECK(memcmp(&again, &plan, sizeof(plan)) == 0);
            Planned &h = g_history[it % 512];
            if (it >= 512 && next() % 4 == 0) {
                gemm_f16_plan_t old;
                memset(&old, 0xEF, sizeof(old));
                const gemm_f16_status_t s_old = gemm_f16_plan_split(
                    h.M, h.N, h.K, (const void *)h.A, h.ta, (const void *)h.B, h.tb, (const void *)h.C, h.config,
                    h.splits, &old);
                CHECK(s_old == h.status);
                if (s_old == GEMM_F16_SUCCESS)
                    CHECK(memcmp(&old, &h.plan, sizeof(old)) == 0);
            }
            h = Planned{M, N, K, ta, tb, A, B, C, config, splits, ps, plan};
        }
        // the workspace-free entry point: same validation, never a split
        const int before = g_launches, red_before = g_reductions;
        const gemm_f16_status_t st = gemm_f16_trans(M, N, K, (const void *)A, ta, (const void *)B, tb, (void *)C,
                                                    (int)(next() % 3), config, nullptr);
        if (st != GEMM_F16_SUCCESS || M == 0 || N == 0)
            CHECK(g_launches == before);
        if (st == GEMM_F16_SUCCESS && M > 0 && N > 0) {
            CHECK(g_launches == before + 1 && g_reductions == red_before);
            gemm_f16_plan_t p1;
            CHECK(gemm_f16_plan_trans(M, N, K, (const void *)A, ta, (const void *)B, tb, (const void *)C, config,
                                      &p1) == GEMM_F16_SUCCESS);
            CHECK(p1.splits == 1 && p1.workspace_bytes == 0 && p1.grid == g_last_grid);
        }
        // a split without a workspace never launches (status 7, or 1 where the
        // stand-in buffers of a huge shape overlap)
        const int b2 = g_launches;
        const gemm_f16_status_t s2 = gemm_f16_split(M, N, K, (const void *)A, ta, (const void *)B, tb, (void *)C,
                                                    0, config, splits, nullptr, 0, nullptr);
        if (ps == GEMM_F16_SUCCESS && plan.splits > 1 && M > 0 && N > 0)
            CHECK((s2 == GEMM_F16_ERROR_WORKSPACE || s2 == GEMM_F16_ERROR_INVALID_VALUE) && g_launches == b2);
        if (s2 != GEMM_F16_SUCCESS)
            CHECK(g_launches == b2);
        // the static-scratch entry point: refused above its limit, else split into the scratch
        const int b3 = g_launches, r3 = g_reductions;
        const gemm_f16_status_t s3 = gemm_f16_split_static(M, N, K, (const void *)A, ta, (const void *)B, tb,
                                                           (void *)C, 0, config, splits, nullptr);
        if (s3 != GEMM_F16_SUCCESS || M == 0 || N == 0)
            CHECK(g_launches == b3 && g_reductions == r3);
        if (ps == GEMM_F16_SUCCESS && M > 0 && N > 0 && plan.workspace_bytes > GEMM_F16_STATIC_WORKSPACE_BYTES)
            CHECK(s3 == GEMM_F16_ERROR_SCRATCH_LIMIT || s3 == GEMM_F16_ERROR_INVALID_VALUE);
        if (s3 == GEMM_F16_SUCCESS && M > 0 && N > 0) {
            CHECK(ps == GEMM_F16_SUCCESS && plan.workspace_bytes <= GEMM_F16_STATIC_WORKSPACE_BYTES);
            CHECK(g_launches == b3 + 1 && g_reductions == r3 + (plan.splits > 1 ? 1 : 0));
            CHECK(g_last_grid == plan.grid);
        }
        // sparse planning and validation
        gemm_f16_plan_t sp;
        const int spc = (int)(next() % (kNumSpConfigs + 2)) - 1;
        if (gemm_f16_plan_sp(M, N, K, (const void *)A, (const void *)C, (const void *)B, tb, (const void *)(C + 64),
                             spc, &sp) == GEMM_F16_SUCCESS) {
            CHECK(K % 16 == 0 && sp.grid >= 0 && sp.lds_bytes <= 163840);
        }
    }
    for (int s = -1; s <= 10; ++s)
        CHECK(gemm_f16_status_string((gemm_f16_status_t)s) != nullptr);
    printf("plan_fuzz: %d iterations, %d launches, %d reductions, %d failed checks\n", iterations, g_launches,
           g_reductions, fails);
    return fails == 0 ? 0 : 1;
}

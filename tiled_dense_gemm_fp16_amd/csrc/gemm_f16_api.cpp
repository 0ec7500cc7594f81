// gemm_f16_api.cpp -- the C ABI of the FP16 GEMM library: argument
// validation, kernel planning and launch.  Validation and planning make no
// HIP call, so they behave identically with or without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <math.h>

#include <algorithm>
#include <mutex>

#include "gemm_f16.h"
#include "gemm_f16_internal.h"

namespace gemm_f16_impl {

// occupancy: workgroups per CU as limited by LDS (160 KiB) and by registers
// (512 per lane per SIMD, VGPRs + AGPRs as the compiler reports them).
constexpr int kNN = 1, kNT = 2, kAllLayouts = 15;   // masks over bit 2 trans_a + trans_b
const ConfigDesc kConfigs[kNumConfigs] = {
    {"256x128x64_s3_direct_m16", 256, 128, 64, 3, 4, true, 8, 8, kAllLayouts, 1},
    {"256x128x64_s3_direct", 256, 128, 64, 3, 4, true, 8, 8, kAllLayouts, 1},
    {"128x128x64_s3_direct", 128, 128, 64, 3, 4, true, 8, 8, kAllLayouts, 1},
    {"128x128x32_s2_staged", 128, 128, 32, 2, 4, false, 1, 1, kAllLayouts, 2},
    {"64x64x64_s2_staged", 64, 64, 64, 2, 4, false, 1, 1, kAllLayouts, 5},
    {"256x256x64_s2_direct_w8n", 256, 256, 64, 2, 8, true, 8, 8, kAllLayouts, 1},
    {"256x128x64_s3_direct_m16_u", 256, 128, 64, 3, 4, true, 2, 2, kAllLayouts, 1},
    {"128x64x64_s4_direct_u", 128, 64, 64, 4, 4, true, 2, 2, kAllLayouts, 1},
    {"256x256x64_s2_direct_m16", 256, 256, 64, 2, 4, true, 8, 8, kAllLayouts, 1},
    {"256x256x64_s2_direct_m16_u", 256, 256, 64, 2, 4, true, 2, 2, kAllLayouts, 1},
    {"256x256x32_s4_direct_m16", 256, 256, 32, 4, 4, true, 8, 8, kAllLayouts, 1},
    {"256x256x64_s2_direct_m16_persistent", 256, 256, 64, 2, 4, true, 8, 8, kAllLayouts, 1, true},
    {"64x64x64_s4_direct", 64, 64, 64, 4, 4, true, 8, 8, kAllLayouts, 2},
    {"128x128x64_s4_direct_m16", 128, 128, 64, 4, 4, true, 8, 8, kAllLayouts, 1},
    {"128x64x64_s4_direct", 128, 64, 64, 4, 4, true, 8, 8, kAllLayouts, 1},
    {"128x128x64_s4_direct_m16_u", 128, 128, 64, 4, 4, true, 2, 2, kAllLayouts, 1},
    {"64x64x64_s4_direct_u", 64, 64, 64, 4, 4, true, 2, 2, kAllLayouts, 2},
    {"128x128x64_s2_staged", 128, 128, 64, 2, 4, false, 1, 1, kAllLayouts, 1},
};

// Sparse configurations (2:4 A): fields as above; every one takes A as
// compressed values + positions and B as K x N.
const ConfigDesc kSpConfigs[kNumSpConfigs] = {
    {"sp_256x256x64_s3_w8", 256, 256, 64, 3, 8, true, 8, 8, kNN | kNT, 1},
    {"sp_128x128x64_s3", 128, 128, 64, 3, 4, true, 8, 8, kNN | kNT, 1},
    {"sp_256x256x64_s3", 256, 256, 64, 3, 4, true, 8, 8, kNN | kNT, 1},
    {"sp_256x256x64_s3_spread", 256, 256, 64, 3, 4, true, 8, 8, kNN | kNT, 1},
};

namespace {

constexpr int kComputeUnits = 256;   // MI355X

// Tile rows walked together by the kernels' tile remap (L2 reuse); 4 measured
// best on MI355X for 8192-row problems (8: -4 %, 16: -10 %).
#ifndef GEMM_F16_GROUP_M
#define GEMM_F16_GROUP_M 4
#endif

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest vector width v in {8, 4, 2, 1} such that every row of a matrix
// with row pitch `pitch` elements starting at `p` is 2v-byte aligned.
int vec_width(const void *p, int64_t pitch)
{
    uintptr_t addr = (uintptr_t)p;
    for (int v = 8; v > 1; v /= 2)
        if (pitch % v == 0 && addr % (uintptr_t)(2 * v) == 0)
            return v;
    return 1;
}

bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes)
{
    if (a_bytes <= 0 || b_bytes <= 0)
        return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

gemm_f16_status_t validate(int64_t M, int64_t N, int64_t K, const void *A, bool trans_a, const void *B,
                           const void *C, bool check_c_overlap)
{
    if (M < 0 || N < 0 || K < 0)
        return GEMM_F16_ERROR_INVALID_VALUE;
    if (M > GEMM_F16_MAX_DIM || N > GEMM_F16_MAX_N || K > GEMM_F16_MAX_K)
        return GEMM_F16_ERROR_UNSUPPORTED_SIZE;
    // A stored K x M: one k slice of it (up to 64 rows of pitch M) is one
    // buffer range addressed with 32-bit byte offsets
    if (trans_a && M > GEMM_F16_MAX_M_TRANS_A)
        return GEMM_F16_ERROR_UNSUPPORTED_SIZE;
    const bool a_nonempty = M > 0 && K > 0, b_nonempty = K > 0 && N > 0, c_nonempty = M > 0 && N > 0;
    if ((a_nonempty && !A) || (b_nonempty && !B) || (c_nonempty && !C))
        return GEMM_F16_ERROR_INVALID_VALUE;
    if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 1u)
        return GEMM_F16_ERROR_MISALIGNED;
    if (check_c_overlap && c_nonempty &&
        (overlaps(C, 2 * M * N, A, a_nonempty ? 2 * M * K : 0) ||
         overlaps(C, 2 * M * N, B, b_nonempty ? 2 * K * N : 0)))
        return GEMM_F16_ERROR_INVALID_VALUE;
    return GEMM_F16_SUCCESS;
}

// Relative throughput a workgroup of each configuration sustains, from
// measurements on MI355X (8192^3 and 4096^3, random fp16 operands): larger
// tiles reuse each LDS byte more.  Used only to rank configurations.
double config_efficiency(int c)
{
    switch (c) {
    case 8: return 1.06;    // 256x256x64 direct, 4 waves, 16x16x32 MFMAs
    case 9: return 1.02;    // the same for rows only 4-byte aligned
    case 10: return 0.99;   // 256x256x32 direct, 4 stages, 16x16x32 MFMAs (ahead only for A given K x M)
    case 11: return 1.05;   // 256x256x64 16x16x32 tile, persistent over the tiles (within 1 % of 8)
    case 12: return 0.30;   // 64x64x64 direct, 4 stages (latency-bound; many small tiles)
    case 13: return 0.82;   // 128x128x64 direct, 4 stages, 16x16x32 MFMAs
    case 14: return 0.60;   // 128x64x64 direct, 4 stages
    case 15: return 0.80;   // 13 for rows only 4-byte aligned
    case 16: return 0.29;   // 12 for rows only 4-byte aligned

    case 5: return 1.00;    // 256x256x64 direct, 8 waves
    case 0: return 0.94;    // 256x128x64 direct, 3 stages, 16x16x32 MFMAs
    case 1: return 0.90;    // 256x128x64 direct
    case 6: return 0.92;    // 0 for rows only 4-byte aligned
    case 2: return 0.76;    // 128x128x64 direct
    case 7: return 0.58;    // 14 for rows only 4-byte aligned
    case 3: return 0.46;    // 128x128x32 register-staged, any alignment
    case 17: return 0.50;   // 128x128x64 register-staged, any alignment (twice the k step of 3)
    case 4: return 0.25;    // 64x64x64 register-staged, any alignment
    default: return 0.0;
    }
}

// Shape conditions beyond layout and alignment: the persistent tile loop
// needs an even number (>= 2) of k slices, no split, and 8-byte stores of C
// (vc >= 4: N % 4 == 0 and C 8-byte aligned).
bool shape_fits(int c, int64_t K, int vc, int splits)
{
    if (!kConfigs[c].persistent)
        return true;
    const int64_t nk = ceil_div(K, kConfigs[c].block_k);
    return nk >= 2 && nk % 2 == 0 && vc >= 4 && splits <= 1;
}

bool config_fits(int c, int va, int vb, bool ta, bool tb)
{
    if (!(kConfigs[c].layouts & (1 << (2 * (int)ta + (int)tb))))
        return false;
    return va >= kConfigs[c].min_vec && vb >= kConfigs[c].min_vec_b;
}

// Vector width a configuration loads an operand with (is_a: A, else B),
// given the widest the pitch allows.
int kernel_vec(const ConfigDesc &d, int v, bool transposed, bool is_a)
{
    if (d.direct)
        return is_a ? d.min_vec : d.min_vec_b;
    if (transposed)
        return v >= 8 ? 8 : 1;              // transposed layouts, narrow tiles: 16-byte vectors or elements
    return v;
}

// K splits: the K loop of every output tile divided into `splits` ranges of
// k_split elements (a multiple of the tile depth), each run by a workgroup of
// its own.  The fp32 partial sums go to a workspace and a second kernel adds
// them in split order and applies the epilogue.
struct Split {
    int splits;
    int64_t k_split;   // K when not split
};

Split split_geometry(const ConfigDesc &d, int64_t K, int requested)
{
    const int64_t nk = ceil_div(K, d.block_k);
    if (requested <= 1 || nk <= 1)
        return {1, K};
    const int64_t per = ceil_div(nk, requested);   // k tiles per split
    const int s = (int)ceil_div(nk, per);          // no empty split
    if (s <= 1)
        return {1, K};
    return {s, per * d.block_k};
}

// A workgroup's slice of the workspace (block_m rows of N fp32) must be
// addressable with the kernels' 31-bit buffer offsets.
bool split_addressable(const ConfigDesc &d, int64_t N) { return (int64_t)d.block_m * N * 4 < ((int64_t)1 << 31); }

void fill_plan(int c, int64_t M, int64_t N, int64_t K, int va, int vb, int vc, bool ta, bool tb, const Split &sp,
               gemm_f16_plan_t *p)
{
    const ConfigDesc &d = kConfigs[c];
    const bool tr = ta || tb;
    memset(p, 0, sizeof(*p));
    p->config = c;
    p->block_m = d.block_m;
    p->block_n = d.block_n;
    p->block_k = d.block_k;
    p->stages = d.stages;
    p->threads = 64 * d.waves;
    p->direct_lds = d.direct ? 1 : 0;
    p->vec_a = kernel_vec(d, va, tr, true);
    p->vec_b = kernel_vec(d, vb, tr, false);
    p->vec_c = vc;
    p->tiles_m = ceil_div(M, d.block_m);
    p->tiles_n = ceil_div(N, d.block_n);
    p->grid = d.persistent ? std::min<int64_t>(p->tiles_m * p->tiles_n, kComputeUnits)
                           : p->tiles_m * p->tiles_n * sp.splits;
    p->k_tiles = ceil_div(sp.splits > 1 ? sp.k_split : K, d.block_k);
    p->lds_bytes = gemm_f16_stage_bytes(d.block_m, d.block_n, d.block_k, d.stages);
    p->flops = 2.0 * (double)M * (double)N * (double)K;
    p->min_bytes = 2.0 * ((double)M * K + (double)K * N + (double)M * N);
    p->trans_a = ta ? 1 : 0;
    p->trans_b = tb ? 1 : 0;
    p->splits = sp.splits;
    p->k_split = sp.splits > 1 ? sp.k_split : K;
    p->workspace_bytes = sp.splits > 1 ? (int64_t)sp.splits * M * N * 4 : 0;
}

// ---- automatic choice ---------------------------------------------------------
// Measured table (tiled_dense_gemm_fp16_amd/tune.py): for swept shapes,
// layouts and pitch alignments, the configuration and split count that ran
// fastest, and the fastest configuration run unsplit (what a call without a
// workspace runs).
struct TunedEntry {
    int lm, ln, lk;        // log2 of the swept M, N, K
    int trans_a, trans_b;
    int aligned;           // rows of both operands 16-byte aligned (1), both at least 4-byte
                           // aligned (2), otherwise (0)
    int config;
    int splits;
    double tflops;
    int config_unsplit;
    double tflops_unsplit;
};
const TunedEntry kTuned[] = {
#include "gemm_f16_tuned.inc"
    {-1, -1, -1, -1, -1, -1, -1, 0, 0.0, -1, 0.0}   // end marker
};

// The tuned entry for the nearest swept shape (in log2 M, N, K) with the same
// layout and alignment, if one lies within a factor of two overall; null
// otherwise.
const TunedEntry *tuned_entry(int64_t M, int64_t N, int64_t K, bool ta, bool tb, int aligned, int va, int vb)
{
    const double lm = log2((double)(M > 0 ? M : 1)), ln = log2((double)(N > 0 ? N : 1));
    const double lk = log2((double)(K > 0 ? K : 1));
    const TunedEntry *best = nullptr;
    double best_d = 1.0 + 1e-9;
    for (const TunedEntry &e : kTuned) {
        if (e.config < 0)
            break;
        if (e.trans_a != (int)ta || e.trans_b != (int)tb || e.aligned != aligned)
            continue;
        const double d = sqrt((lm - e.lm) * (lm - e.lm) + (ln - e.ln) * (ln - e.ln) + (lk - e.lk) * (lk - e.lk));
        if (d < best_d && e.config < kNumConfigs && config_fits(e.config, va, vb, ta, tb) &&
            e.config_unsplit >= 0 && e.config_unsplit < kNumConfigs && config_fits(e.config_unsplit, va, vb, ta, tb)) {
            best = &e;
            best_d = d;
        }
    }
    return best;
}

// Time model used where the table has no nearby entry.  A workgroup's k tile
// costs its flops at the configuration's sustained per-CU rate divided among
// the workgroups sharing the CU (at most its occupancy); each workgroup adds
// a fixed cost (pipeline fill, write-back) of a few k tiles; workgroups run
// in rounds of CUs x occupancy.  Splitting adds the partial sums' round trip
// through HBM (written 4 bytes, read 4 bytes per split and element) and a
// second launch.
constexpr double kCuFlops = 5.0e12;        // fp16 flop/s of one CU at efficiency 1 (about 1290 TF/s chip-wide)
constexpr double kWgFixedTiles = 3.0;      // per-workgroup overhead in times of a 64-deep k tile
constexpr double kStreamBytes = 4.5e12;    // bytes/s of a streaming kernel
constexpr double kLaunchSeconds = 3e-6;    // one more kernel on the stream
constexpr int64_t kAutoWorkspaceMax = (int64_t)256 << 20;

double model_seconds(int c, int64_t M, int64_t N, int64_t K, const Split &sp)
{
    const ConfigDesc &d = kConfigs[c];
    const double units = (double)(ceil_div(M, d.block_m) * ceil_div(N, d.block_n)) * sp.splits;
    const double rounds = ceil(units / ((double)kComputeUnits * d.occupancy));
    const double sharing = std::min((double)d.occupancy, ceil(units / kComputeUnits));
    const double kt = (double)ceil_div(sp.splits > 1 ? sp.k_split : K, d.block_k);
    const double t_kt = 2.0 * d.block_m * d.block_n * d.block_k * sharing / (kCuFlops * config_efficiency(c));
    double t = rounds * (kt + kWgFixedTiles * 64.0 / d.block_k) * t_kt;
    if (sp.splits > 1)
        t += kLaunchSeconds + (8.0 * sp.splits + 2.0) * (double)M * (double)N / kStreamBytes;
    return t;
}

const int kSplitCandidates[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};

// Best split of configuration c by the model: every split keeps at least two
// k tiles, and more splits must win by 3 %.  requested > 0 fixes the count.
Split model_split(int c, int64_t M, int64_t N, int64_t K, int requested, double *seconds)
{
    const ConfigDesc &d = kConfigs[c];
    Split best = {1, K};
    double best_t = model_seconds(c, M, N, K, best);
    if (requested > 0) {
        best = split_geometry(d, K, requested);
        best_t = model_seconds(c, M, N, K, best);
    } else if (split_addressable(d, N)) {
        const int64_t nk = ceil_div(K, d.block_k);
        for (int s : kSplitCandidates) {
            if (s == 1 || 2 * s > nk)
                continue;
            const Split sp = split_geometry(d, K, s);
            if (sp.splits <= 1 || (int64_t)sp.splits * M * N * 4 > kAutoWorkspaceMax)
                continue;
            const double t = model_seconds(c, M, N, K, sp);
            if (t < best_t * 0.97) {
                best = sp;
                best_t = t;
            }
        }
    }
    if (seconds)
        *seconds = best_t;
    return best;
}

// The one-workgroup-per-tile configuration that computes the same tile as
// persistent configuration c (for shapes the persistent loop does not take).
int one_tile_twin(int c) { return kConfigs[c].persistent ? 8 : c; }

// Configuration (and split) with the lowest modelled time.
int choose_config(int64_t M, int64_t N, int64_t K, int va, int vb, int vc, bool ta, bool tb, int requested,
                  Split *split)
{
    int best = -1;
    double best_t = 0.0;
    for (int c = 0; c < kNumConfigs; ++c) {
        if (!config_fits(c, va, vb, ta, tb) || config_efficiency(c) <= 0.0)
            continue;
        if (kConfigs[c].persistent && (requested > 1 || !shape_fits(c, K, vc, 1)))
            continue;
        double t;
        const Split sp = model_split(c, M, N, K, kConfigs[c].persistent ? 1 : requested, &t);
        if (best < 0 || t < best_t * 0.999) {
            best = c;
            best_t = t;
            *split = sp;
        }
    }
    return best;
}

// The plan of a shape: the pointers matter only through the alignment of
// the rows they start (va, vb: A's and B's rows; vc: C's stores).
gemm_f16_status_t plan_for(int64_t M, int64_t N, int64_t K, bool ta, bool tb, int va, int vb, int vc, int config,
                           int splits, gemm_f16_plan_t *plan)
{
    int c = config;
    Split sp = {1, K};
    if (c == GEMM_F16_CONFIG_AUTO) {
        // alignment class of the table: both operands' rows 16-byte aligned
        // (1), both at least 4-byte aligned (2), otherwise (0); a class-2
        // shape with no class-2 entry near it takes the class-0 entries
        const int cls = (va == 8 && vb == 8) ? 1 : (va >= 2 && vb >= 2) ? 2 : 0;
        const TunedEntry *e = tuned_entry(M, N, K, ta, tb, cls, va, vb);
        if (!e && cls == 2)
            e = tuned_entry(M, N, K, ta, tb, 0, va, vb);
        if (e && splits == 1) {
            c = e->config_unsplit;
        } else if (e && (splits == GEMM_F16_SPLITS_AUTO || splits == e->splits)) {
            c = e->config;
            sp = split_geometry(kConfigs[c], K, e->splits);
            if (sp.splits > 1 && ((int64_t)sp.splits * M * N * 4 > kAutoWorkspaceMax ||
                                  !split_addressable(kConfigs[c], N))) {
                c = e->config_unsplit;
                sp = {1, K};
            }
        } else {
            c = choose_config(M, N, K, va, vb, vc, ta, tb, splits, &sp);
        }
        // a table entry may name the persistent loop for a nearby shape it does not take
        if (c >= 0 && !shape_fits(c, K, vc, sp.splits))
            c = one_tile_twin(c);
    } else if (config_fits(c, va, vb, ta, tb)) {
        if (kConfigs[c].persistent && splits > 1)
            return GEMM_F16_ERROR_INVALID_VALUE;   // the persistent loop has no split form
        sp = model_split(c, M, N, K, kConfigs[c].persistent ? 1 : splits, nullptr);
    }
    if (c < 0 || !config_fits(c, va, vb, ta, tb) || !shape_fits(c, K, vc, sp.splits))
        return GEMM_F16_ERROR_INVALID_VALUE;
    if (sp.splits > 1 && !split_addressable(kConfigs[c], N))
        return GEMM_F16_ERROR_UNSUPPORTED_SIZE;
    fill_plan(c, M, N, K, va, vb, vc, ta, tb, sp, plan);
    if (plan->grid > 0x7fffffff)
        return GEMM_F16_ERROR_UNSUPPORTED_SIZE;
    return GEMM_F16_SUCCESS;
}

// Repeated calls of one shape skip the table search (a few microseconds of
// host time per call): a small per-thread cache of plans, keyed by
// everything plan_for reads.
struct PlanKey {
    int64_t M, N, K;
    int ta, tb, va, vb, vc, config, splits;
    bool operator==(const PlanKey &o) const
    {
        return M == o.M && N == o.N && K == o.K && ta == o.ta && tb == o.tb && va == o.va && vb == o.vb &&
               vc == o.vc && config == o.config && splits == o.splits;
    }
};
struct PlanSlot {
    bool used;
    PlanKey key;
    gemm_f16_status_t status;
    gemm_f16_plan_t plan;
};
constexpr int kPlanCacheSlots = 64;
thread_local PlanSlot t_plans[kPlanCacheSlots];

gemm_f16_status_t make_plan(int64_t M, int64_t N, int64_t K, const void *A, bool ta, const void *B, bool tb,
                            const void *C, int config, int splits, gemm_f16_plan_t *plan)
{
    if (config != GEMM_F16_CONFIG_AUTO && (config < 0 || config >= kNumConfigs))
        return GEMM_F16_ERROR_INVALID_VALUE;
    if (splits < 0 || splits > GEMM_F16_MAX_SPLITS)
        return GEMM_F16_ERROR_INVALID_VALUE;
    // row pitches of the matrices as stored
    const int64_t lda = ta ? M : K, ldb = tb ? K : N;
    const int va = vec_width(A, lda), vb = vec_width(B, ldb);
    const int vc = (N % 8 == 0 && (uintptr_t)C % 16 == 0) ? 8 : (N % 4 == 0 && (uintptr_t)C % 8 == 0) ? 4 : 1;
    const PlanKey key = {M, N, K, (int)ta, (int)tb, va, vb, vc, config, splits};
    uint64_t h = (uint64_t)M * 0x9E3779B97F4A7C15ull ^ (uint64_t)N * 0xC2B2AE3D27D4EB4Full ^
                 (uint64_t)K * 0x165667B19E3779F9ull;
    h ^= (uint64_t)(((ta * 2 + tb) * 16 + va) * 16 + vb) * 0x27D4EB2F165667C5ull;
    h ^= (uint64_t)((vc * 64 + (config + 1)) * 64 + splits) * 0x94D049BB133111EBull;
    PlanSlot &slot = t_plans[(h >> 32) % kPlanCacheSlots];
    if (slot.used && slot.key == key) {
        *plan = slot.plan;
        return slot.status;
    }
    const gemm_f16_status_t st = plan_for(M, N, K, ta, tb, va, vb, vc, config, splits, plan);
    slot.used = true;
    slot.key = key;
    slot.status = st;
    slot.plan = *plan;
    return st;
}

// Per-device check that the device is gfx950, done once per device.
constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
int g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

gemm_f16_status_t check_device(int *device)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return GEMM_F16_ERROR_NO_DEVICE;
    if (dev >= kMaxDevices)
        return GEMM_F16_ERROR_UNSUPPORTED_DEVICE;
    *device = dev;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return GEMM_F16_ERROR_NO_DEVICE;
        g_dev_state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return g_dev_state[dev] == 1 ? GEMM_F16_SUCCESS : GEMM_F16_ERROR_UNSUPPORTED_DEVICE;
}

// Enqueue a planned call; W is the split-K workspace (plan->splits > 1).
gemm_f16_status_t launch_plan(const gemm_f16_plan_t &plan, int64_t M, int64_t N, int64_t K, const void *A,
                              bool ta, const void *B, bool tb, void *C, float alpha, int epilogue, void *W,
                              hipStream_t s)
{
    KernelArgs a;
    a.A = (const _Float16 *)A;
    a.B = (const _Float16 *)B;
    a.C = (_Float16 *)C;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)plan.tiles_m;
    a.tiles_n = (int)plan.tiles_n;
    a.group_m = GEMM_F16_GROUP_M;
    a.relu = epilogue == GEMM_F16_EPILOGUE_RELU ? 1 : 0;
    a.alpha = alpha;
    a.vec_c = plan.vec_c;
    a.k_split = (int)plan.k_split;
    a.W = plan.splits > 1 ? (float *)W : nullptr;
    a.meta = nullptr;
    hipError_t e = launch(plan.config, a, plan.vec_a, plan.vec_b, ta, tb, plan.grid, s);
    if (e == hipSuccess && plan.splits > 1)
        e = launch_reduce((const float *)W, (_Float16 *)C, M, N, plan.splits, alpha, a.relu, plan.vec_c >= 4, s);
    return e == hipSuccess ? GEMM_F16_SUCCESS : GEMM_F16_ERROR_LAUNCH_FAILED;
}

// workspace: the caller's buffer (workspace_bytes long), or null: a plan
// that splits then fails with GEMM_F16_ERROR_WORKSPACE before any HIP call.
// The library allocates no device memory and never waits on the stream.
gemm_f16_status_t run(int64_t M, int64_t N, int64_t K, const void *A, bool ta, const void *B, bool tb, void *C,
                      float alpha, int epilogue, int config, int splits, void *workspace, int64_t workspace_bytes,
                      void *stream)
{
    gemm_f16_status_t st = validate(M, N, K, A, ta, B, C, true);
    if (st != GEMM_F16_SUCCESS)
        return st;
    if (epilogue != GEMM_F16_EPILOGUE_NONE && epilogue != GEMM_F16_EPILOGUE_RELU)
        return GEMM_F16_ERROR_INVALID_VALUE;
    if (workspace_bytes < 0 || (!workspace && workspace_bytes != 0))
        return GEMM_F16_ERROR_INVALID_VALUE;
    gemm_f16_plan_t plan;
    st = make_plan(M, N, K, A, ta, B, tb, C, config, splits, &plan);
    if (st != GEMM_F16_SUCCESS)
        return st;
    if (M == 0 || N == 0)
        return GEMM_F16_SUCCESS;
    if (plan.splits > 1) {
        if (!workspace)
            return GEMM_F16_ERROR_WORKSPACE;
        if ((uintptr_t)workspace % 16 != 0)
            return GEMM_F16_ERROR_MISALIGNED;
        if (workspace_bytes < plan.workspace_bytes)
            return GEMM_F16_ERROR_WORKSPACE;
        if (overlaps(workspace, plan.workspace_bytes, A, 2 * M * K) ||
            overlaps(workspace, plan.workspace_bytes, B, 2 * K * N) ||
            overlaps(workspace, plan.workspace_bytes, C, 2 * M * N))
            return GEMM_F16_ERROR_INVALID_VALUE;
    }
    int dev = -1;
    st = check_device(&dev);
    if (st != GEMM_F16_SUCCESS)
        return st;
    return launch_plan(plan, M, N, K, A, ta, B, tb, C, alpha, epilogue, workspace, (hipStream_t)stream);
}

// ---- 2:4 structured-sparse A -------------------------------------------------

gemm_f16_status_t validate_sp(int64_t M, int64_t N, int64_t K, const void *vals, const void *meta, const void *B,
                              bool trans_b, const void *C, bool check_c_overlap)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0)
        return GEMM_F16_ERROR_INVALID_VALUE;
    if (M > GEMM_F16_MAX_DIM || N > GEMM_F16_MAX_N || K > GEMM_F16_MAX_K)
        return GEMM_F16_ERROR_UNSUPPORTED_SIZE;
    const bool a_nonempty = M > 0 && K > 0, b_nonempty = K > 0 && N > 0, c_nonempty = M > 0 && N > 0;
    if ((a_nonempty && (!vals || !meta)) || (b_nonempty && !B) || (c_nonempty && !C))
        return GEMM_F16_ERROR_INVALID_VALUE;
    // 16-byte loads of the compressed values and of B: rows of K/2 (K % 16 == 0)
    // and of N (or, B given N x K, K) halves; the position words and C need 2 bytes
    if ((a_nonempty && (uintptr_t)vals % 16) || (b_nonempty && ((uintptr_t)B % 16 || (!trans_b && N % 8))) ||
        ((uintptr_t)meta | (uintptr_t)C) & 1u)
        return GEMM_F16_ERROR_MISALIGNED;
    if (check_c_overlap && c_nonempty &&
        (overlaps(C, 2 * M * N, vals, a_nonempty ? M * K : 0) ||
         overlaps(C, 2 * M * N, meta, a_nonempty ? M * K / 8 : 0) ||
         overlaps(C, 2 * M * N, B, b_nonempty ? 2 * K * N : 0)))
        return GEMM_F16_ERROR_INVALID_VALUE;
    return GEMM_F16_SUCCESS;
}

// Relative per-workgroup throughput of the sparse tiles (ranking only;
// measured at 8192^3 and 4096^3 on MI355X, A's position words stored by
// slices): the sparse MFMA does a 64-deep slice in half the dense time, so
// the tile is bound by issuing its loads, which the spread tile issues half
// per k step (0.564 ms at 8192^3 against 0.624 with all at the step start).
double sp_config_efficiency(int c)
{
    switch (c) {
    case 3: return 1.10;   // 256x256x64, 4 waves, loads spread over the two k steps
    case 0: return 1.09;   // 256x256x64, 8 waves
    case 2: return 1.00;   // 256x256x64, 4 waves
    case 1: return 0.60;   // 128x128x64, 4 waves
    default: return 0.0;
    }
}

gemm_f16_status_t make_plan_sp(int64_t M, int64_t N, int64_t K, int config, gemm_f16_plan_t *p)
{
    if (config != GEMM_F16_CONFIG_AUTO && (config < 0 || config >= kNumSpConfigs))
        return GEMM_F16_ERROR_INVALID_VALUE;
    int c = config;
    if (c == GEMM_F16_CONFIG_AUTO) {
        double best_t = 0.0;
        for (int i = 0; i < kNumSpConfigs; ++i) {
            if (sp_config_efficiency(i) <= 0.0)
                continue;
            const ConfigDesc &d = kSpConfigs[i];
            const double rounds = (double)ceil_div(ceil_div(M, d.block_m) * ceil_div(N, d.block_n), kComputeUnits);
            const double t = rounds * (double)d.block_m * (double)d.block_n / sp_config_efficiency(i);
            if (c < 0 || t < best_t * 0.999) {
                c = i;
                best_t = t;
            }
        }
    }
    const ConfigDesc &d = kSpConfigs[c];
    memset(p, 0, sizeof(*p));
    p->config = c;
    p->block_m = d.block_m;
    p->block_n = d.block_n;
    p->block_k = d.block_k;
    p->stages = d.stages;
    p->threads = 64 * d.waves;
    p->direct_lds = 1;
    p->vec_a = 8;
    p->vec_b = 8;
    p->vec_c = 1;
    p->tiles_m = ceil_div(M, d.block_m);
    p->tiles_n = ceil_div(N, d.block_n);
    p->grid = p->tiles_m * p->tiles_n;
    p->k_tiles = ceil_div(K, d.block_k);
    // LDS: the compressed A tile (bK/2 columns), the B tile and A's position
    // words (two dwords per row of a 64-deep slice) per stage
    p->lds_bytes = gemm_f16_stage_bytes(d.block_m, 0, d.block_k / 2, d.stages) +
                   gemm_f16_stage_bytes(0, d.block_n, d.block_k, d.stages) + (int64_t)d.stages * 8 * d.block_m;
    p->flops = (double)M * (double)N * (double)K;   // 2 M N (K/2): products of kept values
    p->min_bytes = (double)M * K + (double)M * K / 8 + 2.0 * ((double)K * N + (double)M * N);
    p->splits = 1;
    p->k_split = K;
    if (p->grid > 0x7fffffff)
        return GEMM_F16_ERROR_UNSUPPORTED_SIZE;
    return GEMM_F16_SUCCESS;
}

} // namespace
} // namespace gemm_f16_impl

using namespace gemm_f16_impl;

extern "C" {

gemm_f16_status_t gemm_f16(int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C,
                           int epilogue, void *stream)
{
    return run(M, N, K, A, false, B, false, C, 1.0f, epilogue, GEMM_F16_CONFIG_AUTO, 1, nullptr, 0, stream);
}

gemm_f16_status_t gemm_f16_ex(int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C,
                              int epilogue, int config, void *stream)
{
    return run(M, N, K, A, false, B, false, C, 1.0f, epilogue, config, 1, nullptr, 0, stream);
}

gemm_f16_status_t gemm_f16_trans(int64_t M, int64_t N, int64_t K, const void *A, int trans_a, const void *B,
                                 int trans_b, void *C, int epilogue, int config, void *stream)
{
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
        return GEMM_F16_ERROR_INVALID_VALUE;
    return run(M, N, K, A, trans_a != 0, B, trans_b != 0, C, 1.0f, epilogue, config, 1, nullptr, 0, stream);
}

gemm_f16_status_t gemm_f16_scaled(int64_t M, int64_t N, int64_t K, const void *A, int trans_a, const void *B,
                                  int trans_b, void *C, float alpha, int epilogue, int config, void *stream)
{
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
        return GEMM_F16_ERROR_INVALID_VALUE;
    return run(M, N, K, A, trans_a != 0, B, trans_b != 0, C, alpha, epilogue, config, 1, nullptr, 0, stream);
}

gemm_f16_status_t gemm_f16_split_scaled(int64_t M, int64_t N, int64_t K, const void *A, int trans_a,
                                        const void *B, int trans_b, void *C, float alpha, int epilogue, int config,
                                        int splits, void *workspace, int64_t workspace_bytes, void *stream)
{
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
        return GEMM_F16_ERROR_INVALID_VALUE;
    return run(M, N, K, A, trans_a != 0, B, trans_b != 0, C, alpha, epilogue, config, splits, workspace,
               workspace_bytes, stream);
}

gemm_f16_status_t gemm_f16_split(int64_t M, int64_t N, int64_t K, const void *A, int trans_a, const void *B,
                                 int trans_b, void *C, int epilogue, int config, int splits, void *workspace,
                                 int64_t workspace_bytes, void *stream)
{
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
        return GEMM_F16_ERROR_INVALID_VALUE;
    return run(M, N, K, A, trans_a != 0, B, trans_b != 0, C, 1.0f, epilogue, config, splits, workspace,
               workspace_bytes, stream);
}

gemm_f16_status_t gemm_f16_split_static(int64_t M, int64_t N, int64_t K, const void *A, int trans_a,
                                        const void *B, int trans_b, void *C, int epilogue, int config, int splits,
                                        void *stream)
{
    static_assert(GEMM_F16_STATIC_WORKSPACE_BYTES == kStaticScratchBytes, "header and library agree");
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
        return GEMM_F16_ERROR_INVALID_VALUE;
    // validate and plan first (no HIP call), so that an oversized split is
    // refused before the scratch is looked up
    gemm_f16_status_t st = validate(M, N, K, A, trans_a != 0, B, C, true);
    if (st != GEMM_F16_SUCCESS)
        return st;
    gemm_f16_plan_t plan;
    st = make_plan(M, N, K, A, trans_a != 0, B, trans_b != 0, C, config, splits, &plan);
    if (st != GEMM_F16_SUCCESS)
        return st;
    if (plan.workspace_bytes > kStaticScratchBytes)
        return GEMM_F16_ERROR_SCRATCH_LIMIT;
    void *scratch = nullptr;
    if (plan.splits > 1 && M > 0 && N > 0) {
        int dev = -1;
        st = check_device(&dev);
        if (st != GEMM_F16_SUCCESS)
            return st;
        if (static_scratch(&scratch) != hipSuccess)
            return GEMM_F16_ERROR_RUNTIME;
    }
    return run(M, N, K, A, trans_a != 0, B, trans_b != 0, C, 1.0f, epilogue, config, splits, scratch,
               scratch ? kStaticScratchBytes : 0, stream);
}

gemm_f16_status_t gemm_f16_plan(int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                                int config, gemm_f16_plan_t *plan)
{
    return gemm_f16_plan_trans(M, N, K, A, 0, B, 0, C, config, plan);
}

gemm_f16_status_t gemm_f16_plan_trans(int64_t M, int64_t N, int64_t K, const void *A, int trans_a,
                                      const void *B, int trans_b, const void *C, int config,
                                      gemm_f16_plan_t *plan)
{
    return gemm_f16_plan_split(M, N, K, A, trans_a, B, trans_b, C, config, 1, plan);
}

gemm_f16_status_t gemm_f16_plan_split(int64_t M, int64_t N, int64_t K, const void *A, int trans_a,
                                      const void *B, int trans_b, const void *C, int config, int splits,
                                      gemm_f16_plan_t *plan)
{
    if (!plan || (trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
        return GEMM_F16_ERROR_INVALID_VALUE;
    gemm_f16_status_t st = validate(M, N, K, A, trans_a != 0, B, C, false);
    if (st != GEMM_F16_SUCCESS)
        return st;
    return make_plan(M, N, K, A, trans_a != 0, B, trans_b != 0, C, config, splits, plan);
}

gemm_f16_status_t gemm_f16_sp_compress(int64_t M, int64_t K, const void *A, void *vals, void *meta, void *stream)
{
    if (M < 0 || K < 0 || K % 16 != 0)
        return GEMM_F16_ERROR_INVALID_VALUE;
    if (M > GEMM_F16_MAX_DIM || K > GEMM_F16_MAX_K)
        return GEMM_F16_ERROR_UNSUPPORTED_SIZE;
    if (M == 0 || K == 0)
        return GEMM_F16_SUCCESS;
    if (!A || !vals || !meta)
        return GEMM_F16_ERROR_INVALID_VALUE;
    if (((uintptr_t)A | (uintptr_t)vals | (uintptr_t)meta) & 1u)
        return GEMM_F16_ERROR_MISALIGNED;
    if (overlaps(vals, M * K, A, 2 * M * K) || overlaps(meta, M * K / 8, A, 2 * M * K) ||
        overlaps(meta, M * K / 8, vals, M * K))
        return GEMM_F16_ERROR_INVALID_VALUE;
    int dev = -1;
    gemm_f16_status_t st = check_device(&dev);
    if (st != GEMM_F16_SUCCESS)
        return st;
    const bool vec = (uintptr_t)A % 16 == 0 && (uintptr_t)vals % 16 == 0;
    hipError_t e = launch_sp_compress((const _Float16 *)A, (_Float16 *)vals, (uint16_t *)meta, M, K, vec,
                                      (hipStream_t)stream);
    return e == hipSuccess ? GEMM_F16_SUCCESS : GEMM_F16_ERROR_LAUNCH_FAILED;
}

gemm_f16_status_t gemm_f16_plan_sp(int64_t M, int64_t N, int64_t K, const void *vals, const void *meta,
                                   const void *B, int trans_b, const void *C, int config, gemm_f16_plan_t *plan)
{
    if (!plan || (trans_b != 0 && trans_b != 1))
        return GEMM_F16_ERROR_INVALID_VALUE;
    gemm_f16_status_t st = validate_sp(M, N, K, vals, meta, B, trans_b != 0, C, false);
    if (st != GEMM_F16_SUCCESS)
        return st;
    st = make_plan_sp(M, N, K, config, plan);
    plan->trans_b = trans_b;
    return st;
}

gemm_f16_status_t gemm_f16_sp(int64_t M, int64_t N, int64_t K, const void *vals, const void *meta, const void *B,
                              int trans_b, void *C, int epilogue, int config, void *stream)
{
    if (trans_b != 0 && trans_b != 1)
        return GEMM_F16_ERROR_INVALID_VALUE;
    gemm_f16_status_t st = validate_sp(M, N, K, vals, meta, B, trans_b != 0, C, true);
    if (st != GEMM_F16_SUCCESS)
        return st;
    if (epilogue != GEMM_F16_EPILOGUE_NONE && epilogue != GEMM_F16_EPILOGUE_RELU)
        return GEMM_F16_ERROR_INVALID_VALUE;
    gemm_f16_plan_t plan;
    st = make_plan_sp(M, N, K, config, &plan);
    if (st != GEMM_F16_SUCCESS)
        return st;
    if (M == 0 || N == 0)
        return GEMM_F16_SUCCESS;
    int dev = -1;
    st = check_device(&dev);
    if (st != GEMM_F16_SUCCESS)
        return st;
    KernelArgs a;
    a.A = (const _Float16 *)vals;
    a.B = (const _Float16 *)B;
    a.C = (_Float16 *)C;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)plan.tiles_m;
    a.tiles_n = (int)plan.tiles_n;
    a.group_m = GEMM_F16_GROUP_M;
    a.relu = epilogue == GEMM_F16_EPILOGUE_RELU ? 1 : 0;
    a.alpha = 1.0f;
    a.vec_c = (N % 8 == 0 && (uintptr_t)C % 16 == 0) ? 8 : 1;   // 8: the LDS-staged epilogue
    a.k_split = (int)K;
    a.W = nullptr;
    a.meta = (const uint16_t *)meta;
    hipError_t e = launch_sparse(plan.config, a, trans_b != 0, plan.grid, (hipStream_t)stream);
    return e == hipSuccess ? GEMM_F16_SUCCESS : GEMM_F16_ERROR_LAUNCH_FAILED;
}

int gemm_f16_sp_num_configs(void) { return kNumSpConfigs; }

const char *gemm_f16_sp_config_name(int config)
{
    if (config < 0 || config >= kNumSpConfigs)
        return nullptr;
    return kSpConfigs[config].name;
}

int gemm_f16_num_configs(void) { return kNumConfigs; }

const char *gemm_f16_config_name(int config)
{
    if (config < 0 || config >= kNumConfigs)
        return nullptr;
    return kConfigs[config].name;
}

int64_t gemm_f16_stage_bytes(int64_t block_m, int64_t block_n, int64_t block_k, int64_t stages)
{
    if (block_m < 0 || block_n < 0 || block_k < 0 || stages < 0)
        return -1;
    return stages * 2 * block_k * (block_m + block_n);
}

const char *gemm_f16_status_string(gemm_f16_status_t status)
{
    // read as an integer: C callers may pass any int, which need not be a
    // value of the enumeration
    int code;
    memcpy(&code, &status, sizeof(code));
    switch (code) {
    case GEMM_F16_SUCCESS: return "success";
    case GEMM_F16_ERROR_INVALID_VALUE: return "invalid value";
    case GEMM_F16_ERROR_MISALIGNED: return "pointer not aligned";
    case GEMM_F16_ERROR_NO_DEVICE: return "no HIP device";
    case GEMM_F16_ERROR_UNSUPPORTED_DEVICE: return "device is not gfx950";
    case GEMM_F16_ERROR_LAUNCH_FAILED: return "kernel launch failed";
    case GEMM_F16_ERROR_UNSUPPORTED_SIZE: return "size beyond the library's limits";
    case GEMM_F16_ERROR_WORKSPACE: return "split-K workspace missing or too small";
    case GEMM_F16_ERROR_RUNTIME: return "HIP runtime call failed";
    case GEMM_F16_ERROR_SCRATCH_LIMIT: return "split needs more than the static split-K scratch holds";
    }
    return "unknown status";
}

} // extern "C"

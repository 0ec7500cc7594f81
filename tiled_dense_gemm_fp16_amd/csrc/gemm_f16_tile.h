// gemm_f16_tile.h -- the gfx950 tile kernel of the FP16 GEMM C = epi(A . B),
// a template instantiated per layout in gemm_f16_{nn,nt,tn,tt,sparse}.hip.
//
// One workgroup computes one bM x bN output tile, as in the tile program of
// "TileLang：比 Triton 低一层的 tile 语言" (section "第一个 kernel：GEMM"):
// an fp32 accumulator fragment held in registers, a K loop over bK-deep
// slices of A and B staged through a multi-stage shared-memory (LDS) ring so
// that the loads of later slices overlap the math on the current one
// (section "练习", exercises 1-2, on stage counts and their memory cost), and
// a final copy that applies the optional ReLU ("TileLang：让GPU编程像Python一样
// 简单的高性能计算新范式", section "并行计算的优雅表达") and rounds to fp16
// ("5分钟上手TileLang：GPU内核开发指南", section "避坑与调参").
//
// What is CDNA4-specific (the pages' Hopper design -- TMA, wgmma, mbarrier
// producer/consumer warpgroups -- does not exist here):
//  * 256 threads = 4 wave64s in a WM x WN grid; each wave owns a
//    (bM/WM) x (bN/WN) sub-tile made of 32x32 blocks computed with
//    v_mfma_f32_32x32x16_f16 into fp32 accumulators.
//  * The MFMA computes the transposed tile C^T = B^T . A^T: its first operand
//    is a 32(n) x 16(k) slice of B^T and its second a 16(k) x 32(m) slice of
//    A^T, so every lane ends up holding four consecutive n of one output row
//    and writes them with one 8-byte store.
//  * Each operand is staged in LDS the way it lies in memory.  An operand
//    whose rows run along k (A as M x K; B given transposed as N x K) gives
//    its fragments with ds_read_b128; one whose rows run along m or n (B as
//    K x N; A given transposed as K x M) with gfx950's transposing
//    ds_read_b64_tr_b16, which hands each lane four k values of one column.
//    LDS tiles are XOR-swizzled in 16-byte chunks (no padding) so that the
//    reads spread over the LDS banks.
//  * "direct" kernels move operands global -> LDS with 16-byte
//    buffer_load ... lds (no registers, no LDS-write instructions); "staged"
//    kernels load through registers with 16/8/4/2-byte vectors and serve
//    pitches or pointers that are not 16-byte aligned.
//  * All global accesses are raw buffer instructions whose descriptor bounds
//    the matrix panel the workgroup touches: out-of-range rows read as zero
//    and out-of-range stores are dropped by the hardware; columns past the
//    row end are masked explicitly (they would otherwise wrap to the next row).
//  * Workgroup ids are remapped so that each XCD (own L2) receives a
//    contiguous range of tiles, walked in groups of GROUP_M tile rows.
#ifndef GEMM_F16_TILE_H
#define GEMM_F16_TILE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gemm_f16_internal.h"

// Build-time switches kept for tuning sweeps (defaults are the measured best):
// GEMM_F16_SNAKE 1 walks each row of MFMA blocks in alternating direction so
// that consecutive MFMAs share an operand (fewer operand bits toggle);
// GEMM_F16_NO_XCD_REMAP 1 disables the XCD-aware tile order.
#ifndef GEMM_F16_SNAKE
#define GEMM_F16_SNAKE 1
#endif
#ifndef GEMM_F16_NO_XCD_REMAP
#define GEMM_F16_NO_XCD_REMAP 0
#endif
// Placement of the k step's other instructions among its MFMAs: after every
// READ_EVERY-th MFMA come READS_PER_MFMA LDS fragment reads, and after every
// VMEM_EVERY-th MFMA one direct tile load.  32x32x16 tiles: two reads after
// every MFMA, a load after every MFMA (two reads: +4 % on 128x128 tiles over
// one).  16x16x32 tiles (M16_*): one read and one load after every second
// MFMA, measured +3 % over the 32x32 placement on 8192^3 in all four
// layouts (one read per MFMA: +1.5 %; loads every third MFMA: the same).
#ifndef GEMM_F16_READS_PER_MFMA
#define GEMM_F16_READS_PER_MFMA 2
#endif
#ifndef GEMM_F16_READ_EVERY
#define GEMM_F16_READ_EVERY 1
#endif
#ifndef GEMM_F16_VMEM_EVERY
#define GEMM_F16_VMEM_EVERY 1
#endif
#ifndef GEMM_F16_M16_READS_PER_MFMA
#define GEMM_F16_M16_READS_PER_MFMA 1
#endif
#ifndef GEMM_F16_M16_READ_EVERY
#define GEMM_F16_M16_READ_EVERY 2
#endif
#ifndef GEMM_F16_M16_VMEM_EVERY
#define GEMM_F16_M16_VMEM_EVERY 2
#endif
// parts the 16x16x32 tile's loads of a slice are issued in (one per k step)
#ifndef GEMM_F16_M16_SPREAD
#define GEMM_F16_M16_SPREAD 2
#endif

namespace gemm_f16_impl {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))
// Cache policy of the stores of C: non-temporal (the NT bit, 2).  C is
// written once and not read back by the kernel; streamed, it no longer
// displaces the operands' lines in the L2s and the Infinity Cache, whose
// re-reads feed the other tiles (8192^3: +4 %, 1411 -> 1472 TFLOP/s
// interleaved; the operands' loads with the NT bit lost 10-35 %).
#ifndef GEMM_F16_C_CPOL
#define GEMM_F16_C_CPOL 2
#endif

// Descriptor word 3 for gfx9-family raw buffers (untyped, 32-bit dwords).
constexpr int kBufferFlags = 0x00020000;
// Bit 31 set in a voffset puts it at or beyond every descriptor's
// num_records (panels never exceed 2 GiB): reads give 0, writes are dropped.
// It is OR-ed in arithmetically so that the compiler keeps one straight-line
// instruction instead of branching around each access.
__device__ __forceinline__ uint32_t oob_unless(bool ok) { return (uint32_t)(!ok) << 31; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kBufferFlags);
}

// s_waitcnt vmcnt(n) leaving expcnt and lgkmcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt vmcnt(n) lgkmcnt(0): global loads down to n outstanding and every
// LDS access of this wave complete.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// s_waitcnt lgkmcnt(0): every LDS access of this wave complete.
__device__ __forceinline__ void wait_lgkm0()
{
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
}

// ---- LDS swizzles ---------------------------------------------------------
// gfx950 LDS as measured: 64 banks of 4 bytes (a 256-byte window).  A
// ds_read_b128 is served 16 lanes per pass and is conflict-free when those 16
// lanes hit 16 different 16-byte slots of the window; 8-byte reads (plain or
// transposing) are served 32 lanes per pass and are conflict-free when the
// 32 lanes cover the window exactly.  Tiles are stored unpadded and the
// 16-byte chunk index of each row is XOR-ed with a row-dependent value.
//
// A tile: rows of CHUNKS 16-byte chunks.  A fragment read takes one chunk from
// each of 16 consecutive rows per pass; with W = 16 / CHUNKS rows per window
// (rows of 256 bytes or more: W = 1) rows r and r + W must differ in the XOR.
template <int CHUNKS>
__device__ __forceinline__ int swz_a(int row)
{
    if constexpr (CHUNKS >= 16)
        return row & 15;
    else if constexpr (CHUNKS == 8)
        return (row >> 1) & 7;
    else if constexpr (CHUNKS == 4)
        return (row >> 2) & 3;
    else if constexpr (CHUNKS == 2)
        return (row >> 3) & 1;
    else
        return 0;
}

// B tile: rows of CHUNKS 16-byte chunks.  Each 32-lane half of a transposing
// fragment read takes four 64-byte pieces (chunks 4q .. 4q+3) from four
// consecutive rows; XOR-ing the chunk index with a multiple of 4 moves the
// rows' pieces to different quarters of the window.
template <int CHUNKS>
__device__ __forceinline__ int swz_b(int row)
{
    if constexpr (CHUNKS >= 16)
        return 4 * (row & 3);              // one row spans >= 1 window
    else if constexpr (CHUNKS == 8)
        return 4 * ((row >> 1) & 1);       // two rows per window
    else
        return 0;                          // four rows per window already disjoint
}

// B-type tile read as 16x16x32 fragments: a pass reads rows k..k+3 and
// k+8..k+11, 32 bytes each; 4 (row & 3) chunks apart (64 bytes) as swz_b,
// and rows 8 apart a further 2 chunks (32 bytes) apart.
template <int CHUNKS>
__device__ __forceinline__ int swz_b16(int row)
{
    static_assert(CHUNKS >= 16, "rows of at least 256 bytes");
    return 4 * (row & 3) ^ 2 * ((row >> 3) & 1);
}

// ---- sparse A's position words ----------------------------------------------
// Word g of row r (k = 16 g .. 16 g + 15; kw = K / 16 words per row) is
// stored slice-major, so that the words of one 64-deep k slice of a block of
// rows are contiguous: slice s = g / 4 of the kw / 4 whole slices holds the
// M rows' 4 words each, [s][r][g % 4]; the kw % 4 words of a last, partial
// slice follow, [r][g % 4].
__host__ __device__ inline int64_t sp_meta_index(int64_t r, int64_t g, int64_t M, int64_t kw)
{
    const int64_t full = kw / 4, s = g / 4;
    return s < full ? (s * M + r) * 4 + g % 4 : full * M * 4 + r * (kw % 4) + g % 4;
}

// ---- tile index remap -----------------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin (id % 8).  Give XCD x a
// contiguous block of logical tile ids so its L2 sees neighbouring tiles, then
// walk tiles GROUP_M rows at a time (column-major inside the group) so that
// concurrently running tiles share A row-panels and B column-panels.
__device__ __forceinline__ void tile_coords(int wg, int grid, int tiles_m, int tiles_n, int group_m,
                                            int &tm, int &tn, int &split)
{
#if GEMM_F16_NO_XCD_REMAP
    int id = wg;
#else
    constexpr int kXcds = 8;
    int per = grid / kXcds, rem = grid % kXcds;
    int xcd = wg % kXcds, local = wg / kXcds;
    int id = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
#endif
    // split-K: the K splits of the tile space follow one another
    split = id / (tiles_m * tiles_n);
    id -= split * (tiles_m * tiles_n);
    int width = group_m * tiles_n;
    int group = id / width;
    int first_m = group * group_m;
    int gm = min(tiles_m - first_m, group_m);
    int in_group = id - group * width;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// ---- operands ----------------------------------------------------------------
template <int V>
struct VecT;
template <>
struct VecT<8> {
    typedef int4v type;
};
template <>
struct VecT<4> {
    typedef int2v type;
};
template <>
struct VecT<2> {
    typedef int type;
};
template <>
struct VecT<1> {
    typedef short type;
};

template <int V>
__device__ __forceinline__ typename VecT<V>::type buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    if constexpr (V == 8)
        return __builtin_bit_cast(int4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    else if constexpr (V == 4)
        return __builtin_bit_cast(int2v, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    else if constexpr (V == 2)
        return (int)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else
        return (short)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

template <int V>
__device__ __forceinline__ void lds_store(half_t *p, typename VecT<V>::type v)
{
    *reinterpret_cast<typename VecT<V>::type *>(p) = v;
}

// One operand of the product as a workgroup stages it: a BMN x BK slice per
// K step (BMN = bM for A, bN for B).
//
// ROWS_K: the stored matrix's rows run along k -- A given as M x K, or B given
// transposed as N x K.  The LDS tile is [BMN][BK] and an MFMA fragment (8 k
// of one m or n per lane) is one 16-byte read.  The workgroup's BMN rows form
// one buffer descriptor (rows past the matrix read as 0); columns past K are
// masked, since they would read the next row (16-byte chunks wholly past K
// by their offsets; with rows only 4-byte aligned, the part past K of the
// chunk that straddles the row end is zeroed in LDS by fix_tail).
//
// Otherwise the stored rows run along m or n -- A given transposed as K x M,
// or B given as K x N.  The LDS tile is [BK][BMN] (as in memory) and a
// fragment comes from two transposing reads: in each 16-lane group g (which
// covers half g % 2 of the 32 m or n and k half g / 2) lane j supplies the
// address of row 8 (g / 2) + j / 4 (+4 for the second read), columns
// 16 (g % 2) + 4 (j % 4) .. +3, and lane j receives column 16 (g % 2) + j.
// Each k slice is one buffer descriptor (rows past K read as 0); columns past
// the matrix edge are not masked: they only reach output rows or columns
// that are never stored.
// M16: the tile is read as 16x16x32 fragments (frag16); an mn-rows tile then
// uses swz_b16, which also separates rows 8 apart.
template <bool ROWS_K, int BMN, int BK, int THREADS, bool DIRECT, int V, bool M16 = false>
struct Operand {
    static constexpr int STAGE = BMN * BK;                   // halves per LDS stage
    static constexpr int ROW = ROWS_K ? BK : BMN;            // halves per LDS tile row
    static constexpr int CHUNKS = ROW / 8;                   // 16-byte chunks per row
    static constexpr int WAVES = THREADS / 64;
    static_assert(CHUNKS >= 2 && (CHUNKS & (CHUNKS - 1)) == 0, "rows of a power-of-two number of chunks");
    // direct: each lane moves one 16-byte chunk per load, so one wave
    // instruction fills 1 KiB of LDS, lane l at byte 16 l.  V is the
    // alignment of the stored rows in halves: 8 (16-byte rows) or 2 (rows
    // only 4-byte aligned).  The memory path serves 16-byte loads at any
    // 4-byte alignment (measured: with such rows 8-12 % faster than four
    // times as many 4-byte loads).  A k-rows operand's row of 4-byte
    // alignment ends inside a chunk when K % 8 != 0: that chunk's part past
    // K holds the next row's first elements until fix_tail zeroes it.
    static constexpr int WB = 16;
    static constexpr int WAVE_BYTES = 64 * WB;
    static constexpr int DMA = STAGE * 2 / (THREADS * WB);   // loads per thread per stage
    static_assert(!DIRECT || STAGE * 2 % (THREADS * WB) == 0, "whole block-wide loads");
    static_assert(!DIRECT || V == 8 || V == 2, "direct rows 16-byte or 4-byte aligned");
    static constexpr bool KTAIL = DIRECT && ROWS_K && V < 8;
    static_assert(!DIRECT || ROW * 2 <= WAVE_BYTES, "a row fits in one wave instruction");
    static constexpr int ROWS_PER_LOAD = DIRECT ? WAVE_BYTES / (ROW * 2) : 1;
    // consecutive direct loads of a thread are ROW_STEP rows apart, a multiple
    // of the swizzle period, so they share one column and one base offset
    static constexpr int ROW_STEP = WAVES * ROWS_PER_LOAD;
    // ... except: swz_b16 repeats every 16 rows, but its bit from row bit 3
    // flips every 8, and swz_a of 8-chunk rows (period 16) flips its bit 2
    // with row bit 3; loads whose row step is an odd multiple of 8 then
    // alternate between two columns
    static constexpr bool ALT_COLUMN = DIRECT && (ROWS_K ? CHUNKS == 8 : M16) && (ROW_STEP / 8) % 2 == 1;
    static_assert(!DIRECT || ROW_STEP % (ROWS_K ? (CHUNKS == 8 ? 8 : 16) : (M16 ? 8 : 4)) == 0,
                  "row step keeps the swizzle phase");
    // staged: vectors of V halves through registers
    static constexpr int VECS = STAGE / V / THREADS;
    static_assert(DIRECT || STAGE % (V * THREADS) == 0, "staged tiles split evenly over the threads");
    static constexpr int LOADS = DIRECT ? DMA : VECS;
    static constexpr int VEC_DIV = DIRECT ? 1 : VECS;

    __device__ __forceinline__ static int swz(int row)
    {
        if constexpr (ROWS_K)
            return swz_a<CHUNKS>(row);
        else if constexpr (M16)
            return swz_b16<CHUNKS>(row);
        else
            return swz_b<CHUNKS>(row);
    }

    const half_t *X;       // the stored matrix
    int ld;                // its row pitch (elements)
    int mn0;               // first m (A) or n (B) of the workgroup's tile
    int mn_total;          // M (A) or N (B)
    int K;                 // end of the workgroup's k range
    int kbase;             // start of the workgroup's k range (split-K), a multiple of BK
    __amdgpu_buffer_rsrc_t panel;   // ROWS_K: the workgroup's BMN rows
    uint32_t off0, step;   // direct: byte offset of the first chunk, distance between loads
    uint32_t alt;          // direct, ALT_COLUMN: offset change (mod 2^32) on odd loads
    int kcol0;             // direct, ROWS_K: k column of the thread's even loads
    int kcol1;             // ... and of its odd loads
    uint32_t voff[DIRECT ? DMA : 1];   // direct: the vector offset of each load of a slice
    uint32_t offv[VEC_DIV];
    int kcolv[VEC_DIV];
    int ldsv[VEC_DIV];
    typename VecT<V>::type reg[VEC_DIV];

    __device__ __forceinline__ void init(const half_t *x, int ld_, int mn0_, int mn_total_, int k_begin, int k_end,
                                         int tid, int wave, int lane)
    {
        X = x;
        ld = ld_;
        K = k_end;
        kbase = k_begin;
        mn_total = mn_total_;
        set_tile(mn0_);
        if constexpr (DIRECT) {
            const int byte = wave * WAVE_BYTES + lane * WB;
            const int r = byte / (ROW * 2);
            const int pos = (byte % (ROW * 2)) / 16;        // 16-byte chunk of the LDS row
            const int c = (pos ^ swz(r)) * 8;
            kcol0 = c;
            // (an mn-rows operand's tile origin mn0 is in its slice's base
            // address, so these offsets do not depend on the tile)
            off0 = ((uint32_t)r * (uint32_t)ld + (uint32_t)c) * 2u;
            step = (uint32_t)ROW_STEP * (uint32_t)ld * 2u;
            if constexpr (ALT_COLUMN) {
                // row r + ROW_STEP flips one bit of the row's XOR: the chunk moves
                const int c_odd = (pos ^ swz(r + ROW_STEP)) * 8;
                alt = (uint32_t)((c_odd - c) * 2);
                kcol1 = c_odd;
            } else {
                alt = 0;
                kcol1 = c;
            }
#pragma unroll
            for (int i = 0; i < DMA; ++i)
                voff[i] = off0 + (uint32_t)i * step + ((ALT_COLUMN && (i & 1)) ? alt : 0u);
        } else {
#pragma unroll
            for (int i = 0; i < VECS; ++i) {
                const int v = tid + THREADS * i;
                const int r = v / (ROW / V);
                const int c = (v % (ROW / V)) * V;
                kcolv[i] = c;
                offv[i] = ((uint32_t)r * (uint32_t)ld + (uint32_t)(ROWS_K ? c : mn0 + c)) * 2u;
                ldsv[i] = r * ROW + (((c / 8) ^ swz(r)) * 8) + (c % 8);
            }
        }
    }

    // Point the operand at the tile whose m (A) or n (B) range starts at
    // mn0_: the k-rows operand's panel of at most BMN rows (rows past the
    // matrix read as zero); an mn-rows operand keeps mn0 for its slices'
    // base address.
    __device__ __forceinline__ void set_tile(int mn0_)
    {
        mn0 = mn0_;
        if constexpr (ROWS_K) {
            const int rows = min(BMN, mn_total - mn0);
            panel = make_rsrc(X + (int64_t)mn0 * ld, (uint32_t)rows * (uint32_t)ld * 2u);
        }
    }

    // Start the loads of k slice kt of the workgroup's range: into LDS at dst
    // (direct) or into the registers (staged).  kt past the last slice is
    // allowed and reads zeros.  Direct loads may be issued in `nparts` parts
    // (part `part` of them here), spread over a tile's k steps.
    __device__ __forceinline__ void issue(int kt, half_t *dst, int wave, int part = 0, int nparts = 1)
    {
        const int k0 = kbase + kt * BK;
        __amdgpu_buffer_rsrc_t rs;
        uint32_t shift = 0;
        if constexpr (ROWS_K) {
            rs = panel;
            shift = (uint32_t)k0 * 2u;
        } else if constexpr (DIRECT) {
            // the slice's rows from column mn0 on: rows past K read as zero;
            // uniform by construction, readfirstlane keeps it in SGPRs
            const int rows = __builtin_amdgcn_readfirstlane(max(0, min(BK, K - k0)));
            const int m = __builtin_amdgcn_readfirstlane(mn0);
            rs = make_rsrc(X + (int64_t)k0 * ld + m,
                           rows > 0 ? (uint32_t)rows * (uint32_t)ld * 2u - (uint32_t)m * 2u : 0u);
        } else {
            // uniform by construction; readfirstlane keeps the descriptor in SGPRs
            const int rows = __builtin_amdgcn_readfirstlane(max(0, min(BK, K - k0)));
            rs = make_rsrc(X + (int64_t)k0 * ld, (uint32_t)rows * (uint32_t)ld * 2u);
        }
        if constexpr (DIRECT) {
            // Each load's vector offset comes from a register set up once;
            // the slice's k position is a scalar offset (k-rows operand) or
            // the slice's own buffer range (mn-rows operand).  The row part
            // stays in the range-checked vector offset, so rows past the
            // matrix read as zero; chunks that start at or past K get the
            // out-of-range bit OR-ed in.  (An mn-rows chunk that runs past
            // the matrix edge brings the next row's first elements into
            // columns past M or N, whose outputs are never stored.)
            const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((int)shift);
            const uint32_t mask0 = ROWS_K ? oob_unless(k0 + kcol0 < K) : 0u;
            const uint32_t mask1 = ROWS_K ? oob_unless(k0 + kcol1 < K) : 0u;
#pragma unroll
            for (int i = 0; i < DMA; ++i) {
                if (i * nparts / DMA != part)
                    continue;
                const bool odd = ALT_COLUMN && (i & 1);
                const uint32_t off = ROWS_K ? (voff[i] | (odd ? mask1 : mask0)) : voff[i];
                LDS_AS void *d = (LDS_AS void *)(dst + (wave + WAVES * i) * (WAVE_BYTES / 2));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, off, soff, 0, 0);
            }
        } else {
            (void)dst;
            (void)wave;
#pragma unroll
            for (int i = 0; i < VECS; ++i) {
                // ROWS_K: K % V == 0, so a vector is wholly inside or wholly past the row end
                const uint32_t mask = ROWS_K ? oob_unless(k0 + kcolv[i] < K) : 0u;
                reg[i] = buf_load<V>(rs, (offv[i] + shift) | mask);
            }
        }
    }

    // KTAIL: once this thread's loads of k slice kt (at dst) have landed,
    // zero the halves at or past K of each chunk it loaded that straddles
    // the row end.  K is even (4-byte rows) and a chunk starts at an even
    // column, so a straddling chunk keeps 2, 4 or 6 halves and whole dwords
    // are cleared.  Rows past the matrix already read as zero.
    __device__ __forceinline__ void fix_tail(int kt, half_t *dst, int wave, int lane) const
    {
        if constexpr (KTAIL) {
            const int k0 = kbase + kt * BK;
            const int v0 = K - (k0 + kcol0), v1 = K - (k0 + kcol1);
#pragma unroll
            for (int i = 0; i < DMA; ++i) {
                const int v = (ALT_COLUMN && (i & 1)) ? v1 : v0;   // halves of the chunk before K
                if (v > 0 && v < 8) {
                    uint32_t *p = reinterpret_cast<uint32_t *>(dst + (wave + WAVES * i) * (WAVE_BYTES / 2) + lane * 8);
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        if (2 * d >= v)
                            p[d] = 0u;
                }
            }
        } else {
            (void)kt;
            (void)dst;
            (void)wave;
            (void)lane;
        }
    }

    // staged: write the register-held slice into LDS at dst
    __device__ __forceinline__ void store(half_t *dst)
    {
        if constexpr (!DIRECT) {
#pragma unroll
            for (int i = 0; i < VECS; ++i)
                lds_store<V>(dst + ldsv[i], reg[i]);
        } else {
            (void)dst;
        }
    }

    // v_mfma_f32_16x16x32_f16 fragment: the 16 m (or n) starting at mnb of
    // the 32-deep k step ks; lane l gets 8 k values 32 ks + 8 (l / 16) .. +7
    // of m (or n) mnb + l % 16.  k-rows tile: one 16-byte read (16 rows per
    // pass, conflict-free under swz_a).  mn-rows tile: two transposing reads;
    // in 16-lane group g, lane j gives the address of row 32 ks + 8 g + j / 4
    // (+4), columns mnb + 4 (j % 4) .. +3, and lane i receives column mnb + i.
    // A pass of 32 lanes covers rows k..k+3 and k+8..k+11, 32 bytes each:
    // swz_b16 puts them in 8 different 32-byte slots of the bank window.
    __device__ __forceinline__ half8 frag16(const half_t *stage, int mnb, int ks, int lane) const
    {
        static_assert(M16, "a tile read as 16x16x32 fragments uses the M16 swizzle");
        if constexpr (ROWS_K) {
            const int r = mnb + (lane & 15);
            const int c = 4 * ks + (lane >> 4);
            return *reinterpret_cast<const half8 *>(stage + r * ROW + ((c ^ swz(r)) * 8));
        } else {
            const int g = lane >> 4, j = lane & 15;
            const int r0 = 32 * ks + 8 * g + (j >> 2);
            const int r1 = r0 + 4;
            const int col = mnb + 4 * (j & 3);
            const half_t *p0 = stage + r0 * ROW + (((col >> 3) ^ swz(r0)) * 8) + (col & 7);
            const half_t *p1 = stage + r1 * ROW + (((col >> 3) ^ swz(r1)) * 8) + (col & 7);
            short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4v *)p0);
            short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4v *)p1);
            half4 lo_h = __builtin_bit_cast(half4, lo);
            half4 hi_h = __builtin_bit_cast(half4, hi);
            return half8{lo_h[0], lo_h[1], lo_h[2], lo_h[3], hi_h[0], hi_h[1], hi_h[2], hi_h[3]};
        }
    }

    // MFMA fragment for the 32 m (or n) starting at mnb of k step ks: lane l
    // gets 8 k values 16 ks + 8 (l / 32) .. +7 of m (or n) mnb + l % 32.
    __device__ __forceinline__ half8 frag(const half_t *stage, int mnb, int ks, int lane) const
    {
        if constexpr (ROWS_K) {
            const int r = mnb + (lane & 31);
            const int c = 2 * ks + (lane >> 5);
            return *reinterpret_cast<const half8 *>(stage + r * ROW + ((c ^ swz(r)) * 8));
        } else {
            const int g = lane >> 4, j = lane & 15;
            const int r0 = 16 * ks + 8 * (g >> 1) + (j >> 2);
            const int r1 = r0 + 4;
            const int col = mnb + 16 * (g & 1) + 4 * (j & 3);
            const half_t *p0 = stage + r0 * ROW + (((col >> 3) ^ swz(r0)) * 8) + (col & 7);
            const half_t *p1 = stage + r1 * ROW + (((col >> 3) ^ swz(r1)) * 8) + (col & 7);
            short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4v *)p0);
            short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4v *)p1);
            half4 lo_h = __builtin_bit_cast(half4, lo);
            half4 hi_h = __builtin_bit_cast(half4, hi);
            return half8{lo_h[0], lo_h[1], lo_h[2], lo_h[3], hi_h[0], hi_h[1], hi_h[2], hi_h[3]};
        }
    }
};

// ---- the kernel -------------------------------------------------------------
// SPARSE: A is 2:4 structured-sparse, given as compressed values (M x K/2,
// staged like a k-rows operand of BK/2 columns per tile) and positions
// (M x K/16 uint16 words, loaded straight into registers); the product uses
// v_smfmac_f32_32x32x32_f16, 32 k per step.
// M16: v_mfma_f32_16x16x32_f16 on 16x16 blocks (32 k per step) instead of
// 32x32x16.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool DIRECT, int VA, int VB, bool A_ROWS_K,
          bool B_ROWS_K, bool SPARSE = false, bool M16 = false>
struct Tile {
    static constexpr int kWaves = WM * WN;           // 4 (one per SIMD) or 8 (two per SIMD)
    static constexpr int kThreads = 64 * kWaves;
    static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves");
    static constexpr int WTM = BM / WM;              // wave sub-tile rows (m)
    static constexpr int WTN = BN / WN;              // wave sub-tile cols (n)
    static constexpr int BLK = M16 ? 16 : 32;        // MFMA block edge
    static constexpr int TM = WTM / BLK;             // MFMA blocks per wave along m
    static constexpr int TN = WTN / BLK;             // ... along n
    static_assert(TM >= 1 && TN >= 1 && WTM % BLK == 0 && WTN % BLK == 0, "wave tile");
    static_assert(!M16 || !SPARSE, "16x16x32 blocks: dense only");
    static constexpr int KSTEP = SPARSE || M16 ? 32 : 16;   // k per MFMA step
    static_assert(BK % KSTEP == 0, "whole MFMA steps per tile");
    static_assert(!SPARSE || (A_ROWS_K && DIRECT), "sparse A: compressed rows, direct loads");
    using OpA = Operand<A_ROWS_K, BM, SPARSE ? BK / 2 : BK, kThreads, DIRECT, VA, M16>;
    using OpB = Operand<B_ROWS_K, BN, BK, kThreads, DIRECT, VB, M16>;
    static constexpr int A_STAGE = OpA::STAGE;
    static constexpr int B_STAGE = OpB::STAGE;
    // sparse A's position words of a 64-deep slice, per stage: two dwords
    // per tile row, stored dword-major ([2][BM])
    static constexpr int META_STAGE = SPARSE ? 2 * BM * 4 : 0;
    static constexpr int LDS_BYTES = STAGES * ((A_STAGE + B_STAGE) * 2 + META_STAGE);
    static_assert(LDS_BYTES <= 163840, "LDS budget");
};

// SPREAD (direct kernels): the loads of the tile requested during a step are
// issued in SPREAD parts, one with each of the first SPREAD k steps, instead
// of all at its start, so that the waves do not queue a whole tile of loads
// ahead of their MFMAs at once (measured: 4 parts +3 % for 256x256 tiles
// with 4 waves and +6-8 % for 128x128; 2 parts +0-3 % with 8 waves, where 4
// parts leave the last loads too little time).  1: all at the start.
// EPI_ONLY: 1 compiles the LDS-staged fp16 epilogue alone (no split-K
// partials, N % 8 == 0 and C 16-byte aligned), 2 the split-K partial stores
// alone, 3 the direct fp16 stores alone (8- or 2-byte pieces), 0 every path.  For tiles whose accumulator fills the matrix-core
// registers: with one epilogue path the accumulator does not have to be held
// in vector registers across a branch, where it overflows them and spills to
// scratch.
// WIDE_META (sparse, K % 64 == 0): the four position words of a 64-deep
// slice of every tile row travel to LDS with the slice's operands (4-byte
// direct loads, two per row), and each fragment reads its words from there,
// instead of 2-byte loads into registers per row and k step.  Loads into
// registers would make the compiler wait for them with a count that also
// covers later tiles' loads, draining the prefetch ring every slice.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool DIRECT, int VA, int VB, bool A_ROWS_K,
          bool B_ROWS_K, int SPREAD = 1, bool SPARSE = false, bool M16 = false, int EPI_ONLY = 0,
          bool WIDE_META = false>
__global__ void __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
gemm_f16_kernel(KernelArgs args)
{
    constexpr bool STAGED_ONLY = EPI_ONLY == 1, SPLIT_ONLY = EPI_ONLY == 2, DIRECT_ONLY = EPI_ONLY == 3;
    using T = Tile<BM, BN, BK, WM, WN, STAGES, DIRECT, VA, VB, A_ROWS_K, B_ROWS_K, SPARSE, M16>;
    __shared__ __attribute__((aligned(1024))) half_t lds[T::LDS_BYTES / 2];
    half_t *const As = lds;                                  // STAGES A stages
    half_t *const Bs = lds + STAGES * T::A_STAGE;            // STAGES B stages
    // sparse: STAGES position-word stages after the operand stages
    uint32_t *const Ms = reinterpret_cast<uint32_t *>(lds + STAGES * (T::A_STAGE + T::B_STAGE));

    const int M = args.M, N = args.N, K = args.K;
    int tm, tn, split;
    tile_coords(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, args.group_m, tm, tn, split);
    const int m0 = tm * BM, n0 = tn * BN;
    // the workgroup's k range: all of K, or one split of k_split (a multiple of BK)
    const int k_begin = split * args.k_split;
    const int k_end = min(K, k_begin + args.k_split);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / WN) * T::WTM;                   // wave sub-tile origin in the tile
    const int wn0 = (wave % WN) * T::WTN;

    const int nk = (k_end - k_begin + BK - 1) / BK;

    // A is M x K (lda = K) or, given transposed, K x M (lda = M); B is K x N
    // (ldb = N) or, given transposed, N x K (ldb = K).  Sparse A: the
    // compressed values, M x K/2, addressed in compressed columns.
    typename T::OpA opa;
    typename T::OpB opb;
    if constexpr (SPARSE)
        opa.init(args.A, K / 2, m0, M, k_begin / 2, k_end / 2, tid, wave, lane);
    else
        opa.init(args.A, A_ROWS_K ? K : M, m0, M, k_begin, k_end, tid, wave, lane);
    opb.init(args.B, B_ROWS_K ? K : N, n0, N, k_begin, k_end, tid, wave, lane);

    // Sparse A's positions: lane l of fragment i (row wm0 + 32 i + l % 32)
    // uses, in MFMA step ks of tile kt, the word of its half l / 32 of those
    // 32 k: word (k_begin + kt BK) / 16 + 2 ks + l / 32 of its row.  They are
    // loaded with each tile's operands (before them, so that the waits for a
    // tile cover its words too) into slot kt % STAGES.
    constexpr int NSTEP = BK / T::KSTEP;
    constexpr int MSLOTS = SPARSE ? STAGES : 1;
    static_assert(!WIDE_META || (SPARSE && NSTEP == 2), "wide position loads: two 32-deep steps per slice");
    // vector memory loads of one tile per lane: the operands' and sparse A's
    // position words (one per fragment row, or one per row and k step)
    // wide: each thread moves META_DMA of the stage's 2 BM position dwords
    constexpr int META_DMA = WIDE_META ? 2 * BM / T::kThreads : 1;
    static_assert(!WIDE_META || (2 * BM) % T::kThreads == 0, "whole position loads per thread");
    constexpr int kMetaLoads = SPARSE ? (WIDE_META ? META_DMA : T::TM * NSTEP) : 0;
    constexpr int kLoadsPerTile = T::OpA::LOADS + T::OpB::LOADS + kMetaLoads;
    uint32_t meta[MSLOTS][T::TM][SPARSE && !WIDE_META ? NSTEP : 1];
    const uint32_t mshift = 16u * (uint32_t)(lane >> 5);   // wide: the lane's word in each dword
    static_assert(!SPARSE || BK == 64, "position words are stored by 64-deep slices");
    const int kwords = K / 16;
    // the descriptor of slice s's words for this tile's rows (sp_meta_index):
    // rows of `stride` words from `base`; rows past M, and slices past K,
    // read zeros
    auto meta_slice = [&](int s, int &stride) __attribute__((always_inline)) {
        const int full = kwords / 4;
        const uint32_t rows = (uint32_t)min(BM, M - m0);
        if (s < full) {
            stride = 4;
            return make_rsrc(args.meta + ((int64_t)s * M + m0) * 4, rows * 8u);
        }
        stride = kwords % 4;
        return make_rsrc(args.meta + (int64_t)full * M * 4 + (int64_t)m0 * stride,
                         s == full ? rows * (uint32_t)stride * 2u : 0u);
    };
    auto issue_meta = [&](int kt, int slot) {
        if constexpr (WIDE_META) {
            // the slice's words of the tile's rows are 8 BM contiguous bytes:
            // thread load i moves dword q = (i waves + wave) 64 + lane of them
            // to LDS dword q of the slot (row q / 2, words 2 (q % 2), +1)
            int stride;
            const __amdgpu_buffer_rsrc_t rs = meta_slice((k_begin + kt * BK) / 64, stride);
#pragma unroll
            for (int i = 0; i < META_DMA; ++i) {
                const int q0 = (i * T::kWaves + wave) * 64;
                LDS_AS void *d = (LDS_AS void *)(Ms + slot * 2 * BM + q0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 4, (uint32_t)(q0 + lane) * 4u, 0, 0, 0);
            }
        } else if constexpr (SPARSE) {
            // word 2 ks + lane / 32 of the slice for each fragment row; past
            // the row's words (a partial last slice) reads zero
            int stride;
            const __amdgpu_buffer_rsrc_t rs = meta_slice((k_begin + kt * BK) / 64, stride);
#pragma unroll
            for (int ks = 0; ks < NSTEP; ++ks) {
                const int j = 2 * ks + (lane >> 5);
                const uint32_t mask = oob_unless(j < stride);
#pragma unroll
                for (int i = 0; i < T::TM; ++i)
                    meta[slot][i][ks] = (uint32_t)(unsigned short)__builtin_amdgcn_raw_buffer_load_b16(
                        rs, ((uint32_t)((wm0 + 32 * i + (lane & 31)) * stride + j) * 2u) | mask, 0, 0);
            }
        } else {
            (void)kt;
            (void)slot;
        }
    };

    auto issue_loads = [&](int kt, half_t *dst_a, half_t *dst_b, int part = 0, int nparts = 1,
                           int mslot = 0) __attribute__((always_inline)) {
        if (part == 0)
            issue_meta(kt, mslot);
        opa.issue(kt, dst_a, wave, part, nparts);
        opb.issue(kt, dst_b, wave, part, nparts);
    };
    auto store_staged = [&](half_t *dst_a, half_t *dst_b) {
        opa.store(dst_a);
        opb.store(dst_b);
    };

    using Acc = typename std::conditional<M16, float4v, float16v>::type;
    Acc acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
            acc[i][j] = Acc{};

    // Fragments of one 16-deep k step: x = B^T slices (one per 32-column
    // block), y = A^T slices (one per 32-row block).
    // Sparse: x holds 32 k of B per lane (two 16-deep fragments: k 8 h .. +7
    // and 16 + 8 h .. +7 of the step, h = lane / 32, the order
    // v_smfmac_f32_32x32x32_f16 pairs with A's compressed values, measured
    // with a one-wave probe), y the 8 compressed values of A (its 16 k), and
    // idx the positions word of each A fragment.
    using BFrag = typename std::conditional<SPARSE, half16, half8>::type;
    struct Frags {
        BFrag x[T::TN];
        half8 y[T::TM];
        uint32_t idx[SPARSE ? T::TM : 1];
    };
    auto load_frags = [&](Frags &f, const half_t *as, const half_t *bs, int ks, int mslot = 0) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            if constexpr (M16)
                f.y[i] = opa.frag16(as, wm0 + 16 * i, ks, lane);
            else
                f.y[i] = opa.frag(as, wm0 + 32 * i, ks, lane);
        }
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            if constexpr (M16) {
                f.x[j] = opb.frag16(bs, wn0 + 16 * j, ks, lane);
            } else if constexpr (SPARSE) {
                const half8 lo = opb.frag(bs, wn0 + 32 * j, 2 * ks, lane);
                const half8 hi = opb.frag(bs, wn0 + 32 * j, 2 * ks + 1, lane);
                f.x[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
            } else {
                f.x[j] = opb.frag(bs, wn0 + 32 * j, ks, lane);
            }
        }
        if constexpr (WIDE_META) {
            // step ks uses word 2 ks + lane / 32 of the row: dword ks of the
            // row shifted by the lane's half (the instruction reads the low half)
            const uint32_t *ms = Ms + mslot * 2 * BM + 2 * (wm0 + (lane & 31)) + ks;
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
                f.idx[i] = ms[64 * i] >> mshift;
        } else if constexpr (SPARSE) {
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
                f.idx[i] = meta[mslot][i][ks];
        } else {
            (void)mslot;
        }
    };
    auto mma = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int jj = 0; jj < T::TN; ++jj) {
#if GEMM_F16_SNAKE
                const int j = (i & 1) ? T::TN - 1 - jj : jj;
#else
                const int j = jj;
#endif
                if constexpr (SPARSE)
                    // C = A . B directly: the sparse operand must come first
                    acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(f.y[i], f.x[j], acc[i][j],
                                                                          (int)f.idx[i], 0, 0);
                else if constexpr (M16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.x[j], f.y[i], acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.x[j], f.y[i], acc[i][j], 0, 0, 0);
            }
    };
    // Ask the scheduler to alternate the MFMAs of one step with the LDS reads
    // of the next step (and, after a barrier, with the next tile's loads and
    // LDS writes), so the matrix core keeps busy while those are in flight.
    constexpr int kMfmaPerStep = T::TM * T::TN;
    constexpr int kReadsPerStep = M16 ? (A_ROWS_K ? 1 : 2) * T::TM + (B_ROWS_K ? 1 : 2) * T::TN
                                      : T::TM + (SPARSE ? 4 : 2) * T::TN + (WIDE_META ? T::TM : 0);
    // The next step's fragment reads are requested during the current step's
    // MFMAs, at the rate set by the placement switches above.
    // (a small 16x16x32 wave tile has fewer MFMAs than reads per step: one
    // MFMA then carries as many reads as it takes)
    constexpr bool kM16Fits = kMfmaPerStep / GEMM_F16_M16_READ_EVERY * GEMM_F16_M16_READS_PER_MFMA >= kReadsPerStep;
    constexpr int kReadsPerMfma = M16 ? (kM16Fits ? GEMM_F16_M16_READS_PER_MFMA
                                                  : (kReadsPerStep + kMfmaPerStep - 1) / kMfmaPerStep)
                                      : GEMM_F16_READS_PER_MFMA;
    constexpr int kReadEvery = M16 ? (kM16Fits ? GEMM_F16_M16_READ_EVERY : 1) : GEMM_F16_READ_EVERY;
    static_assert(!M16 || kMfmaPerStep / kReadEvery * kReadsPerMfma >= kReadsPerStep, "every read has a slot");
    constexpr int kVmemEvery = M16 ? GEMM_F16_M16_VMEM_EVERY : GEMM_F16_VMEM_EVERY;
    auto interleave = [&](int n_vmem, int n_dswrite) {
#pragma unroll
        for (int i = 0; i < kMfmaPerStep; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
#pragma unroll
            for (int r = 0; r < kReadsPerMfma; ++r)
                if (i % kReadEvery == 0 && (i / kReadEvery) * kReadsPerMfma + r < kReadsPerStep)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            if (i < n_dswrite)
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);      // one LDS write
            if (i % kVmemEvery == 0 && i / kVmemEvery < n_vmem)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // one global load
        }
    };

    // ---- pipelined K loop ----
    // Software pipeline over the k steps of a tile with two fragment sets:
    // the reads of step s+1 are in flight while step s multiplies.  The last
    // step of a tile is multiplied after the next barrier, so that the first
    // reads of the next tile overlap MFMA work too.
    //  direct:  stage ring of STAGES tiles filled by DMA, tile kt+STAGES-1
    //           requested at step kt;
    //  staged:  registers hold tile kt+1 at the start of step kt; the step
    //           writes them to the free stage, requests tile kt+2 into the
    //           registers, then multiplies tile kt (two LDS stages suffice).
    constexpr int NS = BK / T::KSTEP;
    static_assert(NS % 2 == 0 || STAGES % 2 == 0, "a constant fragment-set parity per unrolled tile");
    static_assert(DIRECT || STAGES == 2, "register-staged kernels use two LDS stages");
    constexpr int LOOKAHEAD = DIRECT ? STAGES - 1 : 2;
    // Two fragment sets, f0 and f1: set `cur` receives step 0 of a tile and
    // the sets alternate over its steps; a tile's last step is multiplied by
    // the next tile's step call (or after the loop).  With an even number of
    // steps per tile every tile has cur 0; with an odd number cur alternates.
    // (Named variables, not an array: they must stay in registers.)
    Frags f0, f1 = {};   // f1 zero: an empty K loop multiplies zeros below
    // One tile: bring tile kt_next toward LDS -- (wr_a, wr_b) is the stage it
    // (direct) or the register-held tile (staged) goes to -- then the math on
    // stage (rd_a, rd_b); the set other than `cur` holds the previous tile's
    // last step when `pending`.  The restrict qualifiers tell the compiler that the stage
    // being filled is not the stage being read, so it does not make the LDS
    // reads wait for those loads or writes.
    constexpr bool SPREAD_LOADS = DIRECT && SPREAD > 1;
    constexpr int PARTS = SPREAD_LOADS ? SPREAD : 1;
    static_assert(PARTS <= NS && (T::OpA::LOADS + T::OpB::LOADS) % PARTS == 0, "whole parts, one per k step at most");
    // rd_slot / wr_slot: the stage indices of (rd_a, rd_b) and (wr_a, wr_b),
    // which are also the register slots of sparse A's position words
    auto step = [&](auto cur_c, const half_t *__restrict__ rd_a, const half_t *__restrict__ rd_b,
                    half_t *__restrict__ wr_a, half_t *__restrict__ wr_b, int kt_next, bool pending,
                    int rd_slot, int wr_slot) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur_c)::value;
        // direct, spread: part p of the requested tile goes out with k step p
        auto issue_part = [&](int p) __attribute__((always_inline)) {
            if constexpr (SPREAD_LOADS)
                if (p < PARTS)
                    issue_loads(kt_next, wr_a, wr_b, p, PARTS, wr_slot);
        };
        if constexpr (DIRECT) {
            // past the last tile: zeros into a retired stage
            if constexpr (SPREAD_LOADS)
                issue_part(0);
            else
                issue_loads(kt_next, wr_a, wr_b, 0, 1, wr_slot);
        } else {
            wait_vmcnt<0>();                    // tile kt+1 is in the registers
            store_staged(wr_a, wr_b);
            issue_loads(kt_next, nullptr, nullptr);
        }
        if constexpr (CUR == 0) {
            load_frags(f0, rd_a, rd_b, 0, rd_slot);
            if (pending)
                mma(f1);
        } else {
            load_frags(f1, rd_a, rd_b, 0, rd_slot);
            if (pending)
                mma(f0);
        }
        constexpr int PART_LOADS = kLoadsPerTile / PARTS;
        interleave(DIRECT ? PART_LOADS : 0, DIRECT ? 0 : kLoadsPerTile);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 1; ks < NS; ++ks) {
            issue_part(ks);
            if ((CUR + ks) & 1) {          // a constant once the loop is unrolled
                load_frags(f1, rd_a, rd_b, ks, rd_slot);
                mma(f0);
            } else {
                load_frags(f0, rd_a, rd_b, ks, rd_slot);
                mma(f1);
            }
            interleave(SPREAD_LOADS && ks < PARTS ? PART_LOADS : 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // set (CUR + NS - 1) & 1 now holds step NS-1 of this tile, multiplied by the next call
    };
    // Wait until tile kt (in stage `stage`) is in LDS for every wave: this
    // wave's loads (direct) or LDS writes (staged) of it have completed, and
    // so have its reads of the stage about to be refilled; then the
    // workgroup barrier.  Rows only 4-byte aligned: in the range's last
    // tile each thread first clears the halves past K of the chunks it
    // loaded that straddle a row end.
    auto tile_ready = [&](int kt, int stage) {
        if constexpr (DIRECT) {
            if (kt + STAGES - 2 < nk)
                wait_vm_lgkm0<(STAGES - 2) * kLoadsPerTile>();
            else
                wait_vm_lgkm0<0>();
            if constexpr (T::OpA::KTAIL || T::OpB::KTAIL) {
                if (kt == nk - 1) {
                    // (the last tile waited for every load; the clobber keeps
                    // the compiler from moving the clears above that wait)
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                    opa.fix_tail(kt, As + stage * T::A_STAGE, wave, lane);
                    opb.fix_tail(kt, Bs + stage * T::B_STAGE, wave, lane);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
            }
        } else {
            (void)stage;
            (void)kt;
            wait_lgkm0();
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (DIRECT) {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nk)
                issue_loads(s, As + s * T::A_STAGE, Bs + s * T::B_STAGE, 0, 1, s);
    } else {
        if (nk > 0) {
            issue_loads(0, nullptr, nullptr);
            wait_vmcnt<0>();
            store_staged(As, Bs);
            issue_loads(1, nullptr, nullptr);
        }
    }
    // the stage written during step kt is (kt + W_OFF) % STAGES
    constexpr int W_OFF = DIRECT ? LOOKAHEAD : 1;
    if (nk > 0) {
        tile_ready(0, 0);
        step(std::integral_constant<int, 0>{}, As, Bs, As + (W_OFF % STAGES) * T::A_STAGE,
             Bs + (W_OFF % STAGES) * T::B_STAGE, LOOKAHEAD, false, 0, W_OFF % STAGES);
    }
    // tiles 1 .. nk-1 in groups of STAGES, unrolled so that every stage index
    // (and fragment-set parity) is a constant
    for (int kt0 = 1; kt0 < nk; kt0 += STAGES) {
#pragma unroll
        for (int u = 0; u < STAGES; ++u) {
            const int kt = kt0 + u;
            const int s = (1 + u) % STAGES;                 // stage holding tile kt
            const int w = (s + W_OFF) % STAGES;
            if (kt < nk) {
                tile_ready(kt, s);
                // kt0 = 1 + STAGES j: with NS odd and STAGES even, kt's parity is (1 + u)'s
                if (((1 + u) * NS) & 1)
                    step(std::integral_constant<int, 1>{}, As + s * T::A_STAGE, Bs + s * T::B_STAGE,
                         As + w * T::A_STAGE, Bs + w * T::B_STAGE, kt + LOOKAHEAD, true, s, w);
                else
                    step(std::integral_constant<int, 0>{}, As + s * T::A_STAGE, Bs + s * T::B_STAGE,
                         As + w * T::A_STAGE, Bs + w * T::B_STAGE, kt + LOOKAHEAD, true, s, w);
            }
        }
    }
    // the last tile's last step: set (nk NS - 1) & 1 (set 1, zero, when nk = 0)
    if constexpr (NS % 2 == 0) {
        if (EPI_ONLY != 0 || nk > 0)
            mma(f1);
    } else {
        // nk odd: the last tile (nk - 1, even) ended in f0
        const bool odd = (nk & 1) != 0;
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
            f1.x[j] = odd ? f0.x[j] : f1.x[j];
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
            f1.y[i] = odd ? f0.y[i] : f1.y[i];
        if (EPI_ONLY != 0 || nk > 0)
            mma(f1);
    }
    wait_vmcnt<0>();   // the tail's zero-filling loads must land before the workgroup retires

    const int c_rows = min(BM, M - m0);
    // The accumulator of MFMA block (i, j) holds, in register group g (32x32
    // blocks: g = 0..3; 16x16 blocks: g = 0), four consecutive columns
    // col_of(j, g) .. +3 of the tile in row row_of(i) of the panel (the
    // dense product is computed transposed, C^T = B^T . A^T).
    constexpr int GROUPS = M16 ? 1 : 4;
    auto row_of = [&](int i) { return M16 ? wm0 + 16 * i + (lane & 15) : wm0 + 32 * i + (lane & 31); };
    auto col_of = [&](int j, int g) {
        return M16 ? wn0 + 16 * j + 4 * (lane >> 4) : wn0 + 32 * j + 8 * g + 4 * (lane >> 5);
    };
    if constexpr (SPARSE && STAGED_ONLY) {
        // C = A . B was computed untransposed: lane l of block (i, j) holds
        // column wn0 + 32 j + l % 32, rows wm0 + 32 i + 8 g + 4 (l / 32) + r
        // in accumulator 4 g + r.  N % 8 == 0 and C 16-byte aligned: the fp16
        // tile is staged through the (now idle) LDS, [BM][BN] with each
        // row's 16-byte chunks XOR-ed by 4 when row bit 2 is set (the two
        // half-waves of a write, rows 4 apart, then land in disjoint banks),
        // and leaves as 16-byte pieces of whole rows.
        static_assert(BM * BN * 2 <= T::LDS_BYTES, "the output tile fits in the LDS stages");
        half_t *c_base = args.C + (int64_t)m0 * N;
        const __amdgpu_buffer_rsrc_t c_rsrc = make_rsrc(c_base, (uint32_t)c_rows * (uint32_t)N * 2u);
        const bool relu = args.relu != 0;
        const float alpha = args.alpha;
        auto swz = [](int row) { return ((row >> 2) & 1) * 4; };
        half_t *ct = lds;
        wait_vmcnt<0>();
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();                       // every wave is done with the stages
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int c = wn0 + 32 * j + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm0 + 32 * i + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
                    float x = acc[i][j][v] * alpha;
                    if (relu)
                        x = __builtin_fmaxf(x, 0.0f);
                    ct[r * BN + (((c >> 3) ^ swz(r)) << 3) + (c & 7)] = (half_t)x;
                }
            }
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        constexpr int CHUNKS_PER_ROW = BN / 8;
        constexpr int PER_THREAD = BM * CHUNKS_PER_ROW / T::kThreads;
        static_assert(BM * CHUNKS_PER_ROW % T::kThreads == 0, "output chunks split evenly");
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int id = tid + q * T::kThreads;
            const int r = id / CHUNKS_PER_ROW;
            const int c8 = id % CHUNKS_PER_ROW;
            const int4v v = *reinterpret_cast<const int4v *>(ct + r * BN + ((c8 ^ swz(r)) << 3));
            const int n = n0 + 8 * c8;
            const uint32_t off = ((uint32_t)r * (uint32_t)N + (uint32_t)n) * 2u;
            __builtin_amdgcn_raw_buffer_store_b128(v, c_rsrc, off | oob_unless(n < N), 0, GEMM_F16_C_CPOL);
        }
        return;
    }
    if constexpr (SPARSE) {
        // C = A . B was computed untransposed: lane l of block (i, j) holds
        // column wn0 + 32 j + l % 32, rows wm0 + 32 i + 8 g + 4 (l / 32) + r
        // in accumulator 4 g + r.  Each store writes one element; the 32
        // lanes of a half-wave cover 64 consecutive bytes of one row.
        half_t *c_base = args.C + (int64_t)m0 * N;
        const __amdgpu_buffer_rsrc_t c_rsrc = make_rsrc(c_base, (uint32_t)c_rows * (uint32_t)N * 2u);
        const bool relu = args.relu != 0;
        const float alpha = args.alpha;
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int n = n0 + wn0 + 32 * j + (lane & 31);
                const uint32_t col_mask = oob_unless(n < N);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm0 + 32 * i + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
                    float x = acc[i][j][v] * alpha;
                    if (relu)
                        x = __builtin_fmaxf(x, 0.0f);
                    const half_t h = (half_t)x;
                    const uint32_t off = ((uint32_t)r * (uint32_t)N + (uint32_t)n) * 2u;
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, h), c_rsrc, off | col_mask, 0,
                                                          GEMM_F16_C_CPOL);
                }
            }
        return;
    }
    if (SPLIT_ONLY || (!STAGED_ONLY && !DIRECT_ONLY && args.W)) {
        // split-K: the fp32 partial sums of this split go to its slice of the
        // workspace (row pitch N); the reduction applies the epilogue.  When
        // N % 4 == 0 a lane's four consecutive columns leave as one 16-byte
        // store, else as four 4-byte stores.
        float *w_base = args.W + ((int64_t)split * M + m0) * N;
        const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(w_base, (uint32_t)c_rows * (uint32_t)N * 4u);
        const bool w4 = (N & 3) == 0;
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int r = row_of(i);
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int g = 0; g < GROUPS; ++g) {
                    const int n = n0 + col_of(j, g);
                    const uint32_t off = ((uint32_t)r * (uint32_t)N + (uint32_t)n) * 4u;
                    // element values copied to scalars before any bit cast (see out4)
                    const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                    const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                    if (w4) {
                        const float4v v = {v0, v1, v2, v3};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4v, v), w_rsrc,
                                                               off | oob_unless(n < N), 0, 0);
                    } else {
                        const int bits[4] = {__builtin_bit_cast(int, v0), __builtin_bit_cast(int, v1),
                                             __builtin_bit_cast(int, v2), __builtin_bit_cast(int, v3)};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            __builtin_amdgcn_raw_buffer_store_b32(bits[e], w_rsrc,
                                                                  (off + 4u * e) | oob_unless(n + e < N), 0, 0);
                    }
                }
        }
        return;
    }

    // ---- epilogue: scale, optional ReLU, RNE to fp16, store ----
    half_t *c_base = args.C + (int64_t)m0 * N;
    const __amdgpu_buffer_rsrc_t c_rsrc = make_rsrc(c_base, (uint32_t)c_rows * (uint32_t)N * 2u);
    const bool relu = args.relu != 0;
    const float alpha = args.alpha;
    const int vec_c = args.vec_c;
    // The four values of block (i, j), group g, as fp16 after the epilogue
    // (alpha = 1 leaves the sums unchanged: x * 1 is exact).
    auto out4 = [&](int i, int j, int g, half_t &h0, half_t &h1, half_t &h2, half_t &h3) {
        float v0 = acc[i][j][4 * g + 0] * alpha, v1 = acc[i][j][4 * g + 1] * alpha;
        float v2 = acc[i][j][4 * g + 2] * alpha, v3 = acc[i][j][4 * g + 3] * alpha;
        if (relu) {
            v0 = __builtin_fmaxf(v0, 0.0f);
            v1 = __builtin_fmaxf(v1, 0.0f);
            v2 = __builtin_fmaxf(v2, 0.0f);
            v3 = __builtin_fmaxf(v3, 0.0f);
        }
        // RNE conversions kept as scalars: hipcc mis-lowers a bit_cast of a
        // single element of an fp16 ext_vector (it re-reads element 0)
        h0 = (half_t)v0;
        h1 = (half_t)v1;
        h2 = (half_t)v2;
        h3 = (half_t)v3;
    };
    static_assert(BM * BN * 2 <= T::LDS_BYTES, "the output tile fits in the LDS stages");
    if (STAGED_ONLY || (!DIRECT_ONLY && vec_c == 8)) {
        // N % 8 == 0 and C 16-byte aligned: stage the fp16 tile through the
        // (now idle) LDS and write it as 16-byte pieces of consecutive
        // columns, so that every row of the tile leaves as whole cache lines.
        // LDS layout [BM][BN] with the 8-byte unit index XOR-ed with the row's
        // low bits: the 32 lanes of a pass write 32 different rows of one
        // column unit (32x32 blocks) or 16 rows of two units (16x16 blocks),
        // and SQ_LDS_BANK_CONFLICT reads 0 for both.  (Twice the row's low
        // 4 bits for 16x16 blocks, although distinct per pass in a 64-bank
        // model, measured 1.5 % conflict cycles.)
        constexpr int UNITS = BN / 4;                       // 8-byte units per row
        constexpr int UMASK = (UNITS < 32 ? UNITS : 32) - 1;
        auto swz = [](int row) { return row & UMASK; };
        half_t *ct = lds;
        wait_vmcnt<0>();
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();                       // every wave is done with the stages
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int r = row_of(i);
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int g = 0; g < GROUPS; ++g) {
                    half_t h0, h1, h2, h3;
                    out4(i, j, g, h0, h1, h2, h3);
                    const int u = col_of(j, g) / 4;
                    half4 h = {h0, h1, h2, h3};
                    *reinterpret_cast<half4 *>(ct + r * BN + 4 * (u ^ swz(r))) = h;
                }
        }
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        constexpr int CHUNKS_PER_ROW = BN / 8;
        constexpr int PER_THREAD = BM * CHUNKS_PER_ROW / T::kThreads;
        static_assert(BM * CHUNKS_PER_ROW % T::kThreads == 0, "output chunks split evenly");
#pragma unroll
        for (int q = 0; q < PER_THREAD; ++q) {
            const int id = tid + q * T::kThreads;
            const int r = id / CHUNKS_PER_ROW;
            const int c = id % CHUNKS_PER_ROW;
            const int sw = swz(r);
            // units 2c and 2c+1 sit side by side at unit (2c ^ sw) & ~1, swapped when sw is odd
            int4v v = *reinterpret_cast<const int4v *>(ct + r * BN + 4 * ((2 * c ^ sw) & ~1));
            if (sw & 1)
                v = int4v{v[2], v[3], v[0], v[1]};
            const int n = n0 + 8 * c;
            const uint32_t off = ((uint32_t)r * (uint32_t)N + (uint32_t)n) * 2u;
            __builtin_amdgcn_raw_buffer_store_b128(v, c_rsrc, off | oob_unless(n < N), 0, GEMM_F16_C_CPOL);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
        const int r = row_of(i);                             // row inside the panel
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
#pragma unroll
            for (int g = 0; g < GROUPS; ++g) {
                const int n = n0 + col_of(j, g);
                half_t h0, h1, h2, h3;
                out4(i, j, g, h0, h1, h2, h3);
                const uint32_t off = ((uint32_t)r * (uint32_t)N + (uint32_t)n) * 2u;
                if (vec_c == 4) {
                    // N % 4 == 0: the four columns are all inside or all outside
                    half4 h = {h0, h1, h2, h3};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(int2v, h), c_rsrc,
                                                          off | oob_unless(n < N), 0, GEMM_F16_C_CPOL);
                } else {
                    const short hs[4] = {__builtin_bit_cast(short, h0), __builtin_bit_cast(short, h1),
                                         __builtin_bit_cast(short, h2), __builtin_bit_cast(short, h3)};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b16(hs[e], c_rsrc,
                                                              (off + 2u * e) | oob_unless(n + e < N), 0,
                                                              GEMM_F16_C_CPOL);
                }
            }
        }
    }
}

// ---- persistent tile loop -------------------------------------------------------
// The 256x256x64 tile of 16x16x32 MFMAs (4 waves of 128x128, two LDS stages)
// run by one resident workgroup per CU over a sequence of output tiles.
// Against one workgroup per tile it removes, per tile after a workgroup's
// first: the launch of a new workgroup, the pipeline fill (the next tile's
// first k slice is loaded while the current tile's last slice is
// multiplied) and the accumulator clearing (a tile's first MFMAs take a zero
// accumulator input).  The result leaves straight from the accumulators as
// 8-byte stores of four consecutive columns, so that the LDS stages stay
// free for the next tile's slices; those stores drain while the next tile's
// first slice is multiplied.
// Tile order: workgroups are handed to the 8 XCDs round-robin; XCD x owns a
// contiguous range of the grouped tile order (as in tile_coords) and its
// workgroups take that range's tiles in turn, so in every round the tiles
// running on one XCD are neighbours, as with one workgroup per tile.
// Requirements (checked by the planner): an even number of k slices (at
// least 2), no split, N % 4 == 0 and C 8-byte aligned.
// PLAIN: alpha 1 and no ReLU (the store path converts and stores only).
template <int VA, bool A_ROWS_K, bool B_ROWS_K, bool PLAIN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_f16_persistent_kernel(KernelArgs args)
{
    constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = 2, STAGES = 2, PARTS = 2;
    using T = Tile<BM, BN, BK, WM, WN, STAGES, true, VA, 8, A_ROWS_K, B_ROWS_K, false, true>;
    static_assert(T::KSTEP == 32 && BK / T::KSTEP == 2, "two 32-deep k steps per slice");
    __shared__ __attribute__((aligned(1024))) half_t lds[T::LDS_BYTES / 2];
    half_t *const As = lds;                                  // two A stages
    half_t *const Bs = lds + STAGES * T::A_STAGE;            // two B stages

    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / WN) * T::WTM;
    const int wn0 = (wave % WN) * T::WTN;
    const int nk = (K + BK - 1) / BK;

    // this workgroup's tiles: positions local, local + wgs, ... of its XCD's range
    constexpr int kXcds = 8;
    const int P = (int)gridDim.x;
    const int tiles = args.tiles_m * args.tiles_n;
    const int xcd = (int)blockIdx.x % kXcds, local = (int)blockIdx.x / kXcds;
    const int wgs = P / kXcds + (xcd < P % kXcds ? 1 : 0);
    const int per = tiles / kXcds, rem = tiles % kXcds;
    const int first = xcd * per + min(xcd, rem);
    const int count = per + (xcd < rem ? 1 : 0);
    auto coords = [&](int id, int &m0_, int &n0_) {
        const int width = args.group_m * args.tiles_n;
        const int group = id / width;
        const int first_m = group * args.group_m;
        const int gm = min(args.tiles_m - first_m, args.group_m);
        const int in_group = id - group * width;
        m0_ = (first_m + in_group % gm) * BM;
        n0_ = (in_group / gm) * BN;
    };
    int tl = local;
    if (tl >= count)
        return;
    int m0, n0;
    coords(first + tl, m0, n0);

    typename T::OpA opa;
    typename T::OpB opb;
    opa.init(args.A, A_ROWS_K ? K : M, m0, M, 0, K, tid, wave, lane);
    opb.init(args.B, B_ROWS_K ? K : N, n0, N, 0, K, tid, wave, lane);

    float4v acc[T::TM][T::TN];
    struct Frags {
        half8 x[T::TN];
        half8 y[T::TM];
    };
    Frags f0, f1;
    auto load_frags = [&](Frags &f, const half_t *as, const half_t *bs, int ks) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
            f.y[i] = opa.frag16(as, wm0 + 16 * i, ks, lane);
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
            f.x[j] = opb.frag16(bs, wn0 + 16 * j, ks, lane);
    };
    // ZERO: the tile's first k step, on a zero accumulator input
    auto mma = [&](const Frags &f, auto zero_c) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int jj = 0; jj < T::TN; ++jj) {
#if GEMM_F16_SNAKE
                const int j = (i & 1) ? T::TN - 1 - jj : jj;
#else
                const int j = jj;
#endif
                if constexpr (decltype(zero_c)::value)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.x[j], f.y[i], float4v{}, 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.x[j], f.y[i], acc[i][j], 0, 0, 0);
            }
    };
    using Zero = std::integral_constant<bool, true>;
    using Accumulate = std::integral_constant<bool, false>;
    // k-step placement as in the one-tile kernel's 16x16x32 tile
    constexpr int kMfmaPerStep = T::TM * T::TN;
    constexpr int kReadsPerStep = (A_ROWS_K ? 1 : 2) * T::TM + (B_ROWS_K ? 1 : 2) * T::TN;
    constexpr int kReadsPerMfma = GEMM_F16_M16_READS_PER_MFMA;
    constexpr int kReadEvery = GEMM_F16_M16_READ_EVERY;
    constexpr int kVmemEvery = GEMM_F16_M16_VMEM_EVERY;
    static_assert(kMfmaPerStep / kReadEvery * kReadsPerMfma >= kReadsPerStep, "every read has a slot");
    constexpr int PART_LOADS = (T::OpA::LOADS + T::OpB::LOADS) / PARTS;
    auto interleave = [&](int n_vmem) {
#pragma unroll
        for (int i = 0; i < kMfmaPerStep; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
#pragma unroll
            for (int r = 0; r < kReadsPerMfma; ++r)
                if (i % kReadEvery == 0 && (i / kReadEvery) * kReadsPerMfma + r < kReadsPerStep)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            if (i % kVmemEvery == 0 && i / kVmemEvery < n_vmem)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // one global load
        }
    };
    auto issue = [&](int kt, half_t *dst_a, half_t *dst_b, int part) __attribute__((always_inline)) {
        opa.issue(kt, dst_a, wave, part, PARTS);
        opb.issue(kt, dst_b, wave, part, PARTS);
    };
    // every wave's loads of the stage about to be read have landed (two
    // stages: all of them), its reads of the stage about to be refilled are
    // done, then the workgroup barrier
    auto slice_ready = [&]() {
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // One k slice read from stage (rd_a, rd_b) while slice `req` of the
    // operands' current tile is requested into (wr_a, wr_b), half with each
    // k step.  FIRST: the tile's first slice (no earlier k step pending; its
    // first step starts the accumulators from zero); otherwise f1 holds the
    // previous slice's last step.
    auto step = [&](auto first_c, const half_t *__restrict__ rd_a, const half_t *__restrict__ rd_b,
                    half_t *__restrict__ wr_a, half_t *__restrict__ wr_b, int req) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first_c)::value;
        issue(req, wr_a, wr_b, 0);
        load_frags(f0, rd_a, rd_b, 0);
        if constexpr (!FIRST)
            mma(f1, Accumulate{});
        interleave(PART_LOADS);
        __builtin_amdgcn_sched_barrier(0);
        issue(req, wr_a, wr_b, 1);
        load_frags(f1, rd_a, rd_b, 1);
        if constexpr (FIRST)
            mma(f0, Zero{});
        else
            mma(f0, Accumulate{});
        interleave(PART_LOADS);
        __builtin_amdgcn_sched_barrier(0);
    };

    const bool relu = args.relu != 0;
    const float alpha = args.alpha;
    const uint32_t row_pitch = (uint32_t)N * 2u;
    // Lane l holds, in block (i, j), columns 16 j + 4 (l / 16) .. +3 of row
    // 16 i + l % 16 of its wave's sub-tile.  Each store's offset is a row
    // part (range-checked against the tile's c_rows rows) plus a column part
    // that carries the out-of-range bit for columns past N (N % 4 == 0: four
    // columns are all inside or all outside).
    auto store_tile = [&](int tm0, int tn0) {
        const int c_rows = min(BM, M - tm0);
        const __amdgpu_buffer_rsrc_t c_rsrc =
            make_rsrc(args.C + (int64_t)tm0 * N, (uint32_t)c_rows * row_pitch);
        uint32_t col[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int n = tn0 + wn0 + 16 * j + 4 * (lane >> 4);
            col[j] = ((uint32_t)n * 2u) | oob_unless(n < N);
        }
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const uint32_t row = (uint32_t)(wm0 + 16 * i + (lane & 15)) * row_pitch;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
                if constexpr (!PLAIN) {
                    v0 *= alpha;
                    v1 *= alpha;
                    v2 *= alpha;
                    v3 *= alpha;
                    if (relu) {
                        v0 = __builtin_fmaxf(v0, 0.0f);
                        v1 = __builtin_fmaxf(v1, 0.0f);
                        v2 = __builtin_fmaxf(v2, 0.0f);
                        v3 = __builtin_fmaxf(v3, 0.0f);
                    }
                }
                // element conversions kept as scalars (see the one-tile epilogue)
                const half_t h0 = (half_t)v0, h1 = (half_t)v1, h2 = (half_t)v2, h3 = (half_t)v3;
                const half4 h = {h0, h1, h2, h3};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(int2v, h), c_rsrc, row + col[j], 0,
                                                      GEMM_F16_C_CPOL);
            }
        }
    };
    (void)relu;
    (void)alpha;

    half_t *const A0 = As, *const A1 = As + T::A_STAGE;
    half_t *const B0 = Bs, *const B1 = Bs + T::B_STAGE;
    // the first tile's slice 0 into stage 0 (every later tile's slice 0 is
    // requested by its predecessor's last slice)
    issue(0, A0, B0, 0);
    issue(0, A0, B0, 1);
    while (true) {
        const int tl_next = tl + wgs;
        const bool more = tl_next < count;
        int m0n = m0, n0n = n0;
        if (more)
            coords(first + tl_next, m0n, n0n);
        // slice 0 (stage 0), requesting slice 1 into stage 1
        slice_ready();
        step(Zero{}, A0, B0, A1, B1, 1);
        // slices 1 .. nk-1 in pairs (nk even): stage 1 then stage 0
        for (int kt = 1; kt < nk; kt += 2) {
            int req = kt + 1;
            if (req == nk && more) {
                // the tile's last slice requests the next tile's first one
                opa.set_tile(m0n);
                opb.set_tile(n0n);
                req = 0;
            }
            slice_ready();
            step(Accumulate{}, A1, B1, A0, B0, req);
            if (kt + 1 < nk) {
                slice_ready();
                step(Accumulate{}, A0, B0, A1, B1, kt + 2);
            }
        }
        mma(f1, Accumulate{});       // the tile's last k step
        store_tile(m0, n0);
        if (!more)
            break;
        tl = tl_next;
        m0 = m0n;
        n0 = n0n;
    }
    wait_vmcnt<0>();   // the last request's zero-filling loads land before the workgroup retires
}

// ---- launchers ----------------------------------------------------------------

template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool DIRECT, int VA, int VB, bool AR, bool BR,
          int SPREAD = 1, bool SPARSE = false, bool M16 = false>
static hipError_t launch_one(const KernelArgs &a, int64_t grid, hipStream_t stream)
{
    if constexpr (SPARSE) {
        // wide position loads when K % 64 == 0; the LDS-staged epilogue when
        // N % 8 == 0 and C is 16-byte aligned
        const bool wide = a.K % 64 == 0, staged = a.vec_c == 8;
#define GEMM_F16_SP(ST, WIDE)                                                                                     \
        hipLaunchKernelGGL(                                                                                      \
            (gemm_f16_kernel<BM, BN, BK, WM, WN, STAGES, DIRECT, VA, VB, AR, BR, SPREAD, SPARSE, M16, ST, WIDE>), \
            dim3((unsigned)grid), dim3(64 * WM * WN), 0, stream, a)
        if (staged && wide)
            GEMM_F16_SP(true, true);
        else if (staged)
            GEMM_F16_SP(true, false);
        else if (wide)
            GEMM_F16_SP(false, true);
        else
            GEMM_F16_SP(false, false);
#undef GEMM_F16_SP
        return hipGetLastError();
    }
    // one wave per SIMD holding a 128x128 accumulator (256 registers): each
    // epilogue path has a build of its own (with every path, the build would
    // spill around its epilogue): the staged fp16 stores for the common
    // unsplit, 16-byte-aligned case, the split-K partials, the direct stores
    constexpr bool FULL_ACC = !SPARSE && WM * WN == 4 && BM * BN == 256 * 256;
    if constexpr (FULL_ACC) {
        if (a.W == nullptr && a.vec_c == 8) {
            hipLaunchKernelGGL(
                (gemm_f16_kernel<BM, BN, BK, WM, WN, STAGES, DIRECT, VA, VB, AR, BR, SPREAD, SPARSE, M16, 1>),
                dim3((unsigned)grid), dim3(64 * WM * WN), 0, stream, a);
            return hipGetLastError();
        }
        if (a.W != nullptr)
            hipLaunchKernelGGL(
                (gemm_f16_kernel<BM, BN, BK, WM, WN, STAGES, DIRECT, VA, VB, AR, BR, SPREAD, SPARSE, M16, 2>),
                dim3((unsigned)grid), dim3(64 * WM * WN), 0, stream, a);
        else
            hipLaunchKernelGGL(
                (gemm_f16_kernel<BM, BN, BK, WM, WN, STAGES, DIRECT, VA, VB, AR, BR, SPREAD, SPARSE, M16, 3>),
                dim3((unsigned)grid), dim3(64 * WM * WN), 0, stream, a);
        return hipGetLastError();
    } else {
        hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, BK, WM, WN, STAGES, DIRECT, VA, VB, AR, BR, SPREAD, SPARSE, M16>),
                           dim3((unsigned)grid), dim3(64 * WM * WN), 0, stream, a);
        return hipGetLastError();
    }
}

// the persistent tile loop: `grid` resident workgroups (at most one per CU)
template <int VA, bool AR, bool BR>
static hipError_t launch_persistent(const KernelArgs &a, int64_t grid, hipStream_t stream)
{
    if (a.alpha == 1.0f && a.relu == 0)
        hipLaunchKernelGGL((gemm_f16_persistent_kernel<VA, AR, BR, true>), dim3((unsigned)grid), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((gemm_f16_persistent_kernel<VA, AR, BR, false>), dim3((unsigned)grid), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

// register-staged kernels for every vector width (8, 4, 2 or 1 elements)
template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool AR, bool BR>
static hipError_t launch_staged(const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s)
{
#define GEMM_F16_VB(VA_)                                                                          \
    switch (vb) {                                                                                 \
    case 8: return launch_one<BM, BN, BK, WM, WN, STAGES, false, VA_, 8, AR, BR>(a, grid, s);     \
    case 4: return launch_one<BM, BN, BK, WM, WN, STAGES, false, VA_, 4, AR, BR>(a, grid, s);     \
    case 2: return launch_one<BM, BN, BK, WM, WN, STAGES, false, VA_, 2, AR, BR>(a, grid, s);     \
    default: return launch_one<BM, BN, BK, WM, WN, STAGES, false, VA_, 1, AR, BR>(a, grid, s);    \
    }
    switch (va) {
    case 8: GEMM_F16_VB(8)
    case 4: GEMM_F16_VB(4)
    case 2: GEMM_F16_VB(2)
    default: GEMM_F16_VB(1)
    }
#undef GEMM_F16_VB
}

// Register-staged tiles for the transposed layouts: 16-byte vectors when the
// pitch allows them, else single elements.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool AR, bool BR>
static hipError_t launch_staged_8or1(const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s)
{
    if (va == 8)
        return vb == 8 ? launch_one<BM, BN, BK, WM, WN, STAGES, false, 8, 8, AR, BR>(a, grid, s)
                       : launch_one<BM, BN, BK, WM, WN, STAGES, false, 8, 1, AR, BR>(a, grid, s);
    return vb == 8 ? launch_one<BM, BN, BK, WM, WN, STAGES, false, 1, 8, AR, BR>(a, grid, s)
                   : launch_one<BM, BN, BK, WM, WN, STAGES, false, 1, 1, AR, BR>(a, grid, s);
}

// Configurations of the transposed layouts (A given K x M and/or B given N x K).
template <bool AR, bool BR>
hipError_t launch_transposed(int config, const KernelArgs &a, int va, int vb, int64_t grid,
                                    hipStream_t s)
{
    switch (config) {
    case 0: return launch_one<256, 128, 64, 2, 2, 3, true, 8, 8, AR, BR, 1, false, true>(a, grid, s);
    case 1: return launch_one<256, 128, 64, 2, 2, 3, true, 8, 8, AR, BR, 4>(a, grid, s);
    case 2: return launch_one<128, 128, 64, 2, 2, 3, true, 8, 8, AR, BR, 4>(a, grid, s);
    case 3: return launch_staged_8or1<128, 128, 32, 2, 2, 2, AR, BR>(a, va, vb, grid, s);
    case 4: return launch_staged_8or1<64, 64, 64, 2, 2, 2, AR, BR>(a, va, vb, grid, s);
    case 17: return launch_staged_8or1<128, 128, 64, 2, 2, 2, AR, BR>(a, va, vb, grid, s);
    case 5: return launch_one<256, 256, 64, 2, 4, 2, true, 8, 8, AR, BR, 2>(a, grid, s);
    case 8: return launch_one<256, 256, 64, 2, 2, 2, true, 8, 8, AR, BR, GEMM_F16_M16_SPREAD, false, true>(a, grid, s);
    case 10: return launch_one<256, 256, 32, 2, 2, 4, true, 8, 8, AR, BR, 1, false, true>(a, grid, s);
    case 11: return launch_persistent<8, AR, BR>(a, grid, s);
    case 12: return launch_one<64, 64, 64, 2, 2, 4, true, 8, 8, AR, BR, 1>(a, grid, s);
    case 13: return launch_one<128, 128, 64, 2, 2, 4, true, 8, 8, AR, BR, 1, false, true>(a, grid, s);
    case 14: return launch_one<128, 64, 64, 2, 2, 4, true, 8, 8, AR, BR, 1>(a, grid, s);
    // rows only 4-byte aligned: 6 = 0, 7 = 14, 9 = 8, 15 = 13, 16 = 12
    case 6: return launch_one<256, 128, 64, 2, 2, 3, true, 2, 2, AR, BR, 1, false, true>(a, grid, s);
    case 7: return launch_one<128, 64, 64, 2, 2, 4, true, 2, 2, AR, BR, 1>(a, grid, s);
    case 9: return launch_one<256, 256, 64, 2, 2, 2, true, 2, 2, AR, BR, GEMM_F16_M16_SPREAD, false, true>(a, grid, s);
    case 15: return launch_one<128, 128, 64, 2, 2, 4, true, 2, 2, AR, BR, 1, false, true>(a, grid, s);
    case 16: return launch_one<64, 64, 64, 2, 2, 4, true, 2, 2, AR, BR, 1>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace gemm_f16_impl

#endif

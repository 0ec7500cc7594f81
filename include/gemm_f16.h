/*
 * gemm_f16.h -- C ABI of the tiled FP16 GEMM library for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation is the tiled GEMM that the TileLang pages use as their main
 * example ("TileLang：比 Triton 低一层的 tile 语言", section
 * "第一个 kernel：GEMM"; "5分钟上手TileLang：GPU内核开发指南", section
 * "安装与第一个内核"):
 *
 *     C[M x N] = epi( A[M x K] . B[K x N] )
 *
 * with binary16 operands, products accumulated in fp32 registers over a
 * pipelined K loop, an optional fused ReLU epilogue max(C, 0) applied to the
 * fp32 accumulator ("TileLang：让GPU编程像Python一样简单的高性能计算新范式",
 * section "并行计算的优雅表达"), and one round-to-nearest-even conversion to
 * binary16 in the final copy ("5分钟上手TileLang：GPU内核开发指南", section
 * "避坑与调参").  As on the pages, the caller provides A and B and receives C;
 * here the caller also owns C's memory.
 *
 * Layout: A, B and C are dense, row-major, contiguous device arrays of IEEE
 * binary16 (lda = K, ldb = N, ldc = N).  Pointers need only 2-byte
 * alignment; 16-byte alignment of the pointers and of the row pitches (K and
 * N multiples of 8) selects the fastest kernels, other shapes run a slower
 * path that gives the same results (never an error).
 *
 * Ownership: all buffers belong to the caller.  The library allocates no
 * device memory, keeps no per-call state and never synchronises with the
 * host or the stream; it is safe to call from several host threads.
 *
 * Split-K: when a problem has too few output tiles to fill the GPU's 256
 * CUs, the K loop of each tile may be divided into `splits` ranges run by
 * separate workgroups (a fixed-order form of the persistent / stream-K
 * scheduling that "5分钟上手TileLang：GPU内核开发指南", section
 * "进阶方向：从 GEMM 到真实模型算子", lists among the GEMM variants).  Each
 * range writes fp32 partial sums to a workspace of splits x M x N fp32 that
 * the caller passes to gemm_f16_split; a second kernel adds the partials in
 * split order, applies the epilogue and rounds once to binary16.  gemm_f16,
 * gemm_f16_ex and gemm_f16_trans take no workspace and always run one
 * kernel over the whole of K; gemm_f16_plan_split says whether, and with how
 * large a workspace, a split would pay for a shape.
 *
 * Execution: asynchronous on the given HIP stream (a hipStream_t passed as
 * void*; NULL is the default stream), so every entry point may be captured
 * into a HIP graph.  The result is deterministic: no atomics, and split
 * partials are added in a fixed order, so it is bitwise reproducible run to
 * run for a given shape, kernel configuration and split count.
 *
 * Errors: arguments are validated before any HIP call; on error nothing is
 * launched and C is untouched.  A launch error is reported as
 * GEMM_F16_ERROR_LAUNCH_FAILED.  Faults during execution surface at the
 * caller's next synchronisation, as with any HIP work.  No C++ exception
 * crosses this interface.
 */
#ifndef GEMM_F16_H
#define GEMM_F16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gemm_f16_status {
    GEMM_F16_SUCCESS = 0,
    /* negative dimension, null pointer with a nonzero extent, unknown
     * epilogue or configuration, C overlapping A or B */
    GEMM_F16_ERROR_INVALID_VALUE = 1,
    /* a pointer that is not 2-byte aligned (a caller's split-K workspace:
     * not 16-byte aligned) */
    GEMM_F16_ERROR_MISALIGNED = 2,
    /* no HIP device is visible */
    GEMM_F16_ERROR_NO_DEVICE = 3,
    /* the current device is not gfx950 */
    GEMM_F16_ERROR_UNSUPPORTED_DEVICE = 4,
    /* the kernel launch itself failed */
    GEMM_F16_ERROR_LAUNCH_FAILED = 5,
    /* a dimension beyond the library's limits (see GEMM_F16_MAX_*) */
    GEMM_F16_ERROR_UNSUPPORTED_SIZE = 6,
    /* gemm_f16_split: the plan splits K but no workspace was given, or the
     * caller's workspace is smaller than the plan's workspace_bytes */
    GEMM_F16_ERROR_WORKSPACE = 7,
    /* a HIP runtime call other than a launch failed */
    GEMM_F16_ERROR_RUNTIME = 8,
    /* gemm_f16_split_static: the plan's workspace_bytes exceeds
     * GEMM_F16_STATIC_WORKSPACE_BYTES */
    GEMM_F16_ERROR_SCRATCH_LIMIT = 9
} gemm_f16_status_t;

typedef enum gemm_f16_epilogue {
    GEMM_F16_EPILOGUE_NONE = 0,   /* C = rne16(A . B) */
    GEMM_F16_EPILOGUE_RELU = 1    /* C = rne16(max(A . B, 0)); -0 becomes +0 */
} gemm_f16_epilogue_t;

/* Size limits.  Every global access goes through a buffer range of at most
 * 2 GiB addressed with 32-bit byte offsets: the panel of at most 256 rows of
 * A (stored M x K), of B (stored N x K) or of C that one workgroup touches,
 * and the k slice of at most 64 rows of A (stored K x M) or of B (stored
 * K x N) that one pipeline stage loads.  Hence K and N at most 2^22 (256
 * rows of pitch K or N), M at most 2^24 when A is stored K x M (64 rows of
 * pitch M), M at most 2^31 - 1 otherwise, and at most 2^31 - 1 workgroups.
 * Larger shapes return GEMM_F16_ERROR_UNSUPPORTED_SIZE. */
#define GEMM_F16_MAX_DIM ((int64_t)2147483647)
#define GEMM_F16_MAX_K ((int64_t)1 << 22)
#define GEMM_F16_MAX_N ((int64_t)1 << 22)
#define GEMM_F16_MAX_M_TRANS_A ((int64_t)1 << 24)

/* Automatic kernel choice for gemm_f16_ex / gemm_f16_plan. */
#define GEMM_F16_CONFIG_AUTO (-1)

/* Automatic split count for gemm_f16_split / gemm_f16_plan_split (the
 * measured table or the time model decides; 1 when a split does not pay),
 * and the largest count accepted. */
#define GEMM_F16_SPLITS_AUTO 0
#define GEMM_F16_MAX_SPLITS 64

/*
 * C = epi(A . B) for A (M x K), B (K x N), C (M x N), all binary16 row-major.
 *   M, N, K   : dimensions, >= 0.  M == 0 or N == 0: nothing to do (success,
 *               no launch).  K == 0: C is filled with +0 (the empty sum).
 *   A, B      : device pointers (read only); may be NULL only when the
 *               matrix has no elements.
 *   C         : device pointer (written); must not overlap A or B.
 *   epilogue  : a gemm_f16_epilogue_t value.
 *   stream    : hipStream_t, or NULL for the default stream.
 * Returns GEMM_F16_SUCCESS once the work is enqueued.
 */
gemm_f16_status_t gemm_f16(int64_t M, int64_t N, int64_t K,
                           const void *A, const void *B, void *C,
                           int epilogue, void *stream);

/*
 * As gemm_f16, with an explicit kernel configuration: an index in
 * [0, gemm_f16_num_configs()) or GEMM_F16_CONFIG_AUTO.  A configuration that
 * cannot run this shape or alignment (gemm_f16_plan says why) returns
 * GEMM_F16_ERROR_INVALID_VALUE.  Runs unsplit (one kernel, no workspace),
 * like gemm_f16.  Intended for tests and tuning sweeps; every configuration
 * computes the same function.
 */
gemm_f16_status_t gemm_f16_ex(int64_t M, int64_t N, int64_t K,
                              const void *A, const void *B, void *C,
                              int epilogue, int config, void *stream);

/*
 * C = epi(op(A) . op(B)) with either operand given transposed: the
 * "transpose_B" form of the pages' tile GEMM ("TileLang：比 Triton 低一层的
 * tile 语言", section "FlashAttention：在线 softmax 写成 tile 代码", where the
 * score block is Q . K^T) and its A-side counterpart.
 *   trans_a = 0: A is M x K row-major (lda = K); 1: A is stored K x M
 *                row-major (lda = M) and op(A) = A^T.
 *   trans_b = 0: B is K x N row-major (ldb = N); 1: B is stored N x K
 *                row-major (ldb = K) and op(B) = B^T.
 * Other arguments, ownership and errors as gemm_f16_ex (config may be
 * GEMM_F16_CONFIG_AUTO).  Transposed layouts run on a subset of the
 * configurations; a trans flag other than 0 or 1 is INVALID_VALUE.
 */
gemm_f16_status_t gemm_f16_trans(int64_t M, int64_t N, int64_t K,
                                 const void *A, int trans_a, const void *B, int trans_b,
                                 void *C, int epilogue, int config, void *stream);

/*
 * C = epi(op(A) . op(B)) with an explicit K split (layouts as
 * gemm_f16_trans).
 *   config          : a configuration index or GEMM_F16_CONFIG_AUTO.
 *   splits          : GEMM_F16_SPLITS_AUTO, or 1 .. GEMM_F16_MAX_SPLITS.  The
 *                     count is rounded down so that no split is empty and
 *                     every split spans whole K tiles (gemm_f16_plan_split
 *                     reports the count used; 1 means one kernel and no
 *                     workspace).  The persistent configuration takes no
 *                     split: a count above 1 with it is INVALID_VALUE.
 *   workspace       : a caller-owned device buffer of workspace_bytes
 *                     bytes, 16-byte aligned, overlapping none of A, B, C,
 *                     and at least the plan's workspace_bytes long.  NULL
 *                     (with workspace_bytes 0) is accepted only when the
 *                     plan does not split; otherwise, as for a buffer that is
 *                     too small, GEMM_F16_ERROR_WORKSPACE is returned before
 *                     anything is launched.  Its contents are scratch; calls
 *                     that share one buffer must be ordered (one stream).
 *   workspace_bytes : size of the caller's buffer; 0 when workspace is NULL.
 * Other arguments and errors as gemm_f16_trans.
 */
gemm_f16_status_t gemm_f16_split(int64_t M, int64_t N, int64_t K,
                                 const void *A, int trans_a, const void *B, int trans_b,
                                 void *C, int epilogue, int config, int splits,
                                 void *workspace, int64_t workspace_bytes, void *stream);

/*
 * C = epi(alpha * (op(A) . op(B))): the fp32 result block is multiplied by
 * alpha (an fp32 value) before the epilogue and the single rounding to
 * binary16.  This is the scaling the pages apply to the score block of the
 * transpose_B product, Q . K^T, before anything else touches it
 * ("TileLang：比 Triton 低一层的 tile 语言", section "FlashAttention：在线
 * softmax 写成 tile 代码").  With epilogue RELU the result is
 * rne16(max(alpha * sum, 0)).  alpha = 1 gives exactly gemm_f16_trans's
 * result; any alpha is accepted (IEEE arithmetic for NaN or inf).  Other
 * arguments, layouts and errors as gemm_f16_trans (runs unsplit).
 */
gemm_f16_status_t gemm_f16_scaled(int64_t M, int64_t N, int64_t K,
                                  const void *A, int trans_a, const void *B, int trans_b,
                                  void *C, float alpha, int epilogue, int config, void *stream);

/* gemm_f16_split with the scale of gemm_f16_scaled (applied by the
 * reduction to the sum of the partials, in fp32). */
gemm_f16_status_t gemm_f16_split_scaled(int64_t M, int64_t N, int64_t K,
                                        const void *A, int trans_a, const void *B, int trans_b,
                                        void *C, float alpha, int epilogue, int config, int splits,
                                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gemm_f16_split without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the fp32 partial sums go to a static
 * device array of GEMM_F16_STATIC_WORKSPACE_BYTES that the library holds on
 * each GPU it runs on from module load until the process ends.  The call
 * allocates and frees nothing and does not synchronise; the first call on a
 * device looks up that device's copy of the array.
 *   Arguments, layouts and splits as gemm_f16_split.  A plan whose
 *   workspace_bytes (gemm_f16_plan_split) exceeds the array returns
 *   GEMM_F16_ERROR_SCRATCH_LIMIT before anything is launched.
 *   Every call on one GPU uses the same array and leaves its last contents
 *   there (no part of it needs to start at zero: each partial sum is written
 *   before it is read).  Calls that may overlap on one GPU -- on different
 *   streams, or from several host threads without ordering -- race on it;
 *   order them on one stream.
 */
#define GEMM_F16_STATIC_WORKSPACE_BYTES ((int64_t)32 << 20)
gemm_f16_status_t gemm_f16_split_static(int64_t M, int64_t N, int64_t K,
                                        const void *A, int trans_a, const void *B, int trans_b,
                                        void *C, int epilogue, int config, int splits, void *stream);

/*
 * 2:4 structured-sparse A.  The pages name 2:4 sparse GEMM (`T.gemm_sp`)
 * among TileLang's features ("TileLang：让GPU编程像Python一样简单的高性能计算
 * 新范式", section "高级特性超越基础矩阵乘法") without a storage format; this
 * library's format, matched to gfx950's v_smfmac_f32_32x32x32_f16:
 *   vals : M x K/2 binary16, row-major: in every aligned group of 4
 *          consecutive k of a row, the 2 kept values in position order.
 *   meta : M K/16 uint16 words.  Word w of row i covers k = 16w .. 16w+15;
 *          bits 2s+1..2s give the position (0..3) inside group 4w + s/2 of
 *          kept value s (s = 0..7), i.e. vals[i][8w + s] sits at
 *          k = 16w + 4 (s/2) + position.  The words are stored by 64-deep
 *          k slices, so that a slice's words of consecutive rows are
 *          contiguous: with kw = K/16 and F = kw / 4 whole slices, word w of
 *          row i is at index (w/4 * M + i) * 4 + w % 4 when w/4 < F, and at
 *          F * M * 4 + i * (kw % 4) + w % 4 in the partial last slice.
 * K must be a multiple of 16.
 */

/*
 * Compress A (M x K binary16, row-major, on the device) into vals and meta
 * (device buffers of M*K/2 halves and M*K/16 words, caller-owned, not
 * overlapping A or each other): in each group of 4 the 2 entries of largest
 * magnitude are kept (magnitudes compared exactly; ties: lower position).
 * An already 2:4-sparse A is kept exactly.  Asynchronous on `stream`.
 * K % 16 != 0 or a negative dimension: GEMM_F16_ERROR_INVALID_VALUE;
 * odd pointers: GEMM_F16_ERROR_MISALIGNED.
 */
gemm_f16_status_t gemm_f16_sp_compress(int64_t M, int64_t K, const void *A, void *vals, void *meta,
                                       void *stream);

/*
 * C = epi(A . op(B)) with A given as (vals, meta) above and C M x N binary16
 * row-major; op(B) = B (K x N, trans_b = 0) or B^T (B stored N x K,
 * trans_b = 1).  Products of kept values accumulate in fp32; one RNE
 * rounding to binary16 at the end, as gemm_f16.
 *   config : GEMM_F16_CONFIG_AUTO or an index < gemm_f16_sp_num_configs().
 * Requirements: K % 16 == 0 (else INVALID_VALUE); vals and B 16-byte
 * aligned and (trans_b = 0) N % 8 == 0, meta and C 2-byte aligned (else
 * MISALIGNED); C must not overlap vals, meta or B.  Other rules as gemm_f16.
 */
gemm_f16_status_t gemm_f16_sp(int64_t M, int64_t N, int64_t K, const void *vals, const void *meta,
                              const void *B, int trans_b, void *C, int epilogue, int config, void *stream);

/* Number and names of the sparse kernel configurations. */
int gemm_f16_sp_num_configs(void);
const char *gemm_f16_sp_config_name(int config);

/* How a call would run; filled by gemm_f16_plan without any HIP call. */
typedef struct gemm_f16_plan {
    int32_t config;        /* configuration index actually chosen */
    int32_t block_m;       /* output tile rows per workgroup (bM) */
    int32_t block_n;       /* output tile columns per workgroup (bN) */
    int32_t block_k;       /* K depth of one LDS stage (bK) */
    int32_t stages;        /* LDS ring-buffer stages */
    int32_t threads;       /* threads per workgroup */
    int32_t direct_lds;    /* 1: operands go global -> LDS without registers */
    int32_t vec_a;         /* alignment of A's rows the kernel relies on, in binary16
                              elements: the width of its global loads (register-staged),
                              or 8 / 2 for 16-byte / 4-byte aligned rows (direct_lds,
                              whose loads always move 16-byte chunks) */
    int32_t vec_b;         /* the same for B */
    int32_t vec_c;         /* binary16 elements per store of C */
    int64_t tiles_m;       /* ceil(M / bM) */
    int64_t tiles_n;       /* ceil(N / bN) */
    int64_t grid;          /* workgroups launched: tiles_m * tiles_n * splits, or for a
                              persistent configuration min(tiles_m * tiles_n, 256 CUs) */
    int64_t k_tiles;       /* K-loop trip count of one workgroup: ceil(k_split / bK) */
    int64_t lds_bytes;     /* LDS per workgroup */
    double flops;          /* 2 M N K: the algorithmic work of the call */
    double min_bytes;      /* 2 (M K + K N + M N): operands read once, C written once */
    int32_t trans_a;       /* 1: A stored K x M */
    int32_t trans_b;       /* 1: B stored N x K */
    int32_t splits;        /* K splits (1: unsplit, no reduction kernel) */
    int64_t k_split;       /* K elements per split (K when unsplit) */
    int64_t workspace_bytes; /* splits * M * N * 4 when split, else 0 */
} gemm_f16_plan_t;

/*
 * Describe the kernel a call of gemm_f16 / gemm_f16_ex with these arguments
 * would launch (config may be GEMM_F16_CONFIG_AUTO; the plan never splits).
 * Pointers are used only for alignment checks and may be NULL-but-aligned
 * stand-ins (any multiple of 16) when only the shape matters.  Pure host
 * logic: no HIP call, no GPU needed.
 */
gemm_f16_status_t gemm_f16_plan(int64_t M, int64_t N, int64_t K,
                                const void *A, const void *B, const void *C,
                                int config, gemm_f16_plan_t *plan);

/* As gemm_f16_plan, for the layouts of gemm_f16_trans. */
gemm_f16_status_t gemm_f16_plan_trans(int64_t M, int64_t N, int64_t K,
                                      const void *A, int trans_a, const void *B, int trans_b,
                                      const void *C, int config, gemm_f16_plan_t *plan);

/* As gemm_f16_plan, for gemm_f16_sp (config indexes the sparse list; flops
 * counts the products of kept values, M N K; lds_bytes the compressed A, the
 * B and the position-word stages). */
gemm_f16_status_t gemm_f16_plan_sp(int64_t M, int64_t N, int64_t K, const void *vals, const void *meta,
                                   const void *B, int trans_b, const void *C, int config,
                                   gemm_f16_plan_t *plan);

/* As gemm_f16_plan_trans, for gemm_f16_split with the given split request
 * (GEMM_F16_SPLITS_AUTO: the split the measured table or the time model
 * prefers, with the workspace_bytes the caller must then provide). */
gemm_f16_status_t gemm_f16_plan_split(int64_t M, int64_t N, int64_t K,
                                      const void *A, int trans_a, const void *B, int trans_b,
                                      const void *C, int config, int splits, gemm_f16_plan_t *plan);

/* Number of kernel configurations compiled into the library. */
int gemm_f16_num_configs(void);

/* Short human-readable name of a configuration ("256x256x64_s2_direct", ...)
 * or NULL for an index out of range.  The string is static. */
const char *gemm_f16_config_name(int config);

/*
 * LDS bytes that `stages` ring-buffer stages of an unpadded bM x bK A tile
 * and bK x bN B tile of binary16 occupy: stages * 2 * bK * (bM + bN).  This
 * is the shared-memory budget of the pages' worked exercise
 * ("TileLang：比 Triton 低一层的 tile 语言", section "练习", exercises 1-2);
 * the library's LDS layouts are swizzled, not padded, so their footprint is
 * exactly this.  Returns -1 for negative arguments.
 */
int64_t gemm_f16_stage_bytes(int64_t block_m, int64_t block_n, int64_t block_k,
                             int64_t stages);

/* Static English description of a status code. */
const char *gemm_f16_status_string(gemm_f16_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_H */

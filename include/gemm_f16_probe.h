/*
 * gemm_f16_probe.h -- measurement probe shipped with the FP16 GEMM library
 * (libgemm_f16_probe.so).  Not part of the GEMM itself.
 *
 * It runs the GEMM kernels' inner-loop instruction mix -- per wave a 4 x 4
 * block of v_mfma_f32_32x32x16_f16 on 16 fp32 accumulator tiles, one wave
 * per SIMD -- with register operands only and no memory traffic, to measure
 * the matrix-core throughput the GPU sustains for a kind of operand data.
 * The pages ask for the roofline to be worked out before tuning and compared
 * with measurement ("TileLang：比 Triton 低一层的 tile 语言", section
 * "工程上的几个注意点"); on MI355X the sustained MFMA clock depends on the
 * data, so this gives the measured ceiling next to the nominal one.
 */
#ifndef GEMM_F16_PROBE_H
#define GEMM_F16_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Operand kinds. */
#define GEMM_F16_PROBE_CONSTANT 0          /* the same constant bits in every fragment */
#define GEMM_F16_PROBE_RANDOM_FIXED 1      /* random halves, one fragment set reused */
#define GEMM_F16_PROBE_RANDOM_CHANGING 2   /* random halves, two fragment sets alternating,
                                              as the GEMM's k steps do */
/* Added to a kind: the same work with v_mfma_f32_16x16x32_f16 (an 8 x 8 block
 * of 16x16 tiles per wave) instead of 32x32x16. */
#define GEMM_F16_PROBE_MFMA16 3

/* Number of 8-half (16-byte) vectors the `operands` buffer must hold. */
#define GEMM_F16_PROBE_OPERAND_VECTORS 1024

/*
 * Enqueue the probe on `stream` (a hipStream_t, NULL = default stream).
 *   mode     : one of the GEMM_F16_PROBE_* kinds, plus GEMM_F16_PROBE_MFMA16
 *              for the 16x16x32 instruction.
 *   iters    : loop trips; each trip issues 32 MFMAs per wave.
 *   blocks   : workgroups of 256 threads (use a multiple of the CU count).
 *   operands : device buffer of GEMM_F16_PROBE_OPERAND_VECTORS x 8 binary16
 *              values (ignored for GEMM_F16_PROBE_CONSTANT).
 *   out      : device buffer of blocks x 256 floats (written, to keep the
 *              work observable).
 *   flops    : if not NULL, receives the flops the launch performs.
 * Returns 0 on success, 1 for bad arguments, 2 if the launch failed.
 * Buffers belong to the caller; the call is asynchronous.
 */
int gemm_f16_probe_mfma(int mode, int iters, int64_t blocks, const void *operands, void *out,
                        void *stream, double *flops);

/*
 * Lane-layout probe: one wave of 64 lanes runs one matrix instruction with a
 * zero accumulator on operands given per lane, and writes every lane's
 * accumulators, so that tests can check the operand and result layouts the
 * GEMM kernels are written against.
 *   instr : GEMM_F16_PROBE_LAYOUT_* below.
 *   src0  : 64 x 8 binary16, lane l's first operand (for the sparse
 *           instruction: its 8 kept values).
 *   src1  : lane l's second operand, 64 x 8 binary16 (64 x 16 for the sparse
 *           instruction).
 *   index : 64 int32, lane l's position word (sparse instruction only; may
 *           be NULL otherwise).
 *   out   : 64 x 16 floats (32x32 results) or 64 x 4 (16x16), lane-major.
 * Returns 0 on success, 1 for bad arguments, 2 if the launch failed.
 */
#define GEMM_F16_PROBE_LAYOUT_32X32X16 0         /* v_mfma_f32_32x32x16_f16 */
#define GEMM_F16_PROBE_LAYOUT_16X16X32 1         /* v_mfma_f32_16x16x32_f16 */
#define GEMM_F16_PROBE_LAYOUT_SMFMAC_32X32X32 2  /* v_smfmac_f32_32x32x32_f16 */
int gemm_f16_probe_mfma_layout(int instr, const void *src0, const void *src1, const void *index, void *out,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_PROBE_H */

"""The matrix-instruction lane layouts the GEMM kernels are written against,
checked on the GPU through the layout probe (include/gemm_f16_probe.h).

Each instruction runs once on small-integer binary16 operands placed per
lane as the kernels assume; the result of every lane must equal, exactly,
the matrix product of the operands assembled under that assumption.  The
kernels depend on these layouts for
  * v_mfma_f32_32x32x16_f16: first operand lane l = row l % 32, k 8 (l / 32)
    .. +7; second operand lane l = column l % 32, same k; result lane l =
    column l % 32, rows 8 g + 4 (l / 32) + r in accumulator 4 g + r;
  * v_mfma_f32_16x16x32_f16: first operand lane l = row l % 16, k 8 (l / 16)
    .. +7; second operand lane l = column l % 16, same k; result lane l =
    column l % 16, rows 4 (l / 16) + r in accumulator r;
  * v_smfmac_f32_32x32x32_f16: first operand lane l = row l % 32, the 8 kept
    values of k 16 (l / 32) .. +15 with 2-bit positions in the low 16 bits of
    the lane's index word; second operand lane l = column l % 32, k 8 (l / 32)
    .. +7 then 16 + 8 (l / 32) .. +7; result as the 32x32x16 instruction.
A further case checks that subnormal binary16 inputs are not flushed.
"""
import numpy as np
import pytest
import torch

import tiled_dense_gemm_fp16_amd as g

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run(instr, src0, src1, index=None, n_out=16):
    a = torch.from_numpy(np.ascontiguousarray(src0.astype(np.float16))).to(DEV)
    b = torch.from_numpy(np.ascontiguousarray(src1.astype(np.float16))).to(DEV)
    idx = torch.from_numpy(np.ascontiguousarray(index.astype(np.int32))).to(DEV) if index is not None else None
    out = torch.full((64, n_out), float("nan"), dtype=torch.float32, device=DEV)
    st = g.probe_lib().gemm_f16_probe_mfma_layout(instr, a.data_ptr(), b.data_ptr(),
                                                  idx.data_ptr() if idx is not None else None, out.data_ptr(),
                                                  torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_mfma_32x32x16_layout():
    rng = np.random.default_rng(1)
    s0 = rng.integers(-3, 4, size=(64, 8)).astype(np.float64)
    s1 = rng.integers(-3, 4, size=(64, 8)).astype(np.float64)
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for l in range(64):
        A[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = s0[l]
        B[8 * (l // 32):8 * (l // 32) + 8, l % 32] = s1[l]
    D = A @ B
    got = run(g.PROBE_LAYOUT_32X32X16, s0, s1, n_out=16)
    want = np.array([[D[8 * (e // 4) + 4 * (l // 32) + e % 4, l % 32] for e in range(16)] for l in range(64)])
    assert np.array_equal(got, want)


def test_mfma_16x16x32_layout():
    rng = np.random.default_rng(2)
    s0 = rng.integers(-3, 4, size=(64, 8)).astype(np.float64)
    s1 = rng.integers(-3, 4, size=(64, 8)).astype(np.float64)
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    for l in range(64):
        A[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = s0[l]
        B[8 * (l // 16):8 * (l // 16) + 8, l % 16] = s1[l]
    D = A @ B
    got = run(g.PROBE_LAYOUT_16X16X32, s0, s1, n_out=4)
    want = np.array([[D[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(64)])
    assert np.array_equal(got, want)


def test_smfmac_32x32x32_layout():
    rng = np.random.default_rng(3)
    vals = rng.integers(-3, 4, size=(64, 8)).astype(np.float64)
    s1 = rng.integers(-3, 4, size=(64, 16)).astype(np.float64)
    # two distinct positions, in increasing order, for each kept pair
    index = np.zeros(64, dtype=np.int64)
    A = np.zeros((32, 32))
    for l in range(64):
        word = 0
        for q in range(4):
            lo, hi = sorted(rng.choice(4, size=2, replace=False))
            word |= int(lo) << (4 * q)
            word |= int(hi) << (4 * q + 2)
            A[l % 32, 16 * (l // 32) + 4 * q + lo] = vals[l, 2 * q]
            A[l % 32, 16 * (l // 32) + 4 * q + hi] = vals[l, 2 * q + 1]
        index[l] = word
    B = np.zeros((32, 32))
    for l in range(64):
        B[8 * (l // 32):8 * (l // 32) + 8, l % 32] = s1[l, :8]
        B[16 + 8 * (l // 32):16 + 8 * (l // 32) + 8, l % 32] = s1[l, 8:]
    D = A @ B
    got = run(g.PROBE_LAYOUT_SMFMAC_32X32X32, vals, s1, index=index, n_out=16)
    want = np.array([[D[8 * (e // 4) + 4 * (l // 32) + e % 4, l % 32] for e in range(16)] for l in range(64)])
    assert np.array_equal(got, want)


def test_subnormal_inputs_are_kept():
    # 2^-24 (the smallest binary16 subnormal) times 1 over all 32 k: 32 * 2^-24 = 2^-19
    s0 = np.full((64, 8), 2.0 ** -24)
    s1 = np.ones((64, 8))
    got = run(g.PROBE_LAYOUT_16X16X32, s0, s1, n_out=4)
    assert np.all(got == 2.0 ** -19)
    # a subnormal times a subnormal underflows in binary16 but not in the fp32 accumulator
    s0 = np.full((64, 8), 2.0 ** -14)
    s1 = np.full((64, 8), 2.0 ** -20)        # subnormal binary16
    got = run(g.PROBE_LAYOUT_32X32X16, s0, s1, n_out=16)
    assert np.all(got == 16 * 2.0 ** -34)

"""Pins for the oracle GEMM against facts that do not come from the oracle.

The product it must compute is the tiled GEMM of
"TileLang：比 Triton 低一层的 tile 语言" (section "第一个 kernel：GEMM"):
C = A . B with fp16 operands, a wide accumulator and one fp16 rounding at
the end, plus the fused ReLU of
"TileLang：让GPU编程像Python一样简单的高性能计算新范式" (section
"并行计算的优雅表达").  The pages print no output values, so the oracle is
pinned by:

* exact rational brute force on tiny shapes (bit-exact);
* identity and permutation matrices (exact copies / permutations);
* integer-valued operands, whose product is an exact integer (numpy int64);
* invariants: transposition, scaling by two, ReLU = max(C, 0), sampled
  block = block of the full product, K = 0 is the empty sum;
* the first two moments of C for each input distribution.

A dropped term, a wrong sign, a swapped index or a transposed operand fails
at least one of these.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fractions import Fraction

from tests import brute_force


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def exact_range_operands(rng, shape):
    """binary16 values with exponent in [-8, 0] and random sign: sums of up to
    a few hundred of their products are exact in binary64."""
    mant = rng.integers(1024, 2048, size=shape)
    exp = rng.integers(-8, 1, size=shape)
    sign = rng.choice([-1.0, 1.0], size=shape)
    return f16_bits(sign * mant * np.exp2(exp - 10.0))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (3, 5, 2), (5, 8, 3), (8, 8, 8),
                                   (3, 2, 16), (2, 3, 100)])
@pytest.mark.parametrize("relu", [False, True])
def test_brute_force_exact(M, N, K, relu):
    rng = np.random.default_rng(M * 100 + N * 10 + K + relu)
    A = exact_range_operands(rng, (M, K))
    B = exact_range_operands(rng, (K, N))
    ref = brute_force.gemm(A, B, relu=relu)
    got = oracle.gemm(A, B, relu=relu)
    assert np.array_equal(got, ref)


def test_brute_force_full_range_with_subnormals():
    # binary16 operands including subnormals and values up to 128.  The fp64
    # sum may differ from the exact one by a few binary64 ulps, which can only
    # change the binary16 rounding for a sum within that distance of a tie;
    # this seeded sample has none, so the oracle must equal the exact rounding
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.integers(0x0001, 0x0400, 20),       # subnormals
                           rng.integers(0x0400, 0x5800, 60)]).astype(np.uint16)
    vals = vals | (rng.integers(0, 2, vals.size).astype(np.uint16) << 15)
    A = rng.choice(vals, (4, 6)).astype(np.uint16)
    B = rng.choice(vals, (6, 5)).astype(np.uint16)
    assert np.array_equal(oracle.gemm(A, B), brute_force.gemm(A, B))


def test_brute_force_overflow_to_inf():
    A = f16_bits([[60000.0, 60000.0]])
    B = f16_bits([[1.0], [1.0]])
    assert int(oracle.gemm(A, B)[0, 0]) == 0x7C00 == int(brute_force.gemm(A, B)[0, 0])


def test_identity_and_permutation():
    rng = np.random.default_rng(3)
    A, B = workloads.draw(37, 29, 37, "uniform", 11)
    A, B = bits(A), bits(B)
    I = f16_bits(np.eye(37))
    assert np.array_equal(oracle.gemm(I, B), B)                 # I . B = B
    I29 = f16_bits(np.eye(29))
    assert np.array_equal(oracle.gemm(B, I29), B)               # B . I = B
    p = rng.permutation(37)
    P = f16_bits(np.eye(37)[p])                                 # (P . B)[i] = B[p[i]]
    assert np.array_equal(oracle.gemm(P, B), B[p])
    q = rng.permutation(29)
    Q = f16_bits(np.eye(29)[:, q])                              # (B . Q)[:, j] = B[:, q[j]]
    assert np.array_equal(oracle.gemm(B, Q), B[:, q])
    # a negated identity flips every sign bit (except that 0 stays +0)
    nI = f16_bits(-np.eye(37))
    neg = oracle.gemm(nI, B)
    nz = (B & 0x7FFF) != 0
    assert np.array_equal(neg[nz], B[nz] ^ 0x8000)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (17, 33, 65), (64, 48, 300), (301, 129, 410)])
def test_integer_operands_exact(M, N, K):
    a, b = workloads.draw_ints(M, N, K, seed=M + N + K)
    exact = a.numpy().astype(np.int64) @ b.numpy().astype(np.int64)
    # |C| <= 4K < 2048 here, so every integer is a binary16 value: the exact result
    assert np.abs(exact).max() < 2048
    assert np.array_equal(oracle.gemm(bits(a), bits(b)), f16_bits(exact))


def test_integer_operands_large_rounding():
    # |C| up to ~1000..8000: above 2048 the binary16 spacing is 2 or 4, so the
    # exact integer must be rounded once, ties to even (numpy's int->f16 cast)
    a, b = workloads.draw_ints(12, 10, 2000, seed=5, lo=2, hi=2)
    exact = a.numpy().astype(np.int64) @ b.numpy().astype(np.int64)     # all 8000
    assert np.array_equal(oracle.gemm(bits(a), bits(b)), f16_bits(exact))
    a, b = workloads.draw_ints(9, 7, 3001, seed=6, lo=-1, hi=2)
    exact = a.numpy().astype(np.int64) @ b.numpy().astype(np.int64)
    assert np.array_equal(oracle.gemm(bits(a), bits(b)), f16_bits(exact))


def test_transpose_invariant():
    A, B = workloads.draw(23, 31, 47, "uniform", 2)
    A, B = bits(A), bits(B)
    C = oracle.gemm(A, B)
    CT = oracle.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(CT, C.T)


def test_transposed_operand_is_detected():
    # A (n x n) . B differs from A^T . B: catches an oracle that reads A by columns
    rng = np.random.default_rng(9)
    A = exact_range_operands(rng, (6, 6))
    B = exact_range_operands(rng, (6, 6))
    C = oracle.gemm(A, B)
    assert np.array_equal(C, brute_force.gemm(A, B))
    assert not np.array_equal(C, brute_force.gemm(np.ascontiguousarray(A.T), B))
    assert not np.array_equal(C, brute_force.gemm(A, np.ascontiguousarray(B.T)))


def test_scaling_by_two():
    A, B = workloads.draw(40, 50, 60, "uniform", 4)
    A, B = bits(A), bits(B)
    A2 = oracle.encode(2.0 * oracle.decode(A))                  # exact doubling
    C = oracle.gemm(A, B)
    C2 = oracle.gemm(A2, B)
    c = oracle.decode(C)
    normal = np.abs(c) >= 2.0 ** -13                            # both roundings in the normal range
    assert normal.mean() > 0.9
    assert np.array_equal(oracle.decode(C2)[normal], 2.0 * c[normal])


def test_relu_is_max_of_plain_result():
    A, B = workloads.draw(33, 45, 70, "uniform", 5)
    A, B = bits(A), bits(B)
    C = oracle.gemm(A, B)
    R = oracle.gemm(A, B, relu=True)
    neg = (C & 0x8000) != 0
    assert neg.any() and (~neg).any()
    assert np.array_equal(R[~neg], C[~neg])
    assert np.all(R[neg] == 0)                                  # +0, never -0


def test_sampled_block_equals_full_product_block():
    A, B = workloads.draw(60, 70, 90, "normal", 6)
    A, B = bits(A), bits(B)
    C = oracle.gemm(A, B)
    rows = np.array([59, 0, 17, 17, 3])
    cols = np.array([0, 69, 5, 33])
    S = oracle.gemm_sampled(A, B, rows, cols)
    assert np.array_equal(S, C[np.ix_(rows, cols)])
    with pytest.raises(RuntimeError):
        oracle.gemm_sampled(A, B, np.array([60]), cols)


def test_degenerate_shapes():
    A = np.zeros((4, 0), np.uint16)
    B = np.zeros((0, 3), np.uint16)
    assert np.array_equal(oracle.gemm(A, B), np.zeros((4, 3), np.uint16))      # empty sum = +0
    assert np.array_equal(oracle.gemm(A, B, relu=True), np.zeros((4, 3), np.uint16))
    assert oracle.gemm(np.zeros((0, 5), np.uint16), np.zeros((5, 3), np.uint16)).shape == (0, 3)
    assert oracle.gemm(np.zeros((2, 5), np.uint16), np.zeros((5, 0), np.uint16)).shape == (2, 0)


def test_thread_count_does_not_change_bits():
    A, B = workloads.draw(97, 61, 130, "uniform", 8)
    A, B = bits(A), bits(B)
    one = oracle.gemm(A, B, threads=1)
    assert np.array_equal(one, oracle.gemm(A, B, threads=7))
    assert np.array_equal(one, oracle.gemm(A, B, threads=200))


@pytest.mark.parametrize("dist,K,var", [("uniform", 300, 300 / 9.0), ("normal", 512, 1.0 / 512),
                                        ("mlp", 512, 1.0)])
def test_output_moments_match_distribution(dist, K, var):
    # E[C] = 0; Var[C] = K Var[a] Var[b]: (1/3)^2 K for U[-1,1]; (1/K)^2 K for
    # N(0,1/sqrt K) both; 1 * (1/K) * K for N(0,1) activations and N(0,1/sqrt K) weights
    A, B = workloads.draw(128, 128, K, dist, 10)
    c = oracle.decode(oracle.gemm(bits(A), bits(B)))
    assert abs(c.mean()) < 0.05 * np.sqrt(var)
    assert abs(c.var() / var - 1.0) < 0.08


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
def test_transposed_operands_match_brute_force(ta, tb):
    # op(A) . op(B) with A given K x M and/or B given N x K
    rng = np.random.default_rng(int(ta) * 2 + int(tb))
    M, N, K = 4, 5, 6
    A = exact_range_operands(rng, (K, M) if ta else (M, K))
    B = exact_range_operands(rng, (N, K) if tb else (K, N))
    opA = np.ascontiguousarray(A.T) if ta else A
    opB = np.ascontiguousarray(B.T) if tb else B
    assert np.array_equal(oracle.gemm(A, B, trans_a=ta, trans_b=tb), brute_force.gemm(opA, opB))


# ---- the scale epilogue: C = rne16(epi(alpha * sum)) ----------------------------
# alpha as a binary32 (the library's precision for it), used at its exact value

@pytest.mark.parametrize("alpha", [0.1, -1.5, 1.0 / np.sqrt(128.0), 3.0, -0.0078125])
@pytest.mark.parametrize("relu", [False, True])
def test_scaled_brute_force_exact(alpha, relu):
    """Against exact rational arithmetic with Fraction(alpha): bit-identical,
    except that a zero result may carry either sign in the oracle (IEEE
    products keep the sign of a zero; the rational reference has none)."""
    a32 = oracle.as_binary32(alpha)
    for M, N, K in [(2, 3, 5), (5, 8, 3), (3, 2, 16), (4, 4, 40)]:
        rng = np.random.default_rng(M * 1000 + N * 100 + K + int(relu))
        A = exact_range_operands(rng, (M, K))
        B = exact_range_operands(rng, (K, N))
        ref = brute_force.gemm(A, B, relu=relu, scale=Fraction(a32))
        got = oracle.gemm(A, B, relu=relu, scale=a32)
        zero = (ref & 0x7FFF) == 0
        assert np.array_equal(got[~zero], ref[~zero]), (alpha, relu, M, N, K)
        assert np.all((got[zero] & 0x7FFF) == 0)


def test_scale_one_is_the_plain_product():
    A, B = workloads.draw(37, 29, 90, "uniform", 11)
    A, B = bits(A), bits(B)
    for relu in (False, True):
        assert np.array_equal(oracle.gemm(A, B, relu=relu, scale=1.0), oracle.gemm(A, B, relu=relu))
        assert np.array_equal(oracle.gemm_sampled(A, B, [0, 5, 36], [1, 28], relu=relu, scale=1.0),
                              oracle.gemm(A, B, relu=relu)[[0, 5, 36]][:, [1, 28]])


@pytest.mark.parametrize("e", [-4, -1, 3])
def test_power_of_two_scale_commutes_with_rounding(e):
    """alpha = 2^e: rne16(2^e s) = 2^e rne16(s) wherever neither rounding
    leaves the normal range, so the scaled result is the plain one times 2^e,
    bit for bit."""
    A, B = workloads.draw(40, 50, 60, "uniform", 12)
    A, B = bits(A), bits(B)
    c = oracle.decode(oracle.gemm(A, B))
    cs = oracle.decode(oracle.gemm(A, B, scale=2.0 ** e))
    normal = (np.abs(c) >= 2.0 ** -14) & (np.abs(c) * 2.0 ** e >= 2.0 ** -14) & (np.abs(c) * 2.0 ** e < 60000)
    assert normal.mean() > 0.9
    assert np.array_equal(cs[normal], c[normal] * 2.0 ** e)


def test_relu_applies_after_the_scale():
    """With a negative scale the positive results come from negative sums:
    relu(-0.5 s) is max(-0.5 rne16(s), 0), exactly (a power-of-two scale);
    a ReLU before the scale would leave nothing positive."""
    A, B = workloads.draw(33, 45, 70, "uniform", 13)
    A, B = bits(A), bits(B)
    c = oracle.decode(oracle.gemm(A, B))
    r = oracle.gemm(A, B, relu=True, scale=-0.5)
    want = np.maximum(-0.5 * c, 0.0)
    normal = (np.abs(c) >= 2.0 ** -13) | (c == 0)
    assert (want > 0).any() and (want == 0).any()
    assert np.array_equal(oracle.decode(r)[normal], want[normal])
    assert np.all(r[want == 0] == 0)                            # +0, never -0


def test_zero_scale_gives_zeros():
    A, B = workloads.draw(16, 24, 32, "uniform", 14)
    A, B = bits(A), bits(B)
    assert np.all((oracle.gemm(A, B, scale=0.0) & 0x7FFF) == 0)
    assert np.all(oracle.gemm(A, B, scale=0.0, relu=True) == 0)

"""Pins for the 2:4 structured-sparse oracle against facts that do not come
from the oracle.

The pages name 2:4 sparse GEMM (`T.gemm_sp`) in
"TileLang：让GPU编程像Python一样简单的高性能计算新范式", section
"高级特性超越基础矩阵乘法", without a storage format; the format and the
magnitude rule are this build's reading (oracle/oracle_sparse.c).  Pinned by:

* a hand-derived worked example of the format (tests/golden/sp_meta.txt);
* an independent numpy selection of the kept entries and numpy packing;
* decompression of an already 2:4-sparse matrix giving it back unchanged;
* exact rational brute force of the product on the decompressed matrix;
* positions named twice, whose terms must still add separately;
* integer operands (exact), the sampled block, ReLU = max(C, 0), bad K.
"""
import os

import numpy as np
import pytest

import oracle
from tests import brute_force

HERE = os.path.dirname(os.path.abspath(__file__))


def rng_half(shape, seed, lo=-4, hi=4, integers=True):
    g = np.random.default_rng(seed)
    if integers:
        x = g.integers(lo, hi + 1, size=shape).astype(np.float16)
    else:
        x = g.standard_normal(shape).astype(np.float16)
    return x.view(np.uint16)


def numpy_compress(A_bits):
    """Independent selection: per group, sort positions by (-magnitude, position)."""
    M, K = A_bits.shape
    mag = (A_bits & 0x7FFF).astype(np.int64)
    vals = np.zeros((M, K // 2), dtype=np.uint16)
    meta = np.zeros((M, K // 16), dtype=np.uint16)
    for i in range(M):
        for grp in range(K // 4):
            m = mag[i, 4 * grp:4 * grp + 4]
            order = sorted(range(4), key=lambda p: (-m[p], p))
            keep = sorted(order[:2])
            for t, p in enumerate(keep):
                vals[i, 2 * grp + t] = A_bits[i, 4 * grp + p]
                s = 2 * (grp % 4) + t
                meta[i, grp // 4] |= np.uint16(p << (2 * s))
    return vals, meta


def numpy_decompress(vals, meta):
    M, K = vals.shape[0], 2 * vals.shape[1]
    A = np.zeros((M, K), dtype=np.uint16)
    for i in range(M):
        for w in range(K // 16):
            for s in range(8):
                p = (int(meta[i, w]) >> (2 * s)) & 3
                A[i, 16 * w + 4 * (s // 2) + p] = vals[i, 8 * w + s]
    return A


def test_worked_examples():
    n = 0
    for line in open(os.path.join(HERE, "golden", "sp_meta.txt")):
        line = line.split("#")[0].strip()
        if not line.startswith("row"):
            continue
        dense, kept, word = (part.split() for part in line[3:].split("|"))
        A = np.array([float(x) for x in dense], dtype=np.float16).view(np.uint16)[None, :]
        vals, meta = oracle.sp_compress(A)
        assert np.array_equal(vals[0], np.array([float(x) for x in kept], dtype=np.float16).view(np.uint16))
        assert int(meta[0, 0]) == int(word[0], 16)
        n += 1
    assert n == 2


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_compress_matches_independent_selection(seed):
    # small integers give many magnitude ties; normals give subnormals and signs
    for A in (rng_half((7, 64), seed), rng_half((5, 48), seed + 10, integers=False)):
        v_ref, m_ref = numpy_compress(A)
        vals, meta = oracle.sp_compress(A)
        assert np.array_equal(vals, v_ref) and np.array_equal(meta, m_ref)
        # the dense form keeps exactly the selected entries
        assert np.array_equal(oracle.sp_decompress(vals, meta), numpy_decompress(v_ref, m_ref))


def test_already_sparse_round_trip():
    g = np.random.default_rng(3)
    M, K = 9, 96
    A = np.zeros((M, K), dtype=np.float16)
    for i in range(M):
        for grp in range(K // 4):
            keep = g.choice(4, size=g.integers(0, 3), replace=False)
            A[i, 4 * grp + keep] = g.standard_normal(keep.size).astype(np.float16) + np.float16(3)
    bits = A.view(np.uint16)
    vals, meta = oracle.sp_compress(bits)
    assert np.array_equal(oracle.sp_decompress(vals, meta), bits)


@pytest.mark.parametrize("shape", [(1, 1, 16), (3, 5, 16), (4, 7, 32), (6, 3, 48)])
@pytest.mark.parametrize("relu", [False, True])
def test_product_matches_brute_force(shape, relu):
    M, N, K = shape
    A = rng_half((M, K), M * 100 + K, integers=False)
    B = rng_half((K, N), N * 100 + K + 1, integers=False)
    vals, meta = oracle.sp_compress(A)
    dense = numpy_decompress(vals, meta)
    ref = brute_force.gemm(dense, B, relu=relu)
    got = oracle.gemm_sp(vals, meta, B, relu=relu)
    assert np.array_equal(got, ref)
    # and the dense oracle agrees on the decompressed matrix
    assert np.array_equal(got, oracle.gemm(dense, B, relu=relu))


def test_repeated_position_terms_add_separately():
    # both kept values of a group at one position: two separate products
    M, N, K = 3, 4, 16
    g = np.random.default_rng(5)
    vals = g.integers(-3, 4, size=(M, K // 2)).astype(np.float16).view(np.uint16)
    B = g.integers(-3, 4, size=(K, N)).astype(np.float16).view(np.uint16)
    meta = np.full((M, 1), 0b1010101010101010, dtype=np.uint16)   # every value at position 2
    v = vals.view(np.float16).astype(np.int64)
    b = B.view(np.float16).astype(np.int64)
    exact = np.zeros((M, N), dtype=np.int64)
    for i in range(M):
        for s in range(8):
            exact[i] += v[i, s] * b[4 * (s // 2) + 2]
    assert np.array_equal(oracle.gemm_sp(vals, meta, B), exact.astype(np.float16).view(np.uint16))
    with pytest.raises(ValueError):
        oracle.sp_decompress(vals, meta)


def test_integer_operands_exact():
    M, N, K = 40, 33, 256
    A = rng_half((M, K), 7, -3, 3)
    B = rng_half((K, N), 8, -3, 3)
    vals, meta = oracle.sp_compress(A)
    dense = numpy_decompress(vals, meta).view(np.float16).astype(np.int64)
    exact = dense @ B.view(np.float16).astype(np.int64)       # |C| <= 9 K / 2: exact in fp16 below 2048
    assert np.abs(exact).max() < 2048
    assert np.array_equal(oracle.gemm_sp(vals, meta, B), exact.astype(np.float16).view(np.uint16))


def test_sampled_block_and_relu():
    M, N, K = 50, 40, 64
    A = rng_half((M, K), 11, integers=False)
    B = rng_half((K, N), 12, integers=False)
    vals, meta = oracle.sp_compress(A)
    full = oracle.gemm_sp(vals, meta, B)
    rows, cols = np.array([0, 7, 49]), np.array([39, 0, 5, 6])
    assert np.array_equal(oracle.gemm_sp_sampled(vals, meta, B, rows, cols), full[np.ix_(rows, cols)])
    relu = oracle.gemm_sp(vals, meta, B, relu=True)
    neg = (full & 0x8000) != 0
    assert np.array_equal(relu[~neg], full[~neg]) and np.all(relu[neg] == 0)


def test_k_must_be_a_multiple_of_16():
    with pytest.raises(ValueError):
        oracle.sp_compress(np.zeros((2, 24), dtype=np.uint16))

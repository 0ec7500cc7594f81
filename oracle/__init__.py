"""CPU oracle for the tiled FP16 GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.

The oracle computes the plain definition of the product the tiled kernel
reaches (page "TileLang：比 Triton 低一层的 tile 语言", section
"第一个 kernel：GEMM"; fused ReLU from "TileLang：让GPU编程像Python一样简单的高性能计算新范式",
section "并行计算的优雅表达"):

    C[i, j] = rne16(epi(sum_k a(A[i, k]) * a(B[k, j])))

with exact binary16 decoding, a sequential fp64 sum over k and one
round-to-nearest-even to binary16.  The arithmetic lives in plain C
(``oracle_gemm.c``); this module marshals numpy arrays of binary16 bit
patterns (``uint16``) to it.  The tolerance rule used to compare a GPU
result with the oracle's is here too.

The 2:4 structured-sparse product of the same pages' overview (section
"高级特性超越基础矩阵乘法", ``T.gemm_sp``) is ``oracle_sparse.c``: magnitude
compression to (values, positions) and the product on the compressed operand.

Every function is pinned by the ``-m "not gpu"`` tests against facts that do
not come from the oracle itself: numpy's own binary16 conversion, exact
rational brute force, identity / permutation / integer cases, algebraic
invariants, and (sparse) an independent numpy selection of the kept entries.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i64, u16p, f64p, i64p = (ctypes.c_int64, ctypes.POINTER(ctypes.c_uint16),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64))
        lib.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_decode.restype = ctypes.c_double
        lib.oracle_f16_encode.argtypes = [ctypes.c_double]
        lib.oracle_f16_encode.restype = ctypes.c_uint16
        lib.oracle_f16_decode_array.argtypes = [u16p, f64p, i64]
        lib.oracle_f16_decode_array.restype = None
        lib.oracle_f16_encode_array.argtypes = [f64p, u16p, i64]
        lib.oracle_f16_encode_array.restype = None
        lib.oracle_cpu_threads.argtypes = []
        lib.oracle_cpu_threads.restype = ctypes.c_int
        lib.oracle_gemm_f16.argtypes = [i64, i64, i64, u16p, u16p, ctypes.c_int, u16p, ctypes.c_int]
        lib.oracle_gemm_f16_scaled.argtypes = [i64, i64, i64, u16p, u16p, ctypes.c_double, ctypes.c_int, u16p,
                                               ctypes.c_int]
        lib.oracle_gemm_f16_scaled.restype = ctypes.c_int
        lib.oracle_gemm_f16_sampled_scaled.argtypes = [i64, i64, i64, u16p, u16p, i64p, i64, i64p, i64,
                                                       ctypes.c_double, ctypes.c_int, u16p, ctypes.c_int]
        lib.oracle_gemm_f16_sampled_scaled.restype = ctypes.c_int
        lib.oracle_gemm_f16.restype = ctypes.c_int
        lib.oracle_gemm_f16_sampled.argtypes = [i64, i64, i64, u16p, u16p, i64p, i64, i64p, i64,
                                                ctypes.c_int, u16p, ctypes.c_int]
        lib.oracle_gemm_f16_sampled.restype = ctypes.c_int
        lib.oracle_sp_compress.argtypes = [i64, i64, u16p, u16p, u16p]
        lib.oracle_sp_compress.restype = ctypes.c_int
        lib.oracle_sp_decompress.argtypes = [i64, i64, u16p, u16p, u16p]
        lib.oracle_sp_decompress.restype = ctypes.c_int
        lib.oracle_gemm_f16_sp.argtypes = [i64, i64, i64, u16p, u16p, u16p, ctypes.c_int, u16p, ctypes.c_int]
        lib.oracle_gemm_f16_sp.restype = ctypes.c_int
        lib.oracle_gemm_f16_sp_sampled.argtypes = [i64, i64, i64, u16p, u16p, u16p, i64p, i64, i64p, i64,
                                                   ctypes.c_int, u16p, ctypes.c_int]
        lib.oracle_gemm_f16_sp_sampled.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _as_bits(x, name):
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16:
        raise TypeError(f"{name}: expected binary16 bit patterns (uint16) or float16, got {x.dtype}")
    return np.ascontiguousarray(x)


def cpu_threads() -> int:
    """Threads the oracle uses by default: the process's CPU affinity count."""
    return int(_lib().oracle_cpu_threads())


def decode(h) -> np.ndarray:
    """Exact value (float64) of each binary16 bit pattern."""
    h = _as_bits(h, "h")
    out = np.empty(h.shape, dtype=np.float64)
    _lib().oracle_f16_decode_array(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_double), h.size)
    return out


def encode(x) -> np.ndarray:
    """Nearest binary16 (ties to even) of each float64, as uint16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _lib().oracle_f16_encode_array(_ptr(x, ctypes.c_double), _ptr(out, ctypes.c_uint16), x.size)
    return out


def as_binary32(scale) -> float:
    """The exact value of ``scale`` rounded to binary32, the precision in
    which the library takes the epilogue's scale."""
    return float(np.float32(scale))


def gemm(A, B, relu: bool = False, threads: int = 0, trans_a: bool = False,
         trans_b: bool = False, scale: float = 1.0) -> np.ndarray:
    """C = rne16(epi(scale * (op(A) . op(B)))) for binary16 operands; returns
    uint16 (M x N).

    op(X) is X, or its transpose when the flag is set (A given K x M, B given
    N x K); the transpose is a plain array copy before the product.  ``scale``
    is used at its exact value: pass ``as_binary32(s)`` to mirror a binary32
    scale."""
    A = _as_bits(A, "A")
    B = _as_bits(B, "B")
    if trans_a:
        A = np.ascontiguousarray(A.T)
    if trans_b:
        B = np.ascontiguousarray(B.T)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch: A {A.shape}, B {B.shape}")
    M, K = A.shape
    N = B.shape[1]
    C = np.zeros((M, N), dtype=np.uint16)
    rc = _lib().oracle_gemm_f16_scaled(M, N, K, _ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16),
                                       float(scale), int(bool(relu)), _ptr(C, ctypes.c_uint16), int(threads))
    if rc != 0:
        raise RuntimeError("oracle_gemm_f16_scaled failed")
    return C


def gemm_sampled(A, B, rows, cols, relu: bool = False, threads: int = 0, scale: float = 1.0) -> np.ndarray:
    """The block C[rows x cols] of rne16(epi(scale * (A . B))); returns uint16
    (len(rows) x len(cols))."""
    A = _as_bits(A, "A")
    B = _as_bits(B, "B")
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch: A {A.shape}, B {B.shape}")
    M, K = A.shape
    N = B.shape[1]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    C = np.zeros((rows.size, cols.size), dtype=np.uint16)
    rc = _lib().oracle_gemm_f16_sampled_scaled(M, N, K, _ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16),
                                               _ptr(rows, ctypes.c_int64), rows.size,
                                               _ptr(cols, ctypes.c_int64), cols.size, float(scale),
                                               int(bool(relu)), _ptr(C, ctypes.c_uint16), int(threads))
    if rc != 0:
        raise RuntimeError("oracle_gemm_f16_sampled failed (bad index or allocation failure)")
    return C


# ---- 2:4 structured sparsity (oracle_sparse.c) ------------------------------
# A (M x K, K % 16 == 0) is kept as vals (M x K/2 binary16, the 2 kept values
# of every group of 4 k in increasing position order) and meta (M x K/16
# uint16: bits 2s+1..2s of word w give the position in its group of kept
# value s of dense k 16w .. 16w+15).  See the C file's header for the reading
# of the pages this follows.

def _u16(x, name):
    x = np.asarray(x)
    if x.dtype != np.uint16:
        raise TypeError(f"{name}: expected uint16, got {x.dtype}")
    return np.ascontiguousarray(x)


def sp_compress(A):
    """(vals, meta) of the 2:4 compression of A: per group of 4 k, the 2
    entries of largest magnitude (ties: lower position)."""
    A = _as_bits(A, "A")
    M, K = A.shape
    vals = np.zeros((M, K // 2), dtype=np.uint16)
    meta = np.zeros((M, K // 16), dtype=np.uint16)
    if _lib().oracle_sp_compress(M, K, _ptr(A, ctypes.c_uint16), _ptr(vals, ctypes.c_uint16),
                                 _ptr(meta, ctypes.c_uint16)) != 0:
        raise ValueError(f"K = {K} is not a multiple of 16")
    return vals, meta


def sp_decompress(vals, meta):
    """The dense matrix (binary16 bits) a compressed operand stands for."""
    vals = _as_bits(vals, "vals")
    meta = _u16(meta, "meta")
    M, K = vals.shape[0], 2 * vals.shape[1]
    if meta.shape != (M, K // 16):
        raise ValueError(f"meta shape {meta.shape}, expected {(M, K // 16)}")
    A = np.zeros((M, K), dtype=np.uint16)
    if _lib().oracle_sp_decompress(M, K, _ptr(vals, ctypes.c_uint16), _ptr(meta, ctypes.c_uint16),
                                   _ptr(A, ctypes.c_uint16)) != 0:
        raise ValueError("bad K or a group naming one position twice")
    return A


def gemm_sp(vals, meta, B, relu: bool = False, threads: int = 0) -> np.ndarray:
    """C = rne16(epi(A . B)) for a compressed 2:4-sparse A; returns uint16 (M x N)."""
    vals = _as_bits(vals, "vals")
    meta = _u16(meta, "meta")
    B = _as_bits(B, "B")
    M, K = vals.shape[0], 2 * vals.shape[1]
    if meta.shape != (M, K // 16) or B.shape[0] != K:
        raise ValueError(f"shape mismatch: vals {vals.shape}, meta {meta.shape}, B {B.shape}")
    N = B.shape[1]
    C = np.zeros((M, N), dtype=np.uint16)
    if _lib().oracle_gemm_f16_sp(M, N, K, _ptr(vals, ctypes.c_uint16), _ptr(meta, ctypes.c_uint16),
                                 _ptr(B, ctypes.c_uint16), int(bool(relu)), _ptr(C, ctypes.c_uint16),
                                 int(threads)) != 0:
        raise RuntimeError("oracle_gemm_f16_sp failed")
    return C


def gemm_sp_sampled(vals, meta, B, rows, cols, relu: bool = False, threads: int = 0) -> np.ndarray:
    """The block C[rows x cols] of the sparse product; returns uint16."""
    vals = _as_bits(vals, "vals")
    meta = _u16(meta, "meta")
    B = _as_bits(B, "B")
    M, K = vals.shape[0], 2 * vals.shape[1]
    if meta.shape != (M, K // 16) or B.shape[0] != K:
        raise ValueError(f"shape mismatch: vals {vals.shape}, meta {meta.shape}, B {B.shape}")
    N = B.shape[1]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    C = np.zeros((rows.size, cols.size), dtype=np.uint16)
    if _lib().oracle_gemm_f16_sp_sampled(M, N, K, _ptr(vals, ctypes.c_uint16), _ptr(meta, ctypes.c_uint16),
                                         _ptr(B, ctypes.c_uint16), _ptr(rows, ctypes.c_int64), rows.size,
                                         _ptr(cols, ctypes.c_int64), cols.size, int(bool(relu)),
                                         _ptr(C, ctypes.c_uint16), int(threads)) != 0:
        raise RuntimeError("oracle_gemm_f16_sp_sampled failed (bad index or allocation failure)")
    return C


# ---- tolerance ------------------------------------------------------------

ABS_FLOOR = 1e-3
ULPS = 2


def ulp(r_bits) -> np.ndarray:
    """Spacing of binary16 just above |r|: 2^(max(E, 1) - 25) with E the biased
    exponent field of r (2^-24 for zero and subnormals, 2^-10 in [1, 2))."""
    r_bits = _as_bits(r_bits, "r")
    E = (r_bits.astype(np.int64) >> 10) & 0x1F
    return np.ldexp(1.0, np.maximum(E, 1) - 25)


def compare(got_bits, ref_bits) -> dict:
    """Elementwise check of a GPU result against the oracle's.

    An element passes iff |g - r| <= max(2 * ulp(r), 1e-3), computed in fp64;
    any NaN fails.  Returns counts and the worst errors (in fp64 and in ulps
    of the reference).
    """
    g_bits = _as_bits(got_bits, "got")
    r_bits = _as_bits(ref_bits, "ref")
    if g_bits.shape != r_bits.shape:
        raise ValueError(f"shape mismatch: {g_bits.shape} vs {r_bits.shape}")
    g = decode(g_bits)
    r = decode(r_bits)
    u = ulp(r_bits)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - r)
        bound = np.maximum(ULPS * u, ABS_FLOOR)
        ok = err <= bound
    ok &= ~np.isnan(g) & ~np.isnan(r)
    n = int(g.size)
    n_fail = int(n - np.count_nonzero(ok))
    finite = np.isfinite(err)
    max_abs = float(err[finite].max()) if np.any(finite) else 0.0
    ulp_err = np.where(finite, err / u, np.inf)
    max_ulp = float(ulp_err.max()) if n else 0.0
    return {
        "n": n,
        "n_fail": n_fail,
        "pass": n_fail == 0,
        "max_abs_err": max_abs,
        "max_ulp_err": max_ulp,
        "n_gt_1ulp": int(np.count_nonzero(ulp_err > 1.0)),
        "n_bit_exact": int(np.count_nonzero(g_bits == r_bits)),
    }

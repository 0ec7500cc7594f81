"""The order in which the library stores sparse A's position words, as
include/gemm_f16.h states it: by 64-deep k slices, so that one slice's words
of consecutive rows are contiguous.  Tests use it to bring the library's
words into the row-major M x K/16 matrix the oracle works with."""
import numpy as np


def meta_index(M: int, K: int) -> np.ndarray:
    """idx[i, w] = storage index of word w of row i (M x K/16)."""
    kw = K // 16
    full = kw // 4
    i = np.arange(M, dtype=np.int64)[:, None]
    w = np.arange(kw, dtype=np.int64)[None, :]
    in_full = (w // 4) < full
    return np.where(in_full, ((w // 4) * M + i) * 4 + w % 4, full * M * 4 + i * (kw % 4) + w % 4)


def meta_rows(flat: np.ndarray, M: int, K: int) -> np.ndarray:
    """The stored words (flat, M K/16 of them) as the M x K/16 row-major matrix."""
    flat = np.asarray(flat).reshape(-1)
    assert flat.size == M * (K // 16)
    return flat[meta_index(M, K)] if flat.size else flat.reshape(M, K // 16)


def meta_flat(rows: np.ndarray) -> np.ndarray:
    """Inverse of meta_rows: the row-major words in storage order."""
    M, kw = rows.shape
    out = np.empty(M * kw, dtype=rows.dtype)
    out[meta_index(M, 16 * kw)] = rows
    return out

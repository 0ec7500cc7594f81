"""GPU parity of the 2:4 structured-sparse path against the CPU oracle.

The compression must match oracle.sp_compress bit for bit (it is integer
work: selection by exact magnitude comparison, packing of positions); the
product must match oracle.gemm_sp within max(2 fp16 ulps, 1e-3) per element,
as the dense path does.  The operation is the pages' `T.gemm_sp`
("TileLang：让GPU编程像Python一样简单的高性能计算新范式", section
"高级特性超越基础矩阵乘法"), in the format documented in include/gemm_f16.h.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_fp16_amd as g
import workloads
from sp_layout import meta_flat, meta_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def draw(M, N, K, seed, ties=False):
    a, b = workloads.draw(M, N, K, "uniform", seed)
    if ties:
        # small integers: many equal magnitudes inside a group
        gen = torch.Generator().manual_seed(seed + 7)
        a = torch.randint(-2, 3, (M, K), generator=gen).to(torch.float16)
    return a, b


@pytest.mark.parametrize("shape,ties", [((1, 16), False), ((257, 80), False), ((64, 4096), False),
                                        ((33, 48), True), ((300, 1008), True)])
def test_compress_bit_exact(shape, ties):
    M, K = shape
    a, _ = draw(M, 8, K, M + K, ties)
    print(f"[sparse] compress {M}x{K} ties={ties}", flush=True)
    vals, meta = g.sp_compress(a.to(DEV))
    torch.cuda.synchronize()
    v_ref, m_ref = oracle.sp_compress(u16(a))
    assert np.array_equal(u16(vals), v_ref)
    assert np.array_equal(meta_rows(u16(meta), M, K), m_ref)


def test_compress_unaligned_source():
    # A starting 2 bytes into an allocation: the element-wise path
    M, K = 40, 64
    a, _ = draw(M, 8, K, 5)
    buf = torch.empty(M * K + 1, dtype=torch.float16, device=DEV)
    ad = buf[1:].view(M, K)
    ad.copy_(a.to(DEV))
    vals, meta = g.sp_compress(ad)
    torch.cuda.synchronize()
    v_ref, m_ref = oracle.sp_compress(u16(a))
    assert np.array_equal(u16(vals), v_ref) and np.array_equal(meta_rows(u16(meta), M, K), m_ref)


def check_sp(M, N, K, seed, config=g.CONFIG_AUTO, epilogue="none", trans_b=False):
    a, b = draw(M, N, K, seed)
    vals, meta = g.sp_compress(a.to(DEV))
    b_st = b.t().contiguous() if trans_b else b
    c = g.gemm_sp(vals, meta, b_st.to(DEV), epilogue=epilogue, config=config, trans_b=trans_b)
    torch.cuda.synchronize()
    p = g.plan_sp(M, N, K, vals.data_ptr(), meta.data_ptr(), 1 << 20, 1 << 20, config=config, trans_b=trans_b)
    print(f"[sparse] gemm {M}x{N}x{K} trans_b={trans_b} config={g.sp_config_name(p['config'])} epi={epilogue}",
          flush=True)
    v_ref, m_ref = oracle.sp_compress(u16(a))
    ref = oracle.gemm_sp(v_ref, m_ref, u16(b), relu=(epilogue == "relu"))
    res = oracle.compare(u16(c), ref)
    assert res["pass"], (M, N, K, config, res)
    return u16(c)


# several tiles of both configurations, ragged M and N, K with a half step (K % 32 == 16)
SHAPES = [(256, 256, 256), (300, 264, 1008), (1, 8, 16), (257, 520, 80), (130, 72, 4096), (64, 64, 32)]


@pytest.mark.parametrize("shape", SHAPES)
def test_every_sparse_config(shape):
    for c in range(g.sp_num_configs()):
        check_sp(*shape, seed=sum(shape), config=c)


@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 268, 1008), (1, 4, 16), (130, 72, 4096)])
def test_every_sparse_config_b_transposed(shape):
    # B given N x K (N need not be a multiple of 8 then)
    for c in range(g.sp_num_configs()):
        check_sp(*shape, seed=3 * sum(shape), config=c, trans_b=True)


@pytest.mark.parametrize("epilogue", ["none", "relu"])
def test_sparse_auto_and_relu(epilogue):
    check_sp(520, 392, 512, seed=3, epilogue=epilogue)


def test_sparse_zero_k_and_empty():
    vals = torch.empty((70, 0), dtype=torch.float16, device=DEV)
    meta = torch.empty((0,), dtype=torch.int16, device=DEV)
    b = torch.empty((0, 96), dtype=torch.float16, device=DEV)
    c = torch.full((70, 96), 3.0, dtype=torch.float16, device=DEV)
    g.gemm_sp(vals, meta, b, out=c)
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0


def test_sparse_deterministic_and_guarded():
    M, N, K = 300, 264, 1008
    a, b = draw(M, N, K, 21)
    vals, meta = g.sp_compress(a.to(DEV))
    bd = b.to(DEV)
    guard = 4096
    sentinel = np.float16(-1234.0).view(np.uint16)
    first = None
    for _ in range(3):
        buf = torch.full((M * N + 2 * guard,), -1234.0, dtype=torch.float16, device=DEV)
        g.gemm_sp(vals, meta, bd, out=buf[guard:guard + M * N].view(M, N))
        torch.cuda.synchronize()
        host = u16(buf)
        assert np.all(host[:guard] == sentinel) and np.all(host[guard + M * N:] == sentinel)
        if first is None:
            first = host
        assert np.array_equal(host, first)


def test_sparse_large_sampled():
    # a size that runs the 256 x 256 sparse tile over many k tiles
    M = N = K = 4096
    a, b = draw(M, N, K, 22)
    vals, meta = g.sp_compress(a.to(DEV))
    c = g.gemm_sp(vals, meta, b.to(DEV))
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(1022)
    rows = torch.randperm(M, generator=gen)[:512].numpy()
    cols = torch.randperm(N, generator=gen)[:512].numpy()
    v_ref, m_ref = oracle.sp_compress(u16(a))
    ref = oracle.gemm_sp_sampled(v_ref, m_ref, u16(b), rows, cols)
    got = u16(c)[np.ix_(rows, cols)]
    res = oracle.compare(got, ref)
    print(f"[sparse] 4096^3 sampled: {res}", flush=True)
    assert res["pass"], res


@pytest.mark.parametrize("shape", [(300, 264, 1008), (130, 72, 4096), (257, 520, 80), (257, 136, 1024)])
def test_oracle_operands_through_the_library(shape):
    """The oracle's own compression, put into the library's storage order,
    multiplied by the library: the stored order the kernels read is the one
    the header documents (whole and partial 64-deep slices)."""
    M, N, K = shape
    a, b = draw(M, N, K, 31 + M)
    v_ref, m_ref = oracle.sp_compress(u16(a))
    vals = torch.from_numpy(v_ref.view(np.int16).copy()).view(torch.float16).to(DEV)
    meta = torch.from_numpy(meta_flat(m_ref).view(np.int16)).to(DEV)
    c = g.gemm_sp(vals, meta, b.to(DEV))
    torch.cuda.synchronize()
    res = oracle.compare(u16(c), oracle.gemm_sp(v_ref, m_ref, u16(b)))
    assert res["pass"], res

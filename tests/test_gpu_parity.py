"""GPU parity of the HIP GEMM against the CPU oracle, through the C ABI.

Bar: every element within max(2 fp16 ulps of the oracle's value, 1e-3)
(``oracle.compare``); bit-exact where the exact result is representable
(identity, integer-valued operands); bitwise run-to-run determinism; no write
outside C.  The tile GEMM, its fused ReLU and the fp16 write-back are those
of "TileLang：比 Triton 低一层的 tile 语言" (section "第一个 kernel：GEMM") and
"TileLang：让GPU编程像Python一样简单的高性能计算新范式" (section
"并行计算的优雅表达"); the pages ask for boundary shapes whose M, N, K are not
tile multiples (same page as the first, section "工程上的几个注意点").
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_fp16_amd as g
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run(a, b, epilogue="none", config=g.CONFIG_AUTO):
    c = g.gemm(a.to(DEV), b.to(DEV), epilogue=epilogue, config=config)
    torch.cuda.synchronize()
    return u16(c)


def check(a, b, epilogue="none", config=g.CONFIG_AUTO, label=""):
    print(f"[parity] {label} {tuple(a.shape)}x{tuple(b.shape)} epi={epilogue} config={config}", flush=True)
    got = run(a, b, epilogue, config)
    ref = oracle.gemm(u16(a), u16(b), relu=(epilogue == "relu"))
    res = oracle.compare(got, ref)
    assert res["pass"], f"{label}: {res}"
    return res


def configs_for(M, N, K, trans_a=False, trans_b=False):
    """Every configuration that accepts this (aligned-pointer) shape and layout."""
    out = []
    for c in range(g.num_configs()):
        try:
            g.plan(M, N, K, 1 << 20, 1 << 20, 1 << 20, config=c, trans_a=trans_a, trans_b=trans_b)
            out.append(c)
        except g.GemmError:
            pass
    return out


# shapes spanning several tiles of every configuration, with ragged tails
ALIGNED_SHAPES = [(64, 64, 64), (520, 392, 200), (300, 264, 136), (1, 8, 8), (257, 520, 72),
                  (96, 1040, 8)]


@pytest.mark.parametrize("shape", ALIGNED_SHAPES)
def test_every_config_aligned_shapes(shape):
    M, N, K = shape
    a, b = workloads.draw(M, N, K, "uniform", M + N + K)
    cfgs = configs_for(M, N, K)
    # every tile configuration takes an aligned shape; the persistent loop
    # only an even number (at least two) of 64-deep k tiles
    k_tiles = -(-K // 64)
    want = [c for c in range(g.num_configs())
            if "persistent" not in g.config_name(c) or (k_tiles >= 2 and k_tiles % 2 == 0)]
    assert cfgs == want
    for c in cfgs:
        check(a, b, config=c, label=f"config {g.config_name(c)}")


# K and N that are not multiples of 8 force narrower vectors (staged kernels)
RAGGED_SHAPES = [(37, 45, 53), (130, 129, 67), (200, 300, 100), (65, 66, 34), (3, 5, 7), (129, 36, 1)]


@pytest.mark.parametrize("shape", RAGGED_SHAPES)
@pytest.mark.parametrize("epilogue", ["none", "relu"])
def test_ragged_shapes(shape, epilogue):
    M, N, K = shape
    a, b = workloads.draw(M, N, K, "uniform", 7 * M + N + K)
    check(a, b, epilogue, label="auto")
    for c in configs_for(M, N, K):
        check(a, b, epilogue, config=c, label=f"config {g.config_name(c)}")


# ---- rows only 4-byte aligned: the direct configurations for such rows ----
# Their loads move 16-byte chunks at 4-byte alignment.  Where K % 8 != 0 the
# chunk at the end of a k-row (A given M x K, B given N x K) runs into the
# next row's first elements, which the kernel zeroes in LDS; an mn-row's
# chunk past M or N only reaches outputs that are never stored.
U_NAMES = ("256x256x64_s2_direct_m16_u", "256x128x64_s3_direct_m16_u", "128x128x64_s4_direct_m16_u",
           "128x64x64_s4_direct_u", "64x64x64_s4_direct_u")
# every pitch even; K % 8 in {2, 4, 6}; M and N pitches off 16-byte alignment in some
U_SHAPES = [(300, 264, 130), (520, 392, 198), (258, 522, 66), (64, 64, 2), (510, 268, 4100), (130, 134, 132)]
ALL_LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def u_configs():
    cfgs = [c for c in range(g.num_configs()) if g.config_name(c) in U_NAMES]
    assert len(cfgs) == len(U_NAMES)
    return cfgs


@pytest.mark.parametrize("ta,tb", ALL_LAYOUTS)
@pytest.mark.parametrize("shape", U_SHAPES)
def test_rows_4byte_aligned_direct_configs(ta, tb, shape):
    M, N, K = shape
    a_st, b_st = stored(M, N, K, ta, tb, 11 * M + 3 * N + K)
    a_dev, b_dev = a_st.to(DEV), b_st.to(DEV)
    for epi in ("none", "relu"):
        ref = oracle.gemm(u16(a_st), u16(b_st), relu=(epi == "relu"), trans_a=ta, trans_b=tb)
        for c in u_configs():
            p = g.plan(M, N, K, a_dev.data_ptr(), b_dev.data_ptr(), 1 << 20, config=c, trans_a=ta, trans_b=tb)
            assert (p["direct_lds"], p["vec_a"], p["vec_b"]) == (1, 2, 2)
            print(f"[parity] 4-byte rows ta={ta} tb={tb} {M}x{N}x{K} epi={epi} {g.config_name(c)}", flush=True)
            out = g.gemm(a_dev, b_dev, epilogue=epi, config=c, trans_a=ta, trans_b=tb)
            torch.cuda.synchronize()
            res = oracle.compare(u16(out), ref)
            assert res["pass"], (ta, tb, shape, epi, g.config_name(c), res)


@pytest.mark.parametrize("ta,tb", ALL_LAYOUTS)
def test_rows_4byte_aligned_large_sampled(ta, tb):
    """A large shape whose every row pitch is only 8-byte aligned (K % 8 = 4),
    in each layout, through the automatic choice (a direct configuration for
    4-byte rows): a seeded sample of rows and columns, with the tile edges,
    against the oracle."""
    M, N, K = 4100, 4108, 4100
    a, b = workloads.draw(M, N, K, "normal", 4100 + 2 * ta + tb)
    a_st = a.t().contiguous() if ta else a
    b_st = b.t().contiguous() if tb else b
    a_dev, b_dev = a_st.to(DEV), b_st.to(DEV)
    p = g.plan(M, N, K, a_dev.data_ptr(), b_dev.data_ptr(), 1 << 20, trans_a=ta, trans_b=tb)
    assert p["direct_lds"] == 1 and g.config_name(p["config"]).endswith("_u"), g.config_name(p["config"])
    print(f"[parity] 4-byte rows, large, sampled, ta={ta} tb={tb} {g.config_name(p['config'])}", flush=True)
    out = g.gemm(a_dev, b_dev, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu")
    gen.manual_seed(77 + 2 * ta + tb)
    edges = [0, 1, 127, 128, 255, 256, 4095, 4096]
    rows = sorted(set(torch.randperm(M, generator=gen)[:192].tolist() + edges + [M - 1]))
    cols = sorted(set(torch.randperm(N, generator=gen)[:192].tolist() + edges + [N - 1]))
    got = u16(out[torch.tensor(rows, device=DEV)][:, torch.tensor(cols, device=DEV)])
    ref = oracle.gemm_sampled(u16(a), u16(b), rows, cols)
    res = oracle.compare(got, ref)
    assert res["pass"], (ta, tb, res)


@pytest.mark.parametrize("ta,tb", ALL_LAYOUTS)
def test_rows_4byte_aligned_split_k(ta, tb):
    """The configurations for 4-byte rows with K split three ways: only the
    last split's range ends inside a chunk (K % 8 = 4)."""
    M, N, K = 300, 268, 1348
    a_st, b_st = stored(M, N, K, ta, tb, 31 + 2 * ta + tb)
    a_dev, b_dev = a_st.to(DEV), b_st.to(DEV)
    ref = oracle.gemm(u16(a_st), u16(b_st), trans_a=ta, trans_b=tb)
    ws = torch.empty(3 * M * N, dtype=torch.float32, device=DEV)
    for c in u_configs():
        p = g.plan(M, N, K, a_dev.data_ptr(), b_dev.data_ptr(), 1 << 20, config=c, trans_a=ta, trans_b=tb, splits=3)
        assert p["splits"] == 3, p
        print(f"[parity] 4-byte rows, K split 3, ta={ta} tb={tb} {g.config_name(c)}", flush=True)
        out = g.gemm(a_dev, b_dev, config=c, trans_a=ta, trans_b=tb, splits=3, workspace=ws)
        torch.cuda.synchronize()
        res = oracle.compare(u16(out), ref)
        assert res["pass"], (ta, tb, g.config_name(c), res)


def compare_with_specials(got, ref):
    """NaN and infinity where the oracle has them (same sign); every finite
    reference element within the usual bound."""
    gv, rv = oracle.decode(got), oracle.decode(ref)
    assert np.array_equal(np.isnan(gv), np.isnan(rv))
    assert np.array_equal(np.isposinf(gv), np.isposinf(rv)) and np.array_equal(np.isneginf(gv), np.isneginf(rv))
    fin = np.isfinite(rv)
    res = oracle.compare(got[fin], ref[fin])
    assert res["pass"], res
    return int(np.count_nonzero(~fin))


@pytest.mark.parametrize("K", [130, 132, 134])
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, True)])
def test_rows_4byte_aligned_tail_chunk_is_cleared(K, ta, tb):
    """Infinities and a NaN among the first k of some rows of each k-rows
    operand: the chunk that ends the previous row at K reads them, and the
    previous row's outputs must still equal the oracle's (finite)."""
    M, N = 300, 264
    a, b = workloads.draw(M, N, K, "uniform", 7 * K + 2 * ta + tb)
    a, b = a.clone(), b.clone()
    vals = (float("inf"), float("-inf"), float("nan"), float("inf"))
    if not ta:
        # A given M x K: rows 1, 77, 255, 257 start with a special; B's first
        # rows kept away from zero and subnormals (infinity times them is
        # then infinity, whatever the order of the sum)
        b[:4] = torch.where(b[:4].abs() < 1 / 16, torch.full_like(b[:4], 0.5), b[:4])
        for r, k, v in zip((1, 77, 255, 257), range(4), vals):
            a[r, k] = v
    if tb:
        # B given N x K: columns 1, 130, 257, 263 of the product likewise
        a[:, :4] = torch.where(a[:, :4].abs() < 1 / 16, torch.full_like(a[:, :4], 0.5), a[:, :4])
        for n, k, v in zip((1, 130, 257, 263), range(4), vals):
            b[k, n] = v
    a_st = a.t().contiguous() if ta else a
    b_st = b.t().contiguous() if tb else b
    ref = oracle.gemm(u16(a_st), u16(b_st), trans_a=ta, trans_b=tb)
    a_dev, b_dev = a_st.to(DEV), b_st.to(DEV)
    for c in u_configs():
        print(f"[parity] tail chunk with specials ta={ta} tb={tb} K={K} {g.config_name(c)}", flush=True)
        out = g.gemm(a_dev, b_dev, config=c, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        n_special = compare_with_specials(u16(out), ref)
        assert n_special > 0


def test_rows_4byte_aligned_nt_offset_pointer():
    """B given N x K with a 16-byte aligned pitch, A's pointer only 4-byte
    aligned (a view two elements into a buffer)."""
    M, N, K = 300, 264, 136
    a, b = workloads.draw(M, N, K, "uniform", 1234)
    buf = torch.zeros(M * K + 8, dtype=torch.float16, device=DEV)
    a_dev = buf[2:2 + M * K].view(M, K)
    a_dev.copy_(a.to(DEV))
    bt = b.t().contiguous().to(DEV)
    ref = oracle.gemm(u16(a), u16(b))
    for c in u_configs():
        p = g.plan(M, N, K, a_dev.data_ptr(), bt.data_ptr(), 1 << 20, config=c, trans_b=True)
        assert p["vec_a"] == 2 and p["direct_lds"] == 1
        print(f"[parity] 4-byte rows, NT, A pointer offset by 4 bytes, {M}x{N}x{K} {g.config_name(c)}", flush=True)
        out = g.gemm(a_dev, bt, config=c, trans_b=True)
        torch.cuda.synchronize()
        res = oracle.compare(u16(out), ref)
        assert res["pass"], res


def test_misaligned_pointers():
    # operands and output that start one element into a buffer are only
    # 2-byte aligned; with K, N not multiples of 8 every vector width drops
    M, N, K = 70, 90, 40
    a, b = workloads.draw(M, N, K, "uniform", 11)
    a_buf = torch.empty(M * K + 1, dtype=torch.float16, device=DEV)
    a_buf[1:] = a.to(DEV).flatten()
    a_mis = a_buf[1:].view(M, K)
    c_buf = torch.empty(M * N + 1, dtype=torch.float16, device=DEV)
    c_mis = c_buf[1:].view(M, N)
    assert a_mis.data_ptr() % 4 != 0 and c_mis.data_ptr() % 4 != 0
    p = g.plan(M, N, K, a_mis.data_ptr(), 1 << 20, c_mis.data_ptr())
    assert (p["vec_a"], p["vec_c"]) == (1, 1)
    g.gemm(a_mis, b.to(DEV), out=c_mis)
    torch.cuda.synchronize()
    res = oracle.compare(u16(c_mis), oracle.gemm(u16(a), u16(b)))
    assert res["pass"], res


def test_degenerate_dimensions():
    # K == 0: the empty sum, C = +0 everywhere (also with ReLU)
    a = torch.empty(33, 0, dtype=torch.float16, device=DEV)
    b = torch.empty(0, 17, dtype=torch.float16, device=DEV)
    for epi in ("none", "relu"):
        c = torch.full((33, 17), 7.0, dtype=torch.float16, device=DEV)
        g.gemm(a, b, epilogue=epi, out=c)
        torch.cuda.synchronize()
        assert np.all(u16(c) == 0)
    # M == 0 or N == 0: nothing launched, success
    g.gemm(torch.empty(0, 8, dtype=torch.float16, device=DEV), torch.empty(8, 8, dtype=torch.float16, device=DEV))
    g.gemm(torch.empty(8, 8, dtype=torch.float16, device=DEV), torch.empty(8, 0, dtype=torch.float16, device=DEV))
    # single elements
    a, b = workloads.draw(1, 1, 1, "uniform", 3)
    check(a, b, label="1x1x1")
    a, b = workloads.draw(1, 1, 4096, "uniform", 4)
    check(a, b, label="dot product")


def test_empty_k_every_config():
    # K == 0 with N % 8 == 0: every configuration, including the 256x256
    # four-wave tiles' staged-epilogue build, whose last MFMA then multiplies
    # zeroed fragments; C must hold +0 (also under ReLU)
    M, N = 300, 264
    a = torch.empty(M, 0, dtype=torch.float16, device=DEV)
    b = torch.empty(0, N, dtype=torch.float16, device=DEV)
    cfgs = configs_for(M, N, 0)
    # the persistent loop takes no empty K (its planner runs the one-tile twin)
    assert cfgs == [c for c in range(g.num_configs()) if "persistent" not in g.config_name(c)]
    for cfg in cfgs:
        for epi in ("none", "relu"):
            print(f"[parity] empty K config={cfg} epi={epi}", flush=True)
            c = torch.full((M, N), -5.0, dtype=torch.float16, device=DEV)
            g.gemm(a, b, epilogue=epi, out=c, config=cfg)
            torch.cuda.synchronize()
            assert np.all(u16(c) == 0), (cfg, epi)


@pytest.mark.parametrize("offset", [1, 4])
def test_unaligned_output_every_config(offset):
    # C starting 1 or 4 elements into its buffer (2- or 8-byte aligned): the
    # general epilogue with 2- or 8-byte stores in every configuration, next
    # to the 16-byte operands the direct kernels need
    M, N, K = 300, 264, 136
    a, b = workloads.draw(M, N, K, "uniform", 40 + offset)
    ad, bd = a.to(DEV), b.to(DEV)
    ref = oracle.gemm(u16(a), u16(b))
    guard = 64
    for cfg in configs_for(M, N, K):
        buf = torch.full((M * N + offset + guard,), -1234.0, dtype=torch.float16, device=DEV)
        c = buf[offset:offset + M * N].view(M, N)
        p = g.plan(M, N, K, ad.data_ptr(), bd.data_ptr(), c.data_ptr(), config=cfg)
        assert p["vec_c"] == (1 if offset == 1 else 4)
        print(f"[parity] unaligned C offset={offset} config={cfg}", flush=True)
        g.gemm(ad, bd, out=c, config=cfg)
        torch.cuda.synchronize()
        res = oracle.compare(u16(c), ref)
        assert res["pass"], (cfg, res)
        host = u16(buf)
        sentinel = np.float16(-1234.0).view(np.uint16)
        assert np.all(host[:offset] == sentinel) and np.all(host[offset + M * N:] == sentinel)


def test_no_writes_outside_c():
    M, N, K = 300, 264, 72
    a, b = workloads.draw(M, N, K, "uniform", 21)
    ad, bd = a.to(DEV), b.to(DEV)
    guard = 4096
    for c in [g.CONFIG_AUTO] + configs_for(M, N, K):
        buf = torch.full((M * N + 2 * guard,), -1234.0, dtype=torch.float16, device=DEV)
        out = buf[guard:guard + M * N].view(M, N)
        g.gemm(ad, bd, out=out, config=c)
        torch.cuda.synchronize()
        host = u16(buf)
        sentinel = np.float16(-1234.0).view(np.uint16)
        assert np.all(host[:guard] == sentinel) and np.all(host[guard + M * N:] == sentinel), c
        res = oracle.compare(host[guard:guard + M * N].reshape(M, N), oracle.gemm(u16(a), u16(b)))
        assert res["pass"], (c, res)


def test_exact_cases_bit_identical():
    # identity: I . B == B exactly; integer operands: exact integer products
    n = 264
    _, b = workloads.draw(n, 200, n, "uniform", 5)
    eye = torch.eye(n, dtype=torch.float16)
    assert np.array_equal(run(eye, b), u16(b))
    for c in configs_for(n, 200, n):
        assert np.array_equal(run(eye, b, config=c), u16(b)), c
    M, N, K = 3000, 5000, 4100
    a, b = workloads.draw_ints(M, N, K, seed=8, lo=-2, hi=2)
    got = run(a, b)
    exact = (a.double() @ b.double()).to(torch.float16)     # |C| <= 4K < 2^24: fp64 is exact
    assert np.array_equal(got, u16(exact))


def test_relu_equals_max_of_plain():
    a, b = workloads.draw(520, 392, 200, "uniform", 12)
    for c in configs_for(520, 392, 200):
        plain = run(a, b, "none", c)
        relu = run(a, b, "relu", c)
        neg = (plain & 0x8000) != 0
        assert np.array_equal(relu[~neg], plain[~neg]) and np.all(relu[neg] == 0), c


def test_deterministic():
    a, b = workloads.draw(1000, 1100, 900, "normal", 13)
    ad, bd = a.to(DEV), b.to(DEV)
    first = u16(g.gemm(ad, bd))
    for _ in range(3):
        assert np.array_equal(u16(g.gemm(ad, bd)), first)


# ---- transposed operands: A given K x M and/or B given N x K ----

LAYOUTS = [(False, True), (True, False), (True, True)]


def check_trans(a_st, b_st, ta, tb, epilogue="none", config=g.CONFIG_AUTO):
    print(f"[parity] trans_a={ta} trans_b={tb} {tuple(a_st.shape)} {tuple(b_st.shape)} config={config}",
          flush=True)
    c = g.gemm(a_st.to(DEV), b_st.to(DEV), epilogue=epilogue, config=config, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    ref = oracle.gemm(u16(a_st), u16(b_st), relu=(epilogue == "relu"), trans_a=ta, trans_b=tb)
    res = oracle.compare(u16(c), ref)
    assert res["pass"], (ta, tb, config, res)


def stored(M, N, K, ta, tb, seed):
    a, b = workloads.draw(M, N, K, "uniform", seed)
    return (a.t().contiguous() if ta else a), (b.t().contiguous() if tb else b)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(520, 392, 200), (256, 256, 64), (300, 264, 136), (64, 1040, 8), (300, 268, 132)])
def test_transposed_layouts_every_config(ta, tb, shape):
    M, N, K = shape
    a_st, b_st = stored(M, N, K, ta, tb, M + N + K)
    cfgs = configs_for(M, N, K, ta, tb)
    assert len(cfgs) >= 2
    for c in cfgs:
        check_trans(a_st, b_st, ta, tb, config=c)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(37, 45, 53), (130, 129, 67), (65, 66, 34), (3, 5, 7)])
@pytest.mark.parametrize("epilogue", ["none", "relu"])
def test_transposed_layouts_ragged(ta, tb, shape, epilogue):
    M, N, K = shape
    a_st, b_st = stored(M, N, K, ta, tb, 5 * M + N + K)
    check_trans(a_st, b_st, ta, tb, epilogue)
    for c in configs_for(M, N, K, ta, tb):
        check_trans(a_st, b_st, ta, tb, epilogue, config=c)


def test_transposed_layout_large():
    # Q . K^T-shaped product at a size that runs the 256x256 direct kernel
    M, N, K = 2048, 2304, 1024
    a, b_st = stored(M, N, K, False, True, 99)
    assert g.plan(M, N, K, 1 << 20, 1 << 20, 1 << 20, trans_b=True)["direct_lds"] == 1
    check_trans(a, b_st, False, True)


# ---- the benchmark workloads, in the configuration the benchmark launches ----

@pytest.mark.parametrize("name", ["gemm_256", "gemm_1024_relu", "gemm_4096", "gemm_ragged_3000x5000x4100"])
def test_workload_full(name):
    w = workloads.WORKLOADS[name]
    a, b = workloads.make_inputs(w)
    res = check(a, b, "relu" if w.relu else "none", label=name)
    print(f"[parity] {name}: {res}", flush=True)


@pytest.mark.parametrize("name", ["gemm_8192", "gemm_mlp_8192x28672x8192"])
def test_workload_sampled(name):
    w = workloads.WORKLOADS[name]
    a, b = workloads.make_inputs(w)
    rows, cols = workloads.sample_indices(w)
    print(f"[parity] {name}: gemm on GPU", flush=True)
    c = g.gemm(a.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    got = u16(c[rows.to(DEV)][:, cols.to(DEV)])
    del c
    print(f"[parity] {name}: oracle on {oracle.cpu_threads()} threads", flush=True)
    ref = oracle.gemm_sampled(u16(a), u16(b), rows.numpy(), cols.numpy())
    res = oracle.compare(got, ref)
    print(f"[parity] {name}: {res}", flush=True)
    assert res["pass"], res
    # tile-edge rows and columns of the output, checked separately
    edge_r = np.array(sorted({0, 1, 255, 256, w.M - 1}))
    edge_c = np.array(sorted({0, 1, 255, 256, w.N - 1}))
    c = g.gemm(a.to(DEV), b.to(DEV))
    torch.cuda.synchronize()
    got = u16(c[torch.from_numpy(edge_r).to(DEV)][:, torch.from_numpy(edge_c).to(DEV)])
    res = oracle.compare(got, oracle.gemm_sampled(u16(a), u16(b), edge_r, edge_c))
    assert res["pass"], res


# ---- the scale epilogue: C = rne16(epi(alpha * (op(A) . op(B)))) ----------------
# the pages scale the fp32 score block of the transpose_B product before anything
# else touches it ("TileLang：比 Triton 低一层的 tile 语言", section "FlashAttention：
# 在线 softmax 写成 tile 代码"); the scale there is 1/sqrt(dim) * log2(e)

def qk_scale(dim):
    return float(1.0 / np.sqrt(dim) * 1.44269504)


def stored_operands(M, N, K, ta, tb, seed, dist="uniform"):
    a, b = workloads.draw(M, N, K, dist, seed)
    return a, b, (a.t().contiguous() if ta else a), (b.t().contiguous() if tb else b)


@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_scale_epilogue_every_config(ta, tb):
    M, N, K = 300, 264, 136
    a, b, a_st, b_st = stored_operands(M, N, K, ta, tb, 31 + 2 * ta + tb)
    ad, bd = a_st.to(DEV), b_st.to(DEV)
    for epilogue, alpha in (("none", qk_scale(K)), ("relu", -0.75), ("none", -3.0)):
        ref = oracle.gemm(u16(a), u16(b), relu=(epilogue == "relu"), scale=oracle.as_binary32(alpha))
        for c in configs_for(M, N, K, trans_a=ta, trans_b=tb):
            print(f"[scale] ta={int(ta)} tb={int(tb)} epi={epilogue} alpha={alpha:.6g} config={c}", flush=True)
            got = g.gemm(ad, bd, epilogue=epilogue, config=c, trans_a=ta, trans_b=tb, alpha=alpha, splits=1)
            torch.cuda.synchronize()
            res = oracle.compare(u16(got), ref)
            assert res["pass"], (ta, tb, epilogue, alpha, c, res)


def test_power_of_two_scale_is_exact():
    """alpha = 2^e: the fp32 product is exact and RNE commutes with it, so
    the scaled result is the unscaled one times 2^e, bit for bit, wherever
    neither leaves the normal range (every layout, automatic configuration)."""
    M, N, K = 1024, 768, 1024
    for ta, tb in [(False, False), (False, True), (True, False), (True, True)]:
        _, _, a_st, b_st = stored_operands(M, N, K, ta, tb, 40 + 2 * ta + tb)
        ad, bd = a_st.to(DEV), b_st.to(DEV)
        plain = oracle.decode(u16(g.gemm(ad, bd, trans_a=ta, trans_b=tb, splits=1)))
        for e in (-3, 2):
            scaled = oracle.decode(u16(g.gemm(ad, bd, trans_a=ta, trans_b=tb, alpha=2.0 ** e, splits=1)))
            ok = (np.abs(plain) >= 2.0 ** -14) & (np.abs(plain) * 2.0 ** e >= 2.0 ** -14)
            assert ok.mean() > 0.9
            assert np.array_equal(scaled[ok], plain[ok] * 2.0 ** e), (ta, tb, e)
        one = u16(g.gemm(ad, bd, trans_a=ta, trans_b=tb, alpha=1.0, splits=1))
        assert np.array_equal(oracle.decode(one), plain)


def test_scaled_score_block_shape():
    """The score-block shape of an attention layer (2048 queries x 2304 keys,
    head dimension 1024 as K), B given N x K as in Q . K^T, scaled by the
    pages' 1/sqrt(dim) log2(e): full parity with the automatic choice."""
    M, N, K = 2048, 2304, 1024
    a, b, a_st, b_st = stored_operands(M, N, K, False, True, 50, dist="normal")
    alpha = qk_scale(K)
    got = g.gemm(a_st.to(DEV), b_st.to(DEV), trans_b=True, alpha=alpha, splits=1)
    torch.cuda.synchronize()
    res = oracle.compare(u16(got), oracle.gemm(u16(a), u16(b), scale=oracle.as_binary32(alpha)))
    assert res["pass"], res


def persistent_config():
    names = [g.config_name(c) for c in range(g.num_configs())]
    return [c for c, n in enumerate(names) if n.endswith("_persistent")]


@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_persistent_loop_many_tiles(ta, tb):
    """The persistent tile loop with more tiles than CUs (17 x 18 = 306
    tiles of 256 x 256 on 256 workgroups, so some run two tiles), ragged M
    and N and a K tail (K = 200: four slices, the last 8 deep), against the
    oracle; with ReLU and a scale too."""
    M, N, K = 4304, 4400, 200
    a, b, a_st, b_st = stored_operands(M, N, K, ta, tb, 70 + 2 * ta + tb)
    ad, bd = a_st.to(DEV), b_st.to(DEV)
    for c in persistent_config():
        p = g.plan(M, N, K, ad.data_ptr(), bd.data_ptr(), 1 << 20, config=c, trans_a=ta, trans_b=tb)
        assert p["grid"] == 256 and p["tiles_m"] * p["tiles_n"] == 306
        for epilogue, alpha in (("none", 1.0), ("relu", 0.375)):
            print(f"[persistent] ta={int(ta)} tb={int(tb)} config={c} epi={epilogue} alpha={alpha}", flush=True)
            ref = oracle.gemm(u16(a), u16(b), relu=(epilogue == "relu"), scale=alpha)
            got = g.gemm(ad, bd, epilogue=epilogue, config=c, trans_a=ta, trans_b=tb, alpha=alpha, splits=1)
            torch.cuda.synchronize()
            res = oracle.compare(u16(got), ref)
            assert res["pass"], (ta, tb, c, epilogue, res)


def test_persistent_loop_matches_one_tile_kernel():
    """Same tile, same MFMA order: the persistent loop and the one-tile
    kernel give identical bits on the 8192^3 workload."""
    w = workloads.WORKLOADS["gemm_8192"]
    a, b = workloads.make_inputs(w)
    ad, bd = a.to(DEV), b.to(DEV)
    one = g.gemm(ad, bd, config=g.plan(8192, 8192, 8192, 1 << 20, 1 << 20, 1 << 20)["config"], splits=1)
    for c in persistent_config():
        loop = g.gemm(ad, bd, config=c, splits=1)
        torch.cuda.synchronize()
        assert torch.equal(one, loop)


def test_prepared_call_matches_gemm():
    """prepare() checks and binds the tensors once; every call of the
    returned function enqueues the same product as gemm() (bitwise: the
    same plan and kernel), also when split or scaled or given transposed."""
    M, N, K = 520, 392, 200
    a, b = workloads.draw(M, N, K, "uniform", 77)
    ad, bd = a.to(DEV), b.to(DEV)
    bt = bd.t().contiguous()
    cases = [(bd, {}), (bd, {"epilogue": "relu"}), (bd, {"alpha": 0.5}), (bd, {"splits": 2}),
             (bd, {"config": configs_for(M, N, K)[0]}), (bt, {"trans_b": True})]
    for b_arg, kw in cases:
        print(f"[parity] prepared call {kw}", flush=True)
        want = g.gemm(ad, b_arg, **kw)
        out = torch.empty((M, N), dtype=torch.float16, device=DEV)
        call = g.prepare(ad, b_arg, out=out, **kw)
        for _ in range(3):
            out.fill_(float("nan"))
            assert call() is out
            torch.cuda.synchronize()
            assert torch.equal(out, want), kw
    res = oracle.compare(u16(out), oracle.gemm(u16(a), u16(b)))
    assert res["pass"], res

"""Seeded random cases of the dense and the 2:4-sparse products against the
oracle, through the C ABI.  Dense: shapes from 1 to 300 in each dimension
(ragged tails of every tile), the four layouts, operand and output pointers
offset by 0, 2, 4 or 8 bytes in their buffers (every alignment class), both
epilogues, a scale, and the automatic choice or any configuration that
accepts the case, with and without a K split.  Each case also checks that
nothing outside C is written.  The bar is the parity bar of the other tests
(max(2 ulp, 1e-3)).
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_fp16_amd as g
import workloads
from sp_layout import meta_flat

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = -1234.0


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def placed(host: torch.Tensor, offset_elems: int, guard: int = 32):
    """A device copy of `host` starting offset_elems elements into a buffer
    filled with the sentinel, and the buffer."""
    n = host.numel()
    buf = torch.full((n + offset_elems + guard,), SENTINEL, dtype=torch.float16, device=DEV)
    view = buf[offset_elems:offset_elems + n].view(host.shape)
    view.copy_(host.to(DEV))
    return view, buf


def accepting_configs(M, N, K, a, b, c, ta, tb):
    out = []
    for cfg in range(g.num_configs()):
        try:
            g.plan(M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr(), config=cfg, trans_a=ta, trans_b=tb)
            out.append(cfg)
        except g.GemmError:
            pass
    return out


@pytest.mark.parametrize("block", range(4))
def test_random_cases(block):
    rng = np.random.default_rng(20261203 + block)
    ws = torch.empty(16 * 300 * 300, dtype=torch.float32, device=DEV)
    sentinel = np.float16(SENTINEL).view(np.uint16)
    for case in range(100):
        M, N, K = (int(x) for x in rng.integers(1, 301, size=3))
        if rng.random() < 0.3:      # aligned pitches, so the direct kernels for 16-byte rows take part
            M, N, K = (max(8, (x // 8) * 8) for x in (M, N, K))
        ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        offs = [int(x) for x in rng.choice([0, 1, 2, 4], size=3)]     # elements: 0, 2, 4, 8 bytes
        epi = "relu" if rng.random() < 0.3 else "none"
        alpha = float(rng.choice([1.0, 1.0, 0.5, -2.0]))
        seed = int(rng.integers(1 << 30))
        a, b = workloads.draw(M, N, K, "uniform", seed)
        a_st = a.t().contiguous() if ta else a
        b_st = b.t().contiguous() if tb else b
        ad, _ = placed(a_st, offs[0])
        bd, _ = placed(b_st, offs[1])
        c_host = torch.zeros(M, N, dtype=torch.float16)
        cd, cbuf = placed(c_host, offs[2])
        cd.fill_(SENTINEL)
        cfgs = accepting_configs(M, N, K, ad, bd, cd, ta, tb)
        config = g.CONFIG_AUTO if rng.random() < 0.4 or not cfgs else int(rng.choice(cfgs))
        persistent = config != g.CONFIG_AUTO and "persistent" in g.config_name(config)
        splits = None if config == g.CONFIG_AUTO or persistent else int(rng.choice([1, 1, 2, 3]))
        label = (f"case {block}.{case}: {M}x{N}x{K} ta={ta} tb={tb} offsets={offs} epi={epi} alpha={alpha} "
                 f"config={g.config_name(config) if config >= 0 else 'auto'} splits={splits} seed={seed}")
        print(label, flush=True)
        kw = {}
        if splits is not None:
            kw = {"splits": splits, "workspace": ws}
        g.gemm(ad, bd, epilogue=epi, out=cd, config=config, trans_a=ta, trans_b=tb, alpha=alpha, **kw)
        torch.cuda.synchronize()
        ref = oracle.gemm(u16(a), u16(b), relu=(epi == "relu"), scale=alpha)   # 0.5 and -2 are exact in binary32
        res = oracle.compare(u16(cd), ref)
        assert res["pass"], (label, res)
        host = u16(cbuf)
        assert np.all(host[:offs[2]] == sentinel) and np.all(host[offs[2] + M * N:] == sentinel), label


@pytest.mark.parametrize("block", range(2))
def test_random_sparse_cases(block):
    """The 2:4-sparse product on seeded random cases: M and N from 1 to 300
    (N a multiple of 8 when B is K x N), K a multiple of 16 up to 320 (whole
    and partial 64-deep slices), B as stored or given N x K, C offset by 0,
    2 or 8 bytes, both epilogues, the automatic or any accepting
    configuration.  The library's compression must equal the oracle's, bit
    for bit, and the product the oracle's product of the oracle's operands."""
    rng = np.random.default_rng(991 + block)
    sentinel = np.float16(SENTINEL).view(np.uint16)
    for case in range(50):
        M, K = int(rng.integers(1, 301)), 16 * int(rng.integers(1, 21))
        tb = bool(rng.integers(2))
        N = int(rng.integers(1, 301))
        if not tb:
            N = max(8, (N // 8) * 8)
        epi = "relu" if rng.random() < 0.3 else "none"
        seed = int(rng.integers(1 << 30))
        a, b = workloads.draw(M, N, K, "uniform", seed)
        v_ref, m_ref = oracle.sp_compress(u16(a))
        vals, meta = g.sp_compress(a.to(DEV))
        torch.cuda.synchronize()
        label = f"sparse case {block}.{case}: {M}x{N}x{K} tb={tb} epi={epi} seed={seed}"
        assert np.array_equal(u16(vals), v_ref), label
        assert np.array_equal(u16(meta), meta_flat(m_ref)), label
        bd = (b.t().contiguous() if tb else b).to(DEV)
        off = int(rng.choice([0, 1, 4]))
        cd, cbuf = placed(torch.zeros(M, N, dtype=torch.float16), off)
        cd.fill_(SENTINEL)
        cfgs = []
        for cfg in range(g.sp_num_configs()):
            try:
                g.plan_sp(M, N, K, vals.data_ptr(), meta.data_ptr(), bd.data_ptr(), cd.data_ptr(), config=cfg,
                          trans_b=tb)
                cfgs.append(cfg)
            except g.GemmError:
                pass
        config = g.CONFIG_AUTO if rng.random() < 0.4 or not cfgs else int(rng.choice(cfgs))
        print(f"{label} offset={off} config={config}", flush=True)
        g.gemm_sp(vals, meta, bd, epilogue=epi, out=cd, config=config, trans_b=tb)
        torch.cuda.synchronize()
        res = oracle.compare(u16(cd), oracle.gemm_sp(v_ref, m_ref, u16(b), relu=(epi == "relu")))
        assert res["pass"], (label, res)
        host = u16(cbuf)
        assert np.all(host[:off] == sentinel) and np.all(host[off + M * N:] == sentinel), label


def test_random_large_cases_sampled():
    """Seeded random large shapes (257 to 5000 in each dimension), each
    layout and alignment, the automatic choice (which for such grids picks
    the 256-wide tiles and their tile remap over many rounds): a seeded
    sample of rows and columns, with the first and last, against the oracle."""
    rng = np.random.default_rng(4242)
    for case in range(16):
        M, N, K = (int(x) for x in rng.integers(257, 5001, size=3))
        if case % 2 == 0:
            M, N, K = ((x // 8) * 8 for x in (M, N, K))
        ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        seed = int(rng.integers(1 << 30))
        a, b = workloads.draw(M, N, K, "normal", seed)
        ad = (a.t().contiguous() if ta else a).to(DEV)
        bd = (b.t().contiguous() if tb else b).to(DEV)
        p = g.plan(M, N, K, ad.data_ptr(), bd.data_ptr(), 1 << 20, trans_a=ta, trans_b=tb)
        label = f"large case {case}: {M}x{N}x{K} ta={ta} tb={tb} seed={seed} config={g.config_name(p['config'])}"
        print(label, flush=True)
        out = g.gemm(ad, bd, trans_a=ta, trans_b=tb, splits=1)
        torch.cuda.synchronize()
        rows = sorted(set(rng.choice(M, size=48, replace=False).tolist() + [0, M - 1]))
        cols = sorted(set(rng.choice(N, size=48, replace=False).tolist() + [0, N - 1]))
        got = u16(out[torch.tensor(rows, device=DEV)][:, torch.tensor(cols, device=DEV)])
        res = oracle.compare(got, oracle.gemm_sampled(u16(a), u16(b), rows, cols))
        assert res["pass"], (label, res)

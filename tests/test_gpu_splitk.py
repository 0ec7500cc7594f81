"""GPU parity of split-K runs against the CPU oracle, through the C ABI.

A split run divides the K loop of every output tile among workgroups, writes
fp32 partial sums to a caller-provided workspace and adds them in split order
in a second kernel, which also applies the epilogue and the single rounding
to fp16.  It computes the same function as the unsplit kernel (the tile GEMM
of "TileLang：比 Triton 低一层的 tile 语言", section "第一个 kernel：GEMM"; the
persistent / stream-K GEMM variants that "5分钟上手TileLang：GPU内核开发指南",
section "进阶方向：从 GEMM 到真实模型算子", lists are the scheduling this
stands in for), so the bar is the same: every element within max(2 fp16 ulps,
1e-3) of the oracle, bitwise determinism, no write outside C.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_fp16_amd as g
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FAKE = 1 << 20


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def configs_for(M, N, K, ta=False, tb=False):
    """Every configuration with a split form (all but the persistent loop)
    that accepts this shape."""
    out = []
    for c in range(g.num_configs()):
        if "persistent" in g.config_name(c):
            continue
        try:
            g.plan(M, N, K, FAKE, FAKE, FAKE, config=c, trans_a=ta, trans_b=tb)
            out.append(c)
        except g.GemmError:
            pass
    return out


def stored(M, N, K, ta, tb, seed):
    a, b = workloads.draw(M, N, K, "uniform", seed)
    return (a.t().contiguous() if ta else a), (b.t().contiguous() if tb else b)


class Case:
    """Operands on the GPU and the oracle's result, computed once."""

    def __init__(self, M, N, K, ta=False, tb=False, seed=0):
        self.M, self.N, self.K, self.ta, self.tb = M, N, K, ta, tb
        self.a, self.b = stored(M, N, K, ta, tb, seed)
        self.ad, self.bd = self.a.to(DEV), self.b.to(DEV)
        self._ref = {}

    def ref(self, epilogue):
        if epilogue not in self._ref:
            self._ref[epilogue] = oracle.gemm(u16(self.a), u16(self.b), relu=(epilogue == "relu"),
                                              trans_a=self.ta, trans_b=self.tb)
        return self._ref[epilogue]

    def run(self, config, splits, epilogue="none", workspace=None, out=None):
        p = g.plan(self.M, self.N, self.K, self.ad.data_ptr(), self.bd.data_ptr(), FAKE, config=config,
                   trans_a=self.ta, trans_b=self.tb, splits=splits)
        print(f"[split] {self.M}x{self.N}x{self.K} ta={int(self.ta)} tb={int(self.tb)} epi={epilogue} "
              f"config={p['config']} splits={p['splits']} k_split={p['k_split']}", flush=True)
        c = g.gemm(self.ad, self.bd, epilogue=epilogue, config=config, trans_a=self.ta, trans_b=self.tb,
                   splits=splits, workspace=workspace, out=out)
        torch.cuda.synchronize()
        return u16(c), p

    def check(self, config, splits, epilogue="none", **kw):
        got, p = self.run(config, splits, epilogue, **kw)
        res = oracle.compare(got, self.ref(epilogue))
        assert res["pass"], (config, splits, epilogue, res)
        return got, p


# several tiles, ragged M and N, K not a multiple of the split length
SPLIT_SHAPES = [(300, 264, 1000), (64, 64, 4096), (257, 520, 200), (1, 8, 520), (130, 72, 777)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_every_config_split(shape):
    case = Case(*shape, seed=sum(shape))
    cfgs = configs_for(*shape)
    assert len(cfgs) >= 2
    for c in cfgs:
        for splits in (2, 3, 7):
            _, p = case.check(c, splits)
            nk = -(-shape[2] // p["block_k"])
            per = -(-nk // splits)
            assert p["splits"] == -(-nk // per) and p["k_split"] == per * p["block_k"]


def test_split_relu():
    case = Case(300, 264, 1000, seed=5)
    for c in configs_for(300, 264, 1000):
        case.check(c, 4, "relu")


def test_split_unaligned_n():
    # N % 4 != 0: partial sums leave as 4-byte stores, the reduction runs per element
    for shape in [(130, 70, 777), (37, 45, 530), (65, 66, 3000)]:
        case = Case(*shape, seed=shape[1])
        for c in configs_for(*shape):
            for splits in (2, 5):
                case.check(c, splits)
                case.check(c, splits, "relu")


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
def test_split_transposed(ta, tb):
    for shape in [(300, 264, 1032), (130, 129, 1067)]:
        case = Case(*shape, ta=ta, tb=tb, seed=3 + shape[2])
        for c in configs_for(*shape, ta, tb):
            case.check(c, 3)


def test_split_counts_clamped():
    # more splits requested than k tiles: one k tile per split
    case = Case(200, 136, 128, seed=9)
    _, p = case.check(2, 8)
    assert p["splits"] == 2
    # fewer than two k tiles: unsplit
    case = Case(200, 136, 40, seed=10)
    _, p = case.check(2, 8)
    assert p["splits"] == 1


def test_split_zero_k():
    a = torch.empty((70, 0), dtype=torch.float16, device=DEV)
    b = torch.empty((0, 90), dtype=torch.float16, device=DEV)
    for config in (4, g.CONFIG_AUTO):
        c = torch.full((70, 90), 3.0, dtype=torch.float16, device=DEV)
        g.gemm(a, b, out=c, config=config, splits=4)
        torch.cuda.synchronize()
        assert torch.count_nonzero(c).item() == 0


def test_caller_workspace_matches_binding_workspace():
    """The binding's own workspace (torch's caching allocator) and a caller's
    tensor give bit-identical results; the C call without one is refused."""
    case = Case(300, 264, 1000, seed=11)
    own_out, p = case.check(2, 4)
    need = p["workspace_bytes"]
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    got, _ = case.check(2, 4, workspace=ws)
    assert np.array_equal(own_out, got)
    # a buffer one element short is refused before anything runs
    with pytest.raises(g.GemmError) as e:
        case.run(2, 4, workspace=ws[:-1])
    assert e.value.status == 7
    out = torch.empty((300, 264), dtype=torch.float16, device=DEV)
    st = g.lib().gemm_f16_split(300, 264, 1000, case.ad.data_ptr(), 0, case.bd.data_ptr(), 0, out.data_ptr(), 0,
                                2, 4, None, 0, None)
    assert st == 7


def test_split_deterministic_and_guarded():
    M, N, K = 300, 264, 2000
    case = Case(M, N, K, seed=12)
    guard = 4096
    sentinel = np.float16(-1234.0).view(np.uint16)
    first = None
    for _ in range(3):
        buf = torch.full((M * N + 2 * guard,), -1234.0, dtype=torch.float16, device=DEV)
        got, _ = case.check(2, 6, out=buf[guard:guard + M * N].view(M, N))
        host = u16(buf)
        assert np.all(host[:guard] == sentinel) and np.all(host[guard + M * N:] == sentinel)
        if first is None:
            first = got
        assert np.array_equal(got, first)


def test_automatic_choice_splits_deep_k():
    """Far from every tuned shape a small output over a deep K is split by
    the model when a workspace may be used (the binding supplies one); the
    workspace-free C entry point runs the same shape in one kernel.  Both
    match the oracle."""
    M, N, K = 96, 96, 30000
    p = g.plan(M, N, K, FAKE, FAKE, FAKE, splits=g.SPLITS_AUTO)
    assert p["splits"] > 1, p
    assert g.plan(M, N, K, FAKE, FAKE, FAKE)["splits"] == 1
    case = Case(M, N, K, seed=15)
    print(f"[split] auto plan config={p['config']} splits={p['splits']}", flush=True)
    c = g.gemm(case.ad, case.bd)
    torch.cuda.synchronize()
    res = oracle.compare(u16(c), case.ref("none"))
    assert res["pass"], res
    c1 = torch.empty((M, N), dtype=torch.float16, device=DEV)
    st = g.gemm_f16_raw(M, N, K, case.ad.data_ptr(), case.bd.data_ptr(), c1.data_ptr(), 0,
                        torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    res = oracle.compare(u16(c1), case.ref("none"))
    assert res["pass"], res


def test_split_in_a_captured_graph():
    """Replays of a captured split call (its workspace drawn from the graph's
    memory pool by the binding) match the eager result every time, with
    eager work and synchronisations between the replays."""
    M, N, K = 96, 96, 30000
    case = Case(M, N, K, seed=16)
    ref = case.ref("none")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = torch.empty((M, N), dtype=torch.float16, device=DEV)
    with torch.cuda.stream(side):
        g.gemm(case.ad, case.bd, out=out)
    side.synchronize()
    eager = u16(out)
    assert oracle.compare(eager, ref)["pass"]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        g.gemm(case.ad, case.bd, out=out)
    for _ in range(3):
        out.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(u16(out), eager)
        g.gemm(case.ad, case.bd, splits=3)     # eager split work between the replays
        torch.cuda.synchronize()
    del graph


def test_prepared_calls_in_a_captured_graph():
    """prepare() takes a split's workspace when it binds the call, so a graph
    of prepared calls records kernels only; every replay (with eager work and
    synchronisations between) matches the eager results."""
    split_case = Case(96, 96, 30000, seed=17)
    plain_case = Case(520, 392, 200, tb=True, seed=18)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out1 = torch.empty((96, 96), dtype=torch.float16, device=DEV)
    out2 = torch.empty((520, 392), dtype=torch.float16, device=DEV)
    with torch.cuda.stream(side):
        p1 = g.prepare(split_case.ad, split_case.bd, out=out1, splits=3, epilogue="relu")
        p2 = g.prepare(plain_case.ad, plain_case.bd, out=out2, trans_b=True, alpha=0.5)
        p1()
        p2()
    side.synchronize()
    e1, e2 = u16(out1), u16(out2)
    assert oracle.compare(e1, split_case.ref("relu"))["pass"]
    assert oracle.compare(e2, oracle.gemm(u16(plain_case.a), u16(plain_case.b), trans_b=True, scale=0.5))["pass"]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        p1()
        p2()
    for _ in range(3):
        out1.fill_(7.0)
        out2.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(u16(out1), e1) and np.array_equal(u16(out2), e2)
        g.gemm(split_case.ad, split_case.bd, splits=2)     # eager split work between the replays
        torch.cuda.synchronize()
    del graph


def test_split_scaled():
    """The scale of the scaled entry points on the split path: the reduction
    multiplies the sum of the partials by alpha before the ReLU."""
    for ta, tb, shape in [(False, False, (300, 264, 1000)), (False, True, (130, 72, 777)),
                          (True, True, (257, 520, 600))]:
        case = Case(*shape, ta=ta, tb=tb, seed=60 + shape[2])
        for alpha, epilogue in ((-0.6, "relu"), (0.0883883, "none")):
            ref = oracle.gemm(u16(case.a), u16(case.b), relu=(epilogue == "relu"), trans_a=ta, trans_b=tb,
                              scale=oracle.as_binary32(alpha))
            for c in configs_for(*shape, ta, tb):
                print(f"[split-scaled] {shape} ta={int(ta)} tb={int(tb)} config={c} alpha={alpha}", flush=True)
                out = g.gemm(case.ad, case.bd, epilogue=epilogue, config=c, trans_a=ta, trans_b=tb, splits=3,
                             alpha=alpha)
                torch.cuda.synchronize()
                res = oracle.compare(u16(out), ref)
                assert res["pass"], (shape, c, alpha, res)

"""GPU check of the allocation-free split entry point, through the C ABI.

gemm_f16_split_static keeps the split-K partial sums in a static device
array instead of a caller's workspace.  It runs the same kernels as
gemm_f16_split, so on the same inputs, configuration and split count its
output must equal gemm_f16_split's bit for bit, and both must match the CPU
oracle within max(2 fp16 ulps, 1e-3).  Two calls in a row, the second on a
smaller problem, check that the scratch left by the first call does not leak
into the second.
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


# (M, N, K, config, split request, epilogue, trans_a, trans_b, seed); the first
# is the larger problem, so the second call runs on scratch the first one filled
CALLS = [
    (1024, 1024, 8192, g.CONFIG_AUTO, g.SPLITS_AUTO, "relu", False, False, 21),
    (300, 264, 1000, 2, 3, "none", False, True, 22),
]


def test_static_scratch_matches_caller_workspace_two_calls():
    stream = torch.cuda.current_stream()
    for M, N, K, config, splits, epi, ta, tb, seed in CALLS:
        a, b = workloads.draw(M, N, K, "uniform", seed)
        a_st = a.t().contiguous() if ta else a
        b_st = b.t().contiguous() if tb else b
        ad, bd = a_st.to(DEV), b_st.to(DEV)
        plan = g.plan(M, N, K, ad.data_ptr(), bd.data_ptr(), 1 << 20, config=config, trans_a=ta, trans_b=tb,
                      splits=splits)
        print(f"[no-alloc] {M}x{N}x{K} ta={int(ta)} tb={int(tb)} epi={epi} config={plan['config']} "
              f"splits={plan['splits']} workspace={plan['workspace_bytes']}", flush=True)
        assert plan["splits"] > 1 and 0 < plan["workspace_bytes"] <= g.STATIC_WORKSPACE_BYTES
        ws = torch.empty(plan["workspace_bytes"] // 4, dtype=torch.float32, device=DEV)
        c_ws = torch.full((M, N), -7.0, dtype=torch.float16, device=DEV)
        c_static = torch.full((M, N), 5.0, dtype=torch.float16, device=DEV)
        epi_code = 1 if epi == "relu" else 0
        st = g.lib().gemm_f16_split(M, N, K, ad.data_ptr(), int(ta), bd.data_ptr(), int(tb), c_ws.data_ptr(),
                                    epi_code, config, splits, ws.data_ptr(), plan["workspace_bytes"],
                                    stream.cuda_stream)
        assert st == 0, g.status_string(st)
        st = g.lib().gemm_f16_split_static(M, N, K, ad.data_ptr(), int(ta), bd.data_ptr(), int(tb),
                                           c_static.data_ptr(), epi_code, config, splits, stream.cuda_stream)
        assert st == 0, g.status_string(st)
        torch.cuda.synchronize()
        got, want = u16(c_static), u16(c_ws)
        assert np.array_equal(got, want), "static scratch and caller workspace differ"
        ref = oracle.gemm(u16(a), u16(b), relu=(epi == "relu"))
        res = oracle.compare(got, ref)
        assert res["pass"], res


def test_static_scratch_limit():
    # 4096 x 4096 x 8192 split 2 needs 128 MiB of partial sums: refused before any launch
    a = torch.zeros((4096, 8192), dtype=torch.float16, device=DEV)
    b = torch.zeros((8192, 4096), dtype=torch.float16, device=DEV)
    c = torch.full((4096, 4096), 3.0, dtype=torch.float16, device=DEV)
    st = g.lib().gemm_f16_split_static(4096, 4096, 8192, a.data_ptr(), 0, b.data_ptr(), 0, c.data_ptr(), 0,
                                       2, 2, torch.cuda.current_stream().cuda_stream)
    assert st == 9
    torch.cuda.synchronize()
    assert bool((c == 3.0).all())

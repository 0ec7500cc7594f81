"""Python binding of the gfx950 FP16 GEMM library (libgemm_f16.so).

Argument marshalling only: every step of C = epi(A . B) runs in the HIP
kernels behind the C ABI declared in ``include/gemm_f16.h``.  PyTorch is
used for device memory and streams.  There is no fallback: if the library
has not been built, or the GPU is not a gfx950, calls raise.

The tile program this implements is the GEMM of "TileLang：比 Triton 低一层的
tile 语言" (section "第一个 kernel：GEMM"): C is returned as a new tensor
unless ``out`` is given, as the pages' kernels allocate their output.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_f16.so")
PROBE_LIB_PATH = os.path.join(_HERE, "libgemm_f16_probe.so")

SUCCESS = 0
EPILOGUE_NONE = 0
EPILOGUE_RELU = 1
CONFIG_AUTO = -1
SPLITS_AUTO = 0
MAX_SPLITS = 64
STATIC_WORKSPACE_BYTES = 32 << 20
_EPILOGUES = {"none": EPILOGUE_NONE, "relu": EPILOGUE_RELU}

# exported symbols and their ctypes signatures (mirrors include/gemm_f16.h)
_i64, _vp, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int


class Plan(ctypes.Structure):
    """gemm_f16_plan_t: how a call would run."""
    _fields_ = [
        ("config", ctypes.c_int32), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
        ("block_k", ctypes.c_int32), ("stages", ctypes.c_int32), ("threads", ctypes.c_int32),
        ("direct_lds", ctypes.c_int32), ("vec_a", ctypes.c_int32), ("vec_b", ctypes.c_int32),
        ("vec_c", ctypes.c_int32), ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64),
        ("grid", ctypes.c_int64), ("k_tiles", ctypes.c_int64), ("lds_bytes", ctypes.c_int64),
        ("flops", ctypes.c_double), ("min_bytes", ctypes.c_double),
        ("trans_a", ctypes.c_int32), ("trans_b", ctypes.c_int32),
        ("splits", ctypes.c_int32), ("k_split", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


SIGNATURES = {
    "gemm_f16": ([_i64, _i64, _i64, _vp, _vp, _vp, _int, _vp], _int),
    "gemm_f16_ex": ([_i64, _i64, _i64, _vp, _vp, _vp, _int, _int, _vp], _int),
    "gemm_f16_trans": ([_i64, _i64, _i64, _vp, _int, _vp, _int, _vp, _int, _int, _vp], _int),
    "gemm_f16_plan": ([_i64, _i64, _i64, _vp, _vp, _vp, _int, ctypes.POINTER(Plan)], _int),
    "gemm_f16_split": ([_i64, _i64, _i64, _vp, _int, _vp, _int, _vp, _int, _int, _int, _vp, _i64, _vp], _int),
    "gemm_f16_split_static": ([_i64, _i64, _i64, _vp, _int, _vp, _int, _vp, _int, _int, _int, _vp], _int),
    "gemm_f16_scaled": ([_i64, _i64, _i64, _vp, _int, _vp, _int, _vp, ctypes.c_float, _int, _int, _vp], _int),
    "gemm_f16_split_scaled": ([_i64, _i64, _i64, _vp, _int, _vp, _int, _vp, ctypes.c_float, _int, _int, _int,
                               _vp, _i64, _vp], _int),
    "gemm_f16_plan_trans": ([_i64, _i64, _i64, _vp, _int, _vp, _int, _vp, _int, ctypes.POINTER(Plan)], _int),
    "gemm_f16_plan_split": ([_i64, _i64, _i64, _vp, _int, _vp, _int, _vp, _int, _int, ctypes.POINTER(Plan)],
                            _int),
    "gemm_f16_sp_compress": ([_i64, _i64, _vp, _vp, _vp, _vp], _int),
    "gemm_f16_sp": ([_i64, _i64, _i64, _vp, _vp, _vp, _int, _vp, _int, _int, _vp], _int),
    "gemm_f16_plan_sp": ([_i64, _i64, _i64, _vp, _vp, _vp, _int, _vp, _int, ctypes.POINTER(Plan)], _int),
    "gemm_f16_sp_num_configs": ([], _int),
    "gemm_f16_sp_config_name": ([_int], ctypes.c_char_p),
    "gemm_f16_num_configs": ([], _int),
    "gemm_f16_config_name": ([_int], ctypes.c_char_p),
    "gemm_f16_stage_bytes": ([_i64, _i64, _i64, _i64], _i64),
    "gemm_f16_status_string": ([_int], ctypes.c_char_p),
}

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


def _load_hip_runtime_first():
    """torch ships its own copy of the HIP runtime (same soname as the
    system's).  Loading it before the library makes the library bind to that
    copy; loaded the other way round the process holds two runtimes, and the
    library's, which does not own torch's streams and allocations, reports no
    device."""
    import torch  # noqa: F401


def lib() -> ctypes.CDLL:
    """Load libgemm_f16.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        _load_hip_runtime_first()
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().gemm_f16_status_string(int(status)).decode()


def num_configs() -> int:
    return int(lib().gemm_f16_num_configs())


def config_name(config: int) -> str | None:
    s = lib().gemm_f16_config_name(int(config))
    return s.decode() if s is not None else None


def stage_bytes(block_m: int, block_n: int, block_k: int, stages: int) -> int:
    return int(lib().gemm_f16_stage_bytes(block_m, block_n, block_k, stages))


def plan(M: int, N: int, K: int, A_ptr: int = 0, B_ptr: int = 0, C_ptr: int = 0,
         config: int = CONFIG_AUTO, trans_a: bool = False, trans_b: bool = False,
         splits: int | None = None) -> dict:
    """How a call would run this shape (pure host logic, no GPU needed):
    gemm_f16 / gemm_f16_trans (never split) when ``splits`` is None, else
    gemm_f16_split with that request (SPLITS_AUTO: the planner's choice).
    Pointers only matter for alignment; 0 stands for an aligned buffer."""
    p = Plan()
    if splits is None:
        st = lib().gemm_f16_plan_trans(M, N, K, A_ptr or None, int(trans_a), B_ptr or None, int(trans_b),
                                       C_ptr or None, config, ctypes.byref(p))
    else:
        st = lib().gemm_f16_plan_split(M, N, K, A_ptr or None, int(trans_a), B_ptr or None, int(trans_b),
                                       C_ptr or None, config, int(splits), ctypes.byref(p))
    if st != SUCCESS:
        raise GemmError(st, "gemm_f16_plan")
    return p.as_dict()


def gemm_f16_raw(M: int, N: int, K: int, A_ptr: int, B_ptr: int, C_ptr: int, epilogue: int = 0,
                 stream: int = 0, config: int = CONFIG_AUTO, trans_a: bool = False,
                 trans_b: bool = False) -> int:
    """Call the C entry points with raw device addresses; returns the status code."""
    A, B, C, S = A_ptr or None, B_ptr or None, C_ptr or None, stream or None
    if trans_a or trans_b:
        return int(lib().gemm_f16_trans(M, N, K, A, int(trans_a), B, int(trans_b), C, epilogue, config, S))
    if config == CONFIG_AUTO:
        return int(lib().gemm_f16(M, N, K, A, B, C, epilogue, S))
    return int(lib().gemm_f16_ex(M, N, K, A, B, C, epilogue, config, S))


_split_plans: dict = {}


def _auto_split(M, N, K, a, b, out, config, trans_a, trans_b, splits):
    """(splits, workspace_bytes) that gemm_f16_split would use for this call,
    cached per shape, layout, configuration and pointer alignment."""
    key = (M, N, K, a.data_ptr() % 16, b.data_ptr() % 16, out.data_ptr() % 16, config, trans_a, trans_b, splits)
    hit = _split_plans.get(key)
    if hit is None:
        p = plan(M, N, K, a.data_ptr() or 16, b.data_ptr() or 16, out.data_ptr() or 16, config=config,
                 trans_a=trans_a, trans_b=trans_b, splits=splits)
        hit = (p["splits"], p["workspace_bytes"])
        if len(_split_plans) > 4096:
            _split_plans.clear()
        _split_plans[key] = hit
    return hit


def _bind(a, b, epilogue, out, config, stream, trans_a, trans_b, splits, workspace, alpha):
    """Check the arguments of gemm()/prepare() and choose the entry point:
    (the C function, its arguments, out, the tensors the call uses)."""
    import torch

    if epilogue not in _EPILOGUES:
        raise ValueError(f"epilogue must be one of {sorted(_EPILOGUES)}, got {epilogue!r}")
    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D torch.float16 tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (row-major)")
    K, M = a.shape if trans_a else (a.shape[1], a.shape[0])
    N, K2 = b.shape if trans_b else (b.shape[1], b.shape[0])
    if K != K2:
        raise ValueError(f"inner dimensions differ: a is {tuple(a.shape)} (trans_a={trans_a}), "
                         f"b is {tuple(b.shape)} (trans_b={trans_b})")
    if a.device != b.device:
        raise ValueError("a and b are on different devices")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=a.device)
    elif (out.dtype != torch.float16 or tuple(out.shape) != (M, N) or not out.is_contiguous()
          or out.device != a.device):
        raise ValueError(f"out must be a contiguous float16 tensor of shape {(M, N)} on {a.device}")
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        if workspace.device != a.device:
            raise ValueError("workspace is on another device")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    request = SPLITS_AUTO if splits is None else int(splits)
    if workspace is None and request != 1 and M > 0 and N > 0:
        n_split, ws_bytes = _auto_split(M, N, K, a, b, out, config, trans_a, trans_b, request)
        if n_split > 1:
            with torch.cuda.device(a.device), torch.cuda.stream(stream):
                workspace = torch.empty(-(-ws_bytes // 4), dtype=torch.float32, device=a.device)
        else:
            request = 1
    S = stream.cuda_stream or None
    A, B, C = a.data_ptr() or None, b.data_ptr() or None, out.data_ptr() or None
    epi = _EPILOGUES[epilogue]
    scaled = float(alpha) != 1.0
    h = lib()
    if workspace is None and request in (1, SPLITS_AUTO):
        if scaled:
            fn, args = h.gemm_f16_scaled, (M, N, K, A, int(trans_a), B, int(trans_b), C, float(alpha), epi, config, S)
        elif trans_a or trans_b:
            fn, args = h.gemm_f16_trans, (M, N, K, A, int(trans_a), B, int(trans_b), C, epi, config, S)
        elif config == CONFIG_AUTO:
            fn, args = h.gemm_f16, (M, N, K, A, B, C, epi, S)
        else:
            fn, args = h.gemm_f16_ex, (M, N, K, A, B, C, epi, config, S)
    else:
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        head = (M, N, K, A, int(trans_a), B, int(trans_b), C)
        if scaled:
            fn, args = h.gemm_f16_split_scaled, head + (float(alpha), epi, config, request, ws_ptr or None, ws_bytes, S)
        else:
            fn, args = h.gemm_f16_split, head + (epi, config, request, ws_ptr or None, ws_bytes, S)
    return fn, args, out, (a, b, out, workspace, stream)


def gemm(a, b, epilogue: str = "none", out=None, config: int = CONFIG_AUTO, stream=None,
         trans_a: bool = False, trans_b: bool = False, splits: int | None = None, workspace=None,
         alpha: float = 1.0):
    """C = epi(alpha * (op(a) @ op(b))) for 2-D contiguous float16 GPU tensors.

    a is M x K (or K x M with ``trans_a``), b is K x N (or N x K with
    ``trans_b``).  Returns ``out`` (allocated as an M x N float16 tensor when
    not given).  The kernels are enqueued on ``stream`` (default: torch's
    current stream) and the call returns without synchronising.

    ``splits``: None lets the planner split K when that pays for the shape
    (gemm_f16_split with SPLITS_AUTO), 1 runs one kernel (gemm_f16 /
    gemm_f16_ex / gemm_f16_trans), a larger count asks for that split.  A
    split needs a workspace of fp32 partial sums: ``workspace`` (a contiguous
    GPU tensor used as scratch) or, when it is None, one taken from torch's
    caching allocator on ``stream`` for this call.  The C library itself
    never allocates.  ``alpha`` (taken as an fp32 value) scales the result
    before the epilogue (gemm_f16_scaled / gemm_f16_split_scaled).
    """
    import torch

    fn, args, out, _ = _bind(a, b, epilogue, out, config, stream, trans_a, trans_b, splits, workspace, alpha)
    with torch.cuda.device(a.device):
        st = fn(*args)
    if st != SUCCESS:
        raise GemmError(st, "gemm_f16")
    return out


def prepare(a, b, epilogue: str = "none", out=None, config: int = CONFIG_AUTO, stream=None,
            trans_a: bool = False, trans_b: bool = False, splits: int | None = None, workspace=None,
            alpha: float = 1.0):
    """gemm() bound to fixed tensors, for loops that repeat one product on
    the same buffers (serving, benchmarks).

    Takes gemm()'s arguments, checks them and makes the split decision once
    (a split's workspace is allocated here, once), and returns a function of
    no arguments that enqueues the product on ``stream`` and returns
    ``out``; the C library still validates and plans every call (from its
    per-thread plan cache).  The bound tensors must stay in place: the
    function keeps references to them, not copies.  Call it with the
    tensors' device current."""
    fn, args, out, keep = _bind(a, b, epilogue, out, config, stream, trans_a, trans_b, splits, workspace, alpha)

    def call():
        st = fn(*args)
        if st != SUCCESS:
            raise GemmError(st, "gemm_f16")
        return out

    call.out = out
    call.bound = keep
    return call


# ---- 2:4 structured-sparse A (gemm_f16_sp*, see include/gemm_f16.h) --------

def sp_num_configs() -> int:
    return int(lib().gemm_f16_sp_num_configs())


def sp_config_name(config: int) -> str | None:
    s = lib().gemm_f16_sp_config_name(int(config))
    return s.decode() if s is not None else None


def plan_sp(M: int, N: int, K: int, vals_ptr: int = 0, meta_ptr: int = 0, B_ptr: int = 0, C_ptr: int = 0,
            config: int = CONFIG_AUTO, trans_b: bool = False) -> dict:
    """How gemm_f16_sp would run this shape (host logic only)."""
    p = Plan()
    st = lib().gemm_f16_plan_sp(M, N, K, vals_ptr or None, meta_ptr or None, B_ptr or None, int(trans_b),
                                C_ptr or None, config, ctypes.byref(p))
    if st != SUCCESS:
        raise GemmError(st, "gemm_f16_plan_sp")
    return p.as_dict()


def _check_gpu_2d(t, name, dtype):
    import torch

    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D {dtype} tensor")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")


def sp_compress(a, stream=None):
    """(vals, meta) for a (M x K float16 GPU tensor, K % 16 == 0): vals is
    M x K/2 float16, meta the M K/16 uint16 position words (as int16 bits) in
    the slice-major order include/gemm_f16.h gives, a 1-D tensor."""
    import torch

    _check_gpu_2d(a, "a", torch.float16)
    M, K = a.shape
    vals = torch.empty((M, K // 2), dtype=torch.float16, device=a.device)
    meta = torch.empty((M * (K // 16),), dtype=torch.int16, device=a.device)
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        st = lib().gemm_f16_sp_compress(M, K, a.data_ptr() or None, vals.data_ptr() or None,
                                        meta.data_ptr() or None, stream.cuda_stream or None)
    if st != SUCCESS:
        raise GemmError(st, "gemm_f16_sp_compress")
    return vals, meta


def gemm_sp(vals, meta, b, epilogue: str = "none", out=None, config: int = CONFIG_AUTO, stream=None,
            trans_b: bool = False):
    """C = epi(A @ op(b)) for a 2:4-sparse A given as (vals, meta) from
    sp_compress; b is K x N, or N x K with ``trans_b``."""
    import torch

    if epilogue not in _EPILOGUES:
        raise ValueError(f"epilogue must be one of {sorted(_EPILOGUES)}, got {epilogue!r}")
    _check_gpu_2d(vals, "vals", torch.float16)
    if (not isinstance(meta, torch.Tensor) or meta.dtype != torch.int16 or meta.dim() != 1 or not meta.is_cuda
            or not meta.is_contiguous()):
        raise ValueError("meta must be a 1-D contiguous int16 GPU tensor (as sp_compress returns)")
    _check_gpu_2d(b, "b", torch.float16)
    M, K = vals.shape[0], 2 * vals.shape[1]
    kb, N = (b.shape[1], b.shape[0]) if trans_b else (b.shape[0], b.shape[1])
    if meta.numel() != M * (K // 16) or kb != K:
        raise ValueError(f"shape mismatch: vals {tuple(vals.shape)}, meta {tuple(meta.shape)}, b {tuple(b.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=b.device)
    elif out.dtype != torch.float16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float16 tensor of shape {(M, N)}")
    if stream is None:
        stream = torch.cuda.current_stream(b.device)
    with torch.cuda.device(b.device):
        st = lib().gemm_f16_sp(M, N, K, vals.data_ptr() or None, meta.data_ptr() or None, b.data_ptr() or None,
                               int(trans_b), out.data_ptr() or None, _EPILOGUES[epilogue], config,
                               stream.cuda_stream or None)
    if st != SUCCESS:
        raise GemmError(st, "gemm_f16_sp")
    return out


# ---- measurement probe (libgemm_f16_probe.so, include/gemm_f16_probe.h) ----

PROBE_CONSTANT, PROBE_RANDOM_FIXED, PROBE_RANDOM_CHANGING = 0, 1, 2
PROBE_LAYOUT_32X32X16, PROBE_LAYOUT_16X16X32, PROBE_LAYOUT_SMFMAC_32X32X32 = 0, 1, 2
PROBE_MFMA16 = 3          # added to a kind: the 16x16x32 instruction
PROBE_OPERAND_VECTORS = 1024
PROBE_SIGNATURES = {
    "gemm_f16_probe_mfma": ([_int, _int, _i64, _vp, _vp, _vp, ctypes.POINTER(ctypes.c_double)], _int),
    "gemm_f16_probe_mfma_layout": ([_int, _vp, _vp, _vp, _vp, _vp], _int),
}
_probe = None


def probe_lib() -> ctypes.CDLL:
    global _probe
    if _probe is None:
        _load_hip_runtime_first()
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build the HIP library first")
        h = ctypes.CDLL(PROBE_LIB_PATH)
        for name, (args, res) in PROBE_SIGNATURES.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _probe = h
    return _probe


def probe_mfma_tflops(mode: int, seconds: float = 0.3, seed: int = 0) -> float:
    """Sustained MFMA TFLOP/s of the GEMM's inner-loop instruction mix on
    register operands of the given kind (see include/gemm_f16_probe.h)."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    ops = (torch.randn(PROBE_OPERAND_VECTORS * 8, generator=g) * 0.5).to(torch.float16).cuda()
    blocks = 256 * 4
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    flops = ctypes.c_double()

    def launch(iters):
        st = probe_lib().gemm_f16_probe_mfma(mode, iters, blocks, ops.data_ptr(), out.data_ptr(),
                                             stream.cuda_stream, ctypes.byref(flops))
        if st != 0:
            raise RuntimeError(f"gemm_f16_probe_mfma failed ({st})")

    launch(200)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    iters = 2000
    s.record(stream)
    launch(iters)
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    iters = max(200, int(iters * seconds * 1e3 / max(ms, 1e-3)))   # resize to ~`seconds`
    s.record(stream)
    launch(iters)
    e.record(stream)
    torch.cuda.synchronize()
    return flops.value / (s.elapsed_time(e) * 1e-3) / 1e12

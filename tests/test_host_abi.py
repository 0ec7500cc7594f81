"""CPU tests of the C ABI: symbols, argument validation, planning.

No kernel is launched: validation and planning run before any HIP call, so
these run on a machine without a GPU.
"""
import ctypes
import os
import re

import pytest

import tiled_dense_gemm_fp16_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f16.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "smem_budget.txt")

# an address aligned to 256 bytes that is never dereferenced (validation only)
FAKE = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(g.LIB_PATH) or not os.path.exists(g.PROBE_LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_f16\w*)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"gemm_f16", "gemm_f16_ex", "gemm_f16_plan", "gemm_f16_status_string"} <= set(names)
    lib = ctypes.CDLL(g.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in gemm_f16.h but not exported"
    # and the binding describes exactly the declared functions
    assert set(g.SIGNATURES) == set(names)


def test_probe_library_exports_its_header():
    text = open(os.path.join(ROOT, "include", "gemm_f16_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(gemm_f16_probe\w*)\s*\(", text)))
    assert names == ["gemm_f16_probe_mfma", "gemm_f16_probe_mfma_layout"]
    lib = ctypes.CDLL(g.PROBE_LIB_PATH)
    for name in names:
        assert hasattr(lib, name)
    assert set(g.PROBE_SIGNATURES) == set(names)
    # argument checks happen before any launch
    assert g.probe_lib().gemm_f16_probe_mfma(7, 1, 1, None, FAKE, None, None) == 1
    assert g.probe_lib().gemm_f16_probe_mfma(0, 1, 0, None, FAKE, None, None) == 1
    assert g.probe_lib().gemm_f16_probe_mfma_layout(3, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert g.probe_lib().gemm_f16_probe_mfma_layout(2, FAKE, FAKE, None, FAKE, None) == 1


def test_status_strings():
    for st in range(0, 9):
        assert g.status_string(st) != "unknown status"
    assert g.status_string(99) == "unknown status"


def test_config_table():
    n = g.num_configs()
    assert n >= 2
    names = [g.config_name(c) for c in range(n)]
    assert all(names) and len(set(names)) == n
    assert g.config_name(n) is None and g.config_name(-1) is None
    for c in range(n):
        p = g.plan(4096, 4096, 4096, FAKE, FAKE, FAKE, config=c)
        assert p["config"] == c
        assert p["lds_bytes"] <= 163840                     # MI355X LDS per workgroup
        assert p["lds_bytes"] == g.stage_bytes(p["block_m"], p["block_n"], p["block_k"], p["stages"])
        assert p["threads"] in (256, 512)


def _golden_rows():
    rows, trips = [], []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "ktrip":
            trips.append(tuple(int(x) for x in f[1:4]))
        else:
            rows.append(tuple(int(x) for x in f[:5]))
    return rows, trips


def test_shared_memory_budget_matches_pages():
    rows, trips = _golden_rows()
    assert len(rows) == 6 and len(trips) == 1
    for bm, bn, bk, s, expected in rows:
        assert g.stage_bytes(bm, bn, bk, s) == expected
    assert g.stage_bytes(-1, 1, 1, 1) == -1
    # the pages' H100 remark: 228 KB holds two 96 KB blocks; MI355X's 160 KiB holds one
    assert 228 * 1024 // g.stage_bytes(128, 128, 64, 3) == 2
    assert 163840 // g.stage_bytes(128, 128, 64, 3) == 1
    for K, bk, iters in trips:
        # a configuration with the pages' block_K reports the same trip count
        cfgs = [c for c in range(g.num_configs()) if _plans(c, False)
                and g.plan(K, K, K, FAKE, FAKE, FAKE, config=c)["block_k"] == bk]
        assert cfgs
        for c in cfgs:
            assert g.plan(K, K, K, FAKE, FAKE, FAKE, config=c)["k_tiles"] == iters


def test_plan_geometry_and_vector_widths():
    p = g.plan(3000, 5000, 4100, FAKE, FAKE, FAKE)
    assert p["tiles_m"] == -(-3000 // p["block_m"]) and p["tiles_n"] == -(-5000 // p["block_n"])
    assert p["grid"] == p["tiles_m"] * p["tiles_n"]
    assert p["k_tiles"] == -(-4100 // p["block_k"])
    # K = 4100: A's rows only 8-byte aligned, so the direct configuration
    # for 4-byte rows runs (16-byte loads at 8-byte alignment)
    assert p["vec_a"] == 2 and p["vec_b"] == 2 and p["direct_lds"] == 1
    assert p["vec_c"] == 8                              # N = 5000: 16-byte stores of C
    assert p["flops"] == 2.0 * 3000 * 5000 * 4100
    assert p["min_bytes"] == 2.0 * (3000 * 4100 + 4100 * 5000 + 3000 * 5000)
    # odd pitches and 2-byte-aligned pointers
    p = g.plan(33, 17, 9, FAKE + 2, FAKE + 6, FAKE + 2)
    assert (p["vec_a"], p["vec_b"], p["vec_c"]) == (1, 1, 1)
    p = g.plan(64, 64, 64, FAKE + 4, FAKE + 8, FAKE)
    # a direct configuration reports the rows' alignment it needs (4 bytes),
    # a register-staged one its vector widths
    assert (p["vec_a"], p["vec_b"], p["vec_c"]) == ((2, 2, 8) if p["direct_lds"] else (2, 4, 8))
    p = g.plan(64, 60, 64, FAKE, FAKE, FAKE + 8)
    assert p["vec_c"] == 4
    # large aligned problems take a direct-to-LDS configuration
    assert g.plan(8192, 8192, 8192, FAKE, FAKE, FAKE)["direct_lds"] == 1
    # a direct configuration refuses a misaligned pitch
    direct = [c for c in range(g.num_configs())
              if _plans(c, False) and _plan_or_none(64, 128, 128, c) and _plan_or_none(64, 128, 128, c)["direct_lds"]]
    with pytest.raises(g.GemmError):
        g.plan(64, 128, 132, FAKE, FAKE, FAKE, config=direct[0])


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 4, FAKE, FAKE, FAKE * 2), 1),                   # negative dimension
    ((4, -1, 4, FAKE, FAKE, FAKE * 2), 1),
    ((4, 4, -1, FAKE, FAKE, FAKE * 2), 1),
    ((4, 4, 4, 0, FAKE, FAKE * 2), 1),                       # null A with elements
    ((4, 4, 4, FAKE, 0, FAKE * 2), 1),                       # null B
    ((4, 4, 4, FAKE, FAKE * 3, 0), 1),                       # null C
    ((4, 4, 4, FAKE + 1, FAKE * 3, FAKE * 2), 2),            # odd pointer
    ((4, 4, 4, FAKE, FAKE * 3 + 1, FAKE * 2), 2),
    ((4, 4, 4, FAKE, FAKE * 3, FAKE * 2 + 1), 2),
    ((4, 4, 4, FAKE, FAKE * 3, FAKE + 8), 1),                # C overlaps A
    ((4, 4, 4, FAKE, FAKE * 3, FAKE * 3 - 2), 1),            # C's last element overlaps B's first
    ((4, (1 << 22) + 1, 4, FAKE, FAKE * 3, FAKE * 2), 6),    # N beyond the limit
    ((4, 4, (1 << 22) + 1, FAKE, FAKE * 3, FAKE * 2), 6),    # K beyond the limit
    ((1 << 31, 4, 4, FAKE, FAKE * 3, FAKE * 2), 6),          # M beyond int32
])
def test_invalid_arguments_rejected_before_any_launch(args, status):
    M, N, K, A, B, C = args
    assert g.gemm_f16_raw(M, N, K, A, B, C, 0) == status
    assert g.gemm_f16_raw(M, N, K, A, B, C, 0, config=0) == status


def test_transposed_layout_planning():
    # vector widths follow the pitch of each matrix as stored
    p = g.plan(64, 48, 40, FAKE, FAKE, FAKE, trans_a=True)            # A stored 40 x 64: pitch M = 64
    assert (p["vec_a"], p["trans_a"], p["trans_b"]) == (8, 1, 0)
    p = g.plan(66, 48, 40, FAKE, FAKE, FAKE, trans_a=True)            # pitch 66: 4-byte rows
    assert p["vec_a"] == (2 if p["direct_lds"] else 1)
    p = g.plan(65, 48, 40, FAKE, FAKE, FAKE, trans_a=True)            # pitch 65: single elements
    assert p["vec_a"] == 1 and p["direct_lds"] == 0
    p = g.plan(64, 48, 36, FAKE, FAKE, FAKE, trans_b=True)            # B stored 48 x 36: pitch K = 36
    assert p["vec_b"] in (1, 2) and p["trans_b"] == 1
    p = g.plan(64, 48, 35, FAKE, FAKE, FAKE, trans_b=True)            # pitch 35: single elements
    assert p["vec_b"] == 1 and p["direct_lds"] == 0
    p = g.plan(8192, 8192, 8192, FAKE, FAKE, FAKE, trans_a=True, trans_b=True)
    assert p["direct_lds"] == 1
    # every configuration is compiled for the transposed layouts too
    ok = [c for c in range(g.num_configs()) if _plans(c, True)]
    assert len(ok) == g.num_configs()
    for c in range(g.num_configs()):
        assert _plans(c, False)
    # flags other than 0 / 1
    assert g.lib().gemm_f16_trans(4, 4, 4, FAKE, 2, FAKE * 3, 0, FAKE * 2, 0, -1, None) == 1
    assert g.lib().gemm_f16_trans(4, 4, 4, FAKE, 0, FAKE * 3, -1, FAKE * 2, 0, -1, None) == 1
    assert g.gemm_f16_raw(0, 4, 4, 0, FAKE, 0, 0, trans_a=True) == 0


def _plan_or_none(M, N, K, c, **kw):
    try:
        return g.plan(M, N, K, FAKE, FAKE, FAKE, config=c, **kw)
    except g.GemmError:
        return None


def _plans(c, trans):
    try:
        g.plan(4096, 4096, 4096, FAKE, FAKE, FAKE, config=c, trans_b=trans)
        return True
    except g.GemmError:
        return False


def test_bad_epilogue_and_config():
    assert g.gemm_f16_raw(4, 4, 4, FAKE, FAKE * 3, FAKE * 2, 2) == 1
    assert g.gemm_f16_raw(4, 4, 4, FAKE, FAKE * 3, FAKE * 2, -1) == 1
    assert g.gemm_f16_raw(4, 4, 4, FAKE, FAKE * 3, FAKE * 2, 0, config=g.num_configs()) == 1
    assert g.gemm_f16_raw(4, 4, 4, FAKE, FAKE * 3, FAKE * 2, 0, config=-2) == 1
    with pytest.raises(g.GemmError):
        g.plan(4, 4, 4, FAKE, FAKE, FAKE, config=99)


def test_empty_outputs_succeed_without_a_device():
    # M == 0 or N == 0: nothing to do, no HIP call, so this works on a CPU host too
    assert g.gemm_f16_raw(0, 5, 7, 0, FAKE, 0, 0) == 0
    assert g.gemm_f16_raw(5, 0, 7, FAKE, 0, 0, 1) == 0
    assert g.gemm_f16_raw(0, 0, 0, 0, 0, 0, 0) == 0


def test_python_wrapper_argument_checks():
    import torch

    a = torch.zeros(4, 4, dtype=torch.float16)
    with pytest.raises(ValueError):
        g.gemm(a, a, epilogue="gelu")
    with pytest.raises(ValueError):
        g.gemm(a, a)                                           # CPU tensors
    for kw in ({}, {"epilogue": "gelu"}, {"trans_b": True}):
        with pytest.raises(ValueError):                        # prepare() checks the same, once
            g.prepare(a, a, **kw)
    with pytest.raises(ValueError):
        g.gemm(a.float(), a)


U_NAMES = {"256x256x64_s2_direct_m16_u", "256x128x64_s3_direct_m16_u", "128x128x64_s4_direct_m16_u",
           "128x64x64_s4_direct_u", "64x64x64_s4_direct_u"}


def test_rows_4byte_aligned_take_direct_configs():
    """Operands whose rows (or pointers) are only 4-byte aligned run the
    direct configurations for such rows (16-byte loads at 4-byte alignment)
    in every layout; rows only 2-byte aligned (an odd pitch or pointer) run
    register-staged ones."""
    index = {g.config_name(c): c for c in range(g.num_configs())}
    assert U_NAMES <= set(index)
    for ta in (False, True):
        for tb in (False, True):
            kw = {"trans_a": ta, "trans_b": tb}
            p = g.plan(8192, 8192, 8192, FAKE + 4, FAKE, FAKE, **kw)        # A's pointer 4-byte aligned
            assert g.config_name(p["config"]) in U_NAMES and (p["vec_a"], p["vec_b"], p["direct_lds"]) == (2, 2, 1), kw
            p = g.plan(8196, 8196, 8196, FAKE, FAKE, FAKE, **kw)            # every pitch 8-byte aligned
            assert g.config_name(p["config"]) in U_NAMES, kw
    p = g.plan(8192, 8192, 8193, FAKE, FAKE, FAKE)                        # odd K: 2-byte rows
    assert p["direct_lds"] == 0 and p["vec_a"] == 1
    p = g.plan(8192, 8192, 8192, FAKE + 2, FAKE, FAKE)                    # A's pointer 2-byte aligned
    assert p["direct_lds"] == 0
    for name in U_NAMES:
        g.plan(8192, 8196, 8194, FAKE, FAKE, FAKE, config=index[name])
        for kw in ({"trans_b": True}, {"trans_a": True}):
            g.plan(8194, 8196, 8198, FAKE, FAKE, FAKE, config=index[name], **kw)
        with pytest.raises(g.GemmError):
            g.plan(8192, 8192, 8193, FAKE, FAKE, FAKE, config=index[name])
        with pytest.raises(g.GemmError):
            g.plan(8192, 8192, 8192, FAKE, FAKE + 2, FAKE, config=index[name])


TUNED = os.path.join(ROOT, "tiled_dense_gemm_fp16_amd", "csrc", "gemm_f16_tuned.inc")


def tuned_entries():
    rows = []
    for line in open(TUNED):
        m = re.match(r"\{\s*(-?\d+(?:\s*,\s*-?\d+){7})\s*,\s*([\d.]+)\s*,\s*(-?\d+)\s*,\s*([\d.]+)\s*\},",
                     line)
        if m:
            rows.append(tuple(int(x) for x in m.group(1).split(",")) + (int(m.group(3)),))
    return rows


def test_tuned_table_drives_the_automatic_choice():
    """Every entry of the measured table names configurations that accept
    its shape; for exactly that shape the planner picks the entry's unsplit
    configuration for the workspace-free entry points and its configuration
    and split count for gemm_f16_split with SPLITS_AUTO."""
    rows = tuned_entries()
    assert rows, "the measured configuration table is empty"
    seen = set()
    for lm, ln, lk, ta, tb, aligned, cfg, splits, cfg1 in rows:
        assert 0 <= cfg < g.num_configs() and 0 <= cfg1 < g.num_configs() and 1 <= splits <= g.MAX_SPLITS
        assert splits > 1 or cfg == cfg1
        key = (lm, ln, lk, ta, tb, aligned)
        assert key not in seen
        seen.add(key)
        # class 1: aligned pitches; 2: every pitch off by 4 elements; 0: every pitch odd
        pm, pn, pk = {1: (0, 0, 0), 2: (4, 4, 4), 0: (1, 1, 1)}[aligned]
        M, N, K = (1 << lm) + pm, (1 << ln) + pn, (1 << lk) + pk
        kw = dict(trans_a=bool(ta), trans_b=bool(tb))
        p = g.plan(M, N, K, FAKE, FAKE, FAKE, **kw)
        assert p["config"] == cfg1 and p["splits"] == 1 and p["workspace_bytes"] == 0, (key, p["config"])
        q = g.plan(M, N, K, FAKE, FAKE, FAKE, splits=g.SPLITS_AUTO, **kw)
        assert q["config"] == cfg, (key, q["config"])
        want = g.plan(M, N, K, FAKE, FAKE, FAKE, config=cfg, splits=splits, **kw)
        assert q["splits"] == want["splits"] and q["k_split"] == want["k_split"], key
        assert (p["vec_a"] == 8 and p["vec_b"] == 8) == (aligned == 1)
        assert aligned != 0 or min(p["vec_a"], p["vec_b"]) == 1
    # far from every swept shape the analytic model decides (no table hit):
    # a deep K under a one-tile output is split when a workspace may be used
    p = g.plan(24, 24, 1 << 20, FAKE, FAKE, FAKE, splits=g.SPLITS_AUTO)
    assert p["splits"] > 1 and p["workspace_bytes"] == p["splits"] * 24 * 24 * 4


def test_workspace_free_entry_points_never_split():
    """gemm_f16, gemm_f16_ex and gemm_f16_trans take no workspace: their
    plans run one kernel over all of K even where gemm_f16_split would
    split (table hits and model choices alike)."""
    for M, N, K in [(1024, 1024, 8192), (512, 512, 8192), (96, 96, 30000), (24, 24, 1 << 20), (512, 512, 4096)]:
        for ta, tb in [(False, False), (False, True), (True, False), (True, True)]:
            auto = g.plan(M, N, K, FAKE, FAKE, FAKE, trans_a=ta, trans_b=tb)
            assert auto["splits"] == 1 and auto["workspace_bytes"] == 0 and auto["k_split"] == K
            assert auto["grid"] == auto["tiles_m"] * auto["tiles_n"]
        split = g.plan(M, N, K, FAKE, FAKE, FAKE, splits=g.SPLITS_AUTO)
        assert split["splits"] > 1 and split["workspace_bytes"] == split["splits"] * M * N * 4, (M, N, K)
        for c in range(g.num_configs()):
            try:
                p = g.plan(M, N, K, FAKE, FAKE, FAKE, config=c)
            except g.GemmError:
                continue
            assert p["splits"] == 1 and p["workspace_bytes"] == 0


def test_split_without_a_workspace_is_refused_before_any_launch():
    # 1024 x 1024 x 8192: the planner splits it; no workspace means status 7,
    # returned by validation (so also on a host without a GPU)
    st = g.lib().gemm_f16_split(1024, 1024, 8192, FAKE, 0, FAKE * 64, 0, FAKE * 128, 0, g.CONFIG_AUTO,
                                g.SPLITS_AUTO, None, 0, None)
    assert st == 7
    st = g.lib().gemm_f16_split(1024, 1024, 8192, FAKE, 0, FAKE * 64, 0, FAKE * 128, 0, 2, 4, None, 0, None)
    assert st == 7


def test_static_scratch_entry_point_limit_before_any_launch():
    """gemm_f16_split_static refuses, before any HIP call, a split whose
    partial sums exceed its static scratch (status 9); argument errors come
    first, as for gemm_f16_split."""
    call = g.lib().gemm_f16_split_static
    # 4096 x 4096 split 2: 128 MiB of partial sums > 32 MiB
    assert call(4096, 4096, 8192, FAKE, 0, FAKE * 128, 0, FAKE * 256, 0, 2, 2, None) == 9
    assert g.STATIC_WORKSPACE_BYTES == 32 << 20
    assert call(4096, 4096, 8192, FAKE, 2, FAKE * 128, 0, FAKE * 256, 0, 2, 2, None) == 1      # bad flag
    assert call(-1, 4, 4, FAKE, 0, FAKE * 3, 0, FAKE * 2, 0, -1, 0, None) == 1                  # negative M
    assert call(4, 4, 4, FAKE, 0, FAKE * 3, 0, FAKE * 2, 0, -1, g.MAX_SPLITS + 1, None) == 1    # split count
    assert call(0, 4, 4, 0, 0, FAKE * 3, 0, 0, 0, -1, 0, None) == 0                            # empty output


def test_library_imports_no_allocation_or_synchronisation():
    """The shared library does not even import the HIP calls that allocate
    or free device or host memory, or that wait for a stream or the device:
    no call path can reach them."""
    import shutil
    import subprocess

    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    out = subprocess.run([nm, "-D", "--undefined-only", g.LIB_PATH], capture_output=True, text=True, check=True)
    imported = {line.split()[-1].split("@")[0] for line in out.stdout.splitlines() if line.strip()}
    hip = {name for name in imported if name.startswith("hip")}
    assert "hipGetDevice" in hip                      # the import list was read
    forbidden = re.compile(r"^hip(Ext)?(Malloc|Free|HostAlloc|HostMalloc|HostFree|MemAlloc|MemPool|"
                           r"StreamSynchronize|DeviceSynchronize|EventSynchronize|Memcpy$|Memset$|"
                           r"MemcpyHtoD$|MemcpyDtoH$|MemcpyDtoD$)")
    assert not sorted(n for n in hip if forbidden.match(n)), hip


def test_transposed_a_size_limit():
    """A stored K x M: a 64-row k slice of pitch M must fit a 2 GiB buffer
    range, so M is at most 2^24 there (status 6 beyond, before any launch)."""
    for M in (1 << 25, (1 << 24) + 1, 1 << 26):
        with pytest.raises(g.GemmError) as e:
            g.plan(M, 64, 64, FAKE, FAKE, FAKE, trans_a=True)
        assert e.value.status == 6
        assert g.gemm_f16_raw(M, 64, 64, FAKE, FAKE * 3, FAKE * 2, 0, trans_a=True) == 6
        assert g.lib().gemm_f16_split(M, 64, 64, FAKE, 1, FAKE * 3, 0, FAKE * 2, 0, -1, 2, None, 0, None) == 6
    p = g.plan(1 << 24, 64, 64, FAKE, FAKE, FAKE, trans_a=True)
    assert p["tiles_m"] == (1 << 24) // p["block_m"]
    # the same M with A stored M x K is fine
    g.plan(1 << 25, 64, 64, FAKE, FAKE, FAKE)


# ---- split-K planning and workspace validation (host logic only) ----

def test_split_geometry():
    # 128x128x64 tiles, K = 1000: 16 k tiles
    base = dict(config=2, splits=1)
    p = g.plan(256, 256, 1000, FAKE, FAKE, FAKE, **base)
    assert (p["splits"], p["k_split"], p["workspace_bytes"], p["grid"]) == (1, 1000, 0, 4)
    for req, splits, k_split in [(2, 2, 512), (3, 3, 384), (5, 4, 256), (16, 16, 64), (64, 16, 64)]:
        p = g.plan(256, 256, 1000, FAKE, FAKE, FAKE, config=2, splits=req)
        assert (p["splits"], p["k_split"]) == (splits, k_split), req
        assert p["grid"] == 4 * splits and p["k_tiles"] == k_split // 64
        assert p["workspace_bytes"] == splits * 256 * 256 * 4
        # no split is empty and the splits cover K exactly
        assert (splits - 1) * k_split < 1000 <= splits * k_split
    # one k tile (or none) cannot be split
    assert g.plan(256, 256, 64, FAKE, FAKE, FAKE, config=2, splits=4)["splits"] == 1
    assert g.plan(256, 256, 0, FAKE, FAKE, FAKE, config=2, splits=4)["splits"] == 1
    # the explicit-config entry points never split
    assert g.plan(64, 64, 1 << 20, FAKE, FAKE, FAKE, config=4)["splits"] == 1
    # split counts outside [0, 64] are rejected
    for bad in (-1, g.MAX_SPLITS + 1):
        with pytest.raises(g.GemmError):
            g.plan(256, 256, 1000, FAKE, FAKE, FAKE, config=2, splits=bad)
    # a workgroup's workspace slice must stay addressable: 256 rows x N fp32 < 2 GiB
    with pytest.raises(g.GemmError) as e:
        g.plan(256, 1 << 21, 1024, FAKE, FAKE, FAKE, config=0, splits=2)
    assert e.value.status == 6
    assert g.plan(64, 1 << 21, 1024, FAKE, FAKE, FAKE, config=4, splits=2)["splits"] == 2


def _split_call(ws, ws_bytes, C=FAKE * 2, splits=4):
    return g.lib().gemm_f16_split(256, 256, 1000, FAKE, 0, FAKE * 3, 0, C, 0, 2, splits, ws, ws_bytes, None)


def test_split_workspace_validation_before_any_launch():
    need = 4 * 256 * 256 * 4
    WS = FAKE * 8
    assert _split_call(WS, need - 1) == 7                     # too small
    assert _split_call(WS + 8, need) == 2                     # not 16-byte aligned
    assert _split_call(FAKE * 2 - 16, need) == 1              # overlaps C
    assert _split_call(FAKE, need) == 1                       # overlaps A
    assert _split_call(None, 16) == 1                         # size without a buffer
    assert _split_call(WS, -1) == 1                           # negative size
    assert _split_call(WS, need, splits=65) == 1              # split count beyond the maximum
    # (valid arguments are not tried here: on a GPU host they would launch
    # on these stand-in addresses)


def test_sparse_argument_checks_before_any_launch():
    sp = g.lib().gemm_f16_sp
    V, Mt, B, C = FAKE, FAKE * 4, FAKE * 8, FAKE * 12
    assert sp(64, 64, 40, V, Mt, B, 0, C, 0, -1, None) == 1            # K % 16 != 0
    assert sp(64, 64, 48, V + 8, Mt, B, 0, C, 0, -1, None) == 2        # vals not 16-byte aligned
    assert sp(64, 60, 48, V, Mt, B, 0, C, 0, -1, None) == 2            # N % 8 != 0
    assert sp(64, 64, 48, V, Mt + 1, B, 0, C, 0, -1, None) == 2        # odd meta pointer
    assert sp(64, 64, 48, V, 0, B, 0, C, 0, -1, None) == 1             # no meta
    assert sp(64, 64, 48, V, Mt, B, 0, V, 0, -1, None) == 1            # C overlaps vals
    assert sp(64, 64, 48, V, Mt, B, 0, C, 2, -1, None) == 1            # unknown epilogue
    assert sp(64, 64, 48, V, Mt, B, 0, C, 0, g.sp_num_configs(), None) == 1
    assert sp(0, 64, 48, V, Mt, B, 0, C, 0, -1, None) == 0             # empty: no launch
    assert sp(64, 64, 48, V, Mt, B, 2, C, 0, -1, None) == 1            # trans_b not 0 / 1
    assert sp(0, 60, 48, V, Mt, B, 1, C, 0, -1, None) == 0             # B as N x K: N % 8 not needed
    assert sp(64, 60, 48, V, Mt, B + 8, 1, C, 0, -1, None) == 2        # ... but 16-byte B
    assert g.lib().gemm_f16_sp_compress(4, 24, FAKE, V, Mt, None) == 1
    assert g.lib().gemm_f16_sp_compress(4, 32, FAKE + 1, V, Mt, None) == 2
    assert g.lib().gemm_f16_sp_compress(0, 32, 0, 0, 0, None) == 0
    names = [g.sp_config_name(c) for c in range(g.sp_num_configs())]
    assert all(names) and len(set(names)) == len(names) and g.sp_config_name(-1) is None
    p = g.plan_sp(4096, 4096, 4096, FAKE, FAKE, FAKE, FAKE)
    assert p["flops"] == 4096.0 ** 3 and p["lds_bytes"] <= 163840
    for c in range(g.sp_num_configs()):
        q = g.plan_sp(300, 264, 1008, FAKE, FAKE, FAKE, FAKE, config=c)
        assert q["config"] == c and q["grid"] == q["tiles_m"] * q["tiles_n"]


def test_persistent_config_takes_no_split():
    """The persistent tile loop has no split form: an explicit count above 1
    is refused, SPLITS_AUTO and 1 plan one kernel of at most 256 workgroups."""
    c = [i for i in range(g.num_configs()) if g.config_name(i).endswith("_persistent")]
    assert len(c) == 1
    for sp in (None, 1):
        p = g.plan(4096, 4096, 4096, FAKE, FAKE, FAKE, config=c[0], **({} if sp is None else {"splits": sp}))
        assert p["splits"] == 1 and p["workspace_bytes"] == 0 and p["grid"] == 256
    with pytest.raises(g.GemmError):
        g.plan(4096, 4096, 4096, FAKE, FAKE, FAKE, config=c[0], splits=2)


def test_library_binds_to_torchs_hip_runtime():
    """Loaded through the binding, even before torch is imported, the library
    uses the HIP runtime torch loaded: the process maps one libamdhip64."""
    import subprocess
    import sys
    code = ("import tiled_dense_gemm_fp16_amd as g; g.lib(); g.probe_lib(); import torch; "
            "maps = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_sparse_position_word_order():
    """The documented storage order of the position words is a permutation
    of the M K/16 words that keeps each 64-deep slice's words of
    consecutive rows contiguous."""
    import numpy as np
    from sp_layout import meta_flat, meta_index, meta_rows
    for M, K in [(1, 16), (5, 64), (7, 80), (33, 1008), (64, 4096), (3, 48)]:
        idx = meta_index(M, K)
        assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(M * K // 16))
        for s in range(K // 64):
            block = idx[:, 4 * s:4 * s + 4].reshape(-1)
            assert np.array_equal(block, np.arange(block[0], block[0] + 4 * M))
        rows = np.arange(M * K // 16, dtype=np.uint16).reshape(M, K // 16)
        assert np.array_equal(meta_rows(meta_flat(rows), M, K), rows)

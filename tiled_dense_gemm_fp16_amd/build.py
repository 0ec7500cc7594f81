"""Compile the gfx950 GEMM library (libgemm_f16.so) in-tree with hipcc.

Each source file is compiled to an object of its own (in parallel; the tile
kernel is instantiated per layout in separate files), then the objects are
linked into the shared library.
"""
import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgemm_f16.so")
SOURCES = [os.path.join(CSRC, f) for f in (
    "gemm_f16_api.cpp", "gemm_f16_kernels.hip", "gemm_f16_nn.hip", "gemm_f16_nt.hip", "gemm_f16_tn.hip",
    "gemm_f16_tt.hip", "gemm_f16_sparse.hip")]
# what each kind of source includes (for incremental builds)
HOST_DEPS = [os.path.join(CSRC, f) for f in ("gemm_f16_internal.h", "gemm_f16_tuned.inc")] + \
    [os.path.join(INCLUDE, "gemm_f16.h")]
KERNEL_DEPS = [os.path.join(CSRC, f) for f in ("gemm_f16_internal.h", "gemm_f16_tile.h")]
PROBE_LIB = os.path.join(PKG, "libgemm_f16_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "mfma_probe.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra_flags=None, jobs: int | None = None, incremental: bool = False) -> str:
    """Compile libgemm_f16.so and the measurement probe libgemm_f16_probe.so next
    to this file; return the GEMM library's path.  ``incremental`` reuses an
    object newer than its source and every shared header (same flags
    assumed); by default everything is compiled."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES) + len(PROBE_SOURCES), max(1, (os.cpu_count() or 4) - 1), 8)
    units = [(src, LIB) for src in SOURCES] + [(src, PROBE_LIB) for src in PROBE_SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(lambda u: _compile(u[0], verbose, extra_flags, incremental), units))
    _link([o for o, (_, lib) in zip(objs, units) if lib == LIB], LIB, verbose)
    _link([o for o, (_, lib) in zip(objs, units) if lib == PROBE_LIB], PROBE_LIB, verbose)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 feature flag; that warning is harmless
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            print("\n".join(lines), flush=True)


def _compile(src, verbose, extra_flags, incremental=False):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        deps = HOST_DEPS if src.endswith(".cpp") else KERNEL_DEPS
        newest = max(os.path.getmtime(p) for p in [src, *deps])
        if os.path.getmtime(obj) > newest:
            return obj
    _run([HIPCC, *FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-x", "hip", "-c", src, "-o", obj],
         verbose)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))

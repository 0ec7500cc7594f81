"""Compile the gfx950 GEMM library (libgemm_f16.so) in-tree with hipcc."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemm_f16.so")
SOURCES = [os.path.join(CSRC, "gemm_f16_api.cpp"), os.path.join(CSRC, "gemm_f16_kernels.hip")]
PROBE_LIB = os.path.join(PKG, "libgemm_f16_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "mfma_probe.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile libgemm_f16.so and the measurement probe libgemm_f16_probe.so next
    to this file; return the GEMM library's path."""
    _compile(SOURCES, LIB, verbose, extra_flags)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose, extra_flags)
    return LIB


def _compile(sources, lib, verbose, extra_flags):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-x", "hip", *sources,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 feature flag; that warning is harmless
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            print("\n".join(lines), flush=True)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))

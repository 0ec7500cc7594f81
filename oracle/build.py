"""Build the CPU oracle library (plain C, gcc) next to its source.

Test infrastructure: the oracle is the checker, not the product.  Building
it here does not route any product call through it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_gemm.c")
SRCS = [SRC, os.path.join(HERE, "oracle_sparse.c")]
LIB = os.path.join(HERE, "liboracle_gemm.so")


def build(verbose: bool = False) -> str:
    """Compile oracle_gemm.c and oracle_sparse.c into liboracle_gemm.so and return its path.

    -O2 without -ffast-math keeps IEEE semantics: every element's sum stays
    sequential in k.  -ffp-contract=off is stated for clarity only (products
    of binary16 values are exact in binary64, so contraction cannot change a
    result).
    """
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, *SRCS, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

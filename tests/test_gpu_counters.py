"""The counter the roofline figures lean on, checked against the product's
own arithmetic: rocprofv3's SQ_INSTS_VALU_MFMA_MOPS_F16 counts FP16 matrix
operations in units of 512 flops, so over one GEMM launch on whole tiles it
must read exactly 2 M N K / 512 -- no padded or repeated work, and no
instruction the counter misses.  Runs the profiler on a child process; skipped
where rocprofv3 is not installed."""
import csv
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import tiled_dense_gemm_fp16_amd as g

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPE = (1024, 1536, 2048)   # whole 256 x 256 x 64 tiles, 24 workgroups

CHILD = """
import torch, tiled_dense_gemm_fp16_amd as g
M, N, K = {shape}
a = torch.randn(M, K, device="cuda:0").half()
b = torch.randn(K, N, device="cuda:0").half()
for name in {names}:
    c = next(i for i in range(g.num_configs()) if g.config_name(i) == name)
    g.gemm(a, b, config=c, splits=1)
    torch.cuda.synchronize()
    print("ran", name, flush=True)
"""

NAMES = ["256x128x64_s3_direct_m16", "256x256x64_s2_direct_m16", "256x256x64_s2_direct_m16_persistent"]


def test_mfma_op_counter_matches_2mnk():
    prof = shutil.which("rocprofv3")
    if prof is None:
        pytest.skip("rocprofv3 not installed")
    names = [n for n in NAMES if n in [g.config_name(i) for i in range(g.num_configs())]]
    assert names
    with tempfile.TemporaryDirectory(dir="/tmp") as out:
        env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
        cmd = [prof, "--pmc", "SQ_INSTS_VALU_MFMA_MOPS_F16", "--output-format", "csv", "-d", out, "-o", "run",
               "--", sys.executable, "-c", CHILD.format(shape=SHAPE, names=names)]
        print("running", " ".join(cmd[:8]), flush=True)
        r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=90)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
        paths = glob.glob(os.path.join(out, "**", "*counter_collection.csv"), recursive=True)
        assert paths, r.stdout[-2000:]
        rows = []
        for p in paths:
            with open(p, newline="") as f:
                rows += [row for row in csv.DictReader(f) if "gemm_f16" in row["Kernel_Name"]]
    rows.sort(key=lambda row: int(row["Dispatch_Id"]))
    assert len(rows) == len(names), [row["Kernel_Name"][:60] for row in rows]
    M, N, K = SHAPE
    for name, row in zip(names, rows):
        assert float(row["Counter_Value"]) * 512 == 2 * M * N * K, (name, row["Counter_Value"])

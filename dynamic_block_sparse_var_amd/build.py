"""Build libprism.so (HIP, gfx950) in-tree.

    python -m dynamic_block_sparse_var_amd.build [--jobs N]

Every source under csrc/ is compiled by hipcc for gfx950 into an object, in parallel, and
the objects are linked into dynamic_block_sparse_var_amd/libprism.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libprism.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "stats.hip", "permute_pool.hip", "select.hip", "attn.hip", "attn_mfma.hip"]

COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-munsafe-fp-atomics",
    # no packed-fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, extra: list[str], bdir: str = BUILD) -> str:
    obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)
    return obj


def build(jobs: int | None = None, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile every source into `out` (default: the package's libprism.so); objects of a build
    with extra flags go to a build folder of their own."""
    extra = list(extra or [])
    out = out or LIB
    bdir = BUILD if not extra or extra == ["-Rpass-analysis=kernel-resource-usage"] else BUILD + "_" + "_".join(
        f.strip("-").replace("=", "_") for f in extra)
    os.makedirs(bdir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, bdir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--resource-usage", action="store_true", help="print per-kernel register/LDS usage")
    ap.add_argument("--debug", action="store_true",
                    help="bounds-checked build: the kernels assert that every row, tile and list entry they touch "
                         "lies inside its tensor (PRISM_DEBUG)")
    ap.add_argument("--out", default=None, help="library path (default: the package's libprism.so)")
    a = ap.parse_args()
    ex = ["-Rpass-analysis=kernel-resource-usage"] if a.resource_usage else []
    if a.debug:
        ex.append("-DPRISM_DEBUG")
    print(build(a.jobs, ex, out=a.out))

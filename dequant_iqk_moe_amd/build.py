"""Build the HIP C-ABI library ``libiqk.so`` in-tree for gfx950.

Every ``.hip`` file is compiled for ``--offload-arch=gfx950`` with packed-FP32
instructions disabled; the dequantization kernels additionally forbid FMA
contraction so each float32 step of the reconstruction rounds on its own.
Run ``python dequant_iqk_moe_amd/build.py`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libiqk.so")
ARCH = os.environ.get("IQK_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PER_FILE = {
    "iqk_dequant.hip": ["-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero"],
    "iqk_gemv.hip": [],
    "iqk_prefill.hip": [],
    "iqk_fused.hip": [],
    "iqk_glue.hip": [],
    "iqk_noalloc.hip": [],
    "iqk_host.cpp": [],
    "iqk_relayout.cpp": [],
    "iqk_status.cpp": [],
}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> None:
    flags = COMMON + PER_FILE[src]
    if src.endswith(".hip"):
        flags = flags + DEVICE
    cmd = [_hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(PER_FILE)
    objs = [os.path.join(objdir, s + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        list(ex.map(_compile, srcs, objs))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)

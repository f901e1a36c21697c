"""Builds librattn.so (HIP for gfx950) in-tree with hipcc.

    python -m shared_base_residual_amd.build

Every HIP source is compiled with packed-fp32 instruction selection disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns
that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librattn.so")
SOURCES = ["api.cpp", "decode.hip", "prefill.hip", "gather.hip", "cache_write.hip", "pagepool.cpp", "quant.hip", "recon.hip",
           "values3.hip"]
# the benchmark's HBM read-bandwidth probe: a library of its own, not librattn
PROBE_LIB = os.path.join(HERE, "libhbm_probe.so")
PROBE_SOURCES = ["hbm_probe.hip"]
ARCH = "gfx950"


def source_hash() -> str:
    """Hash of every library source (kernels, host planner, public header): a
    measurement taken on other sources no longer describes the built kernels."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(set(os.listdir(CSRC)) - set(PROBE_SOURCES)) + ["../../include/rattn.h"]:
        path = os.path.normpath(os.path.join(CSRC, name))
        if os.path.isfile(path):
            with open(path, "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    # -amdgpu-mfma-vgpr-form: MFMA accumulators live in ordinary VGPRs (the
    # kernels fit in 256), so the online-softmax rescale and the epilogue need no
    # AGPR <-> VGPR copies.
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        cmd = [cc, *flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose:
            errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
            if errs:
                print("\n".join(errs), file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    n = len(SOURCES)
    for lib, lib_objs in ((LIB, objs[:n]), (PROBE_LIB, objs[n:])):
        tmp = lib + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *lib_objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libdsv.so (C ABI + gfx950 HIP kernels) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsv.so")
SOURCES = ["dsv_api.cpp", "dsv_plan.cpp", "topk.hip", "attn_fwd.hip", "attn_bwd.hip"]
ARCH = os.environ.get("DSV_OFFLOAD_ARCH", "gfx950")
# The forward keeps its output accumulators in VGPRs (MFMA results written to VGPRs, not
# AGPRs): its lazy rescale multiplies them with VALU ops, and with AGPR accumulators the
# compiler copies all of them to VGPRs on every chunk, rescaled or not.
# The backward's staging format is chosen per chunk by a branch that is the same in every
# lane; left unstructurized (a plain if/else), the compiler's waits for the prefetched K/V
# rows at the top of its loop leave the previous chunk's stores in flight. With MFMA results
# in VGPRs it also fits in 512 registers without spilling.
EXTRA_FLAGS = {"attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form",
                                "-mllvm", "-structurizecfg-skip-uniform-regions=true"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def common_flags():
    return ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
            # keep the compiler from emitting packed fp32 VALU ops
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source for gfx950 and link libdsv.so; returns the library path."""
    cc = hipcc()
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
               "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libdflash.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m block_diffusion_drafter_injection_amd.build [--jobs N]
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdflash.so")
SOURCES = ["api.cpp", "gemm.hip", "attention.hip", "elementwise.hip", "verify.hip"]
ARCH = os.environ.get("DFLASH_ARCH", "gfx950")
# per-source flags: the attention kernels keep their MFMA accumulators in
# ordinary VGPRs (the default form parks them in AGPRs and copies them back
# and forth around the softmax rescale)
FILE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def compile_flags():
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
            # packed fp32 instructions stay off in every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result"]


DEBUG_LIB = os.path.join(PKG, "libdflash_debug.so")


def build(jobs=5, verbose=False, defines=(), out=None, objdir=None, debug_variant=True):
    """Compile every source and link libdflash.so; with debug_variant also link
    libdflash_debug.so, whose host layer (api.cpp built with DFLASH_DEBUG)
    checks device-resident indices before launching the same kernels."""
    cc = hipcc()
    objdir = objdir or os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def one(job):
        src, extra, stem = job
        obj = os.path.join(objdir, stem + ".o")
        cmd = [cc, *compile_flags(), *FILE_FLAGS.get(src, []), *[f"-D{d}" for d in defines], *extra, "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
        if verbose and r.stderr.strip():
            err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
            if err.strip():
                print(err)
        return obj

    jobs_list = [(src, [], os.path.splitext(src)[0]) for src in SOURCES]
    if debug_variant:
        jobs_list.append(("api.cpp", ["-DDFLASH_DEBUG"], "api_debug"))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, jobs_list))

    def link(lib, parts):
        tmp = lib + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
        os.replace(tmp, lib)

    lib = out or LIB
    kernels = objs[1:len(SOURCES)]
    link(lib, [objs[0], *kernels])
    if debug_variant:
        link(DEBUG_LIB, [objs[-1], *kernels])
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=5)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.v))

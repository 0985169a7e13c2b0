"""Build libkvpub.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc,
and libkvpub_floor.so (the plain-stream floor kernel the benchmark times beside it)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvpub.so")
SOURCES = ["kvpub_api.hip", "store_kernel.hip", "fence_kernel.hip", "gather_kernel.hip", "vmm.hip"]
FLOOR_LIB = os.path.join(PKG, "libkvpub_floor.so")
FLOOR_SOURCES = ["floor_kernel.hip"]
ARCH = "gfx950"

# No fast-math, no FP contraction (explicit fmaf only); packed-fp32 instructions
# off for every HIP file.
# Kernel arguments that are plain scalars are preloaded into SGPRs at wave
# launch (the first 14 dwords: the store kernel's row pointers and strides).
HIPFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-DKVPUB_BUILD_SHARED", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=14",
            "-Wall", "-I", INCLUDE, "-I", CSRC]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; install ROCm or put it on PATH")
    return exe


def build_library(out=LIB, extra_flags=(), sources=None):
    """Compile every HIP source and link the shared library.  Always rebuilds."""
    sources = SOURCES if sources is None else sources
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIPFLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(sources)) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = out + ".tmp"
    r = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build_floor_library(out=FLOOR_LIB):
    """The measurement-only floor kernel library.  Always rebuilds."""
    return build_library(out, sources=FLOOR_SOURCES)


def build_all():
    return build_library(), build_floor_library()


if __name__ == "__main__":
    print(build_all())

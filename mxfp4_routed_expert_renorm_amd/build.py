"""Build libmoe_mi355x.so for gfx950 in-tree with hipcc (no GPU needed).

Every HIP source is compiled with packed-FP32 instruction generation turned
off; objects go to _build/ beside the package, the shared library next to
this file, where the binding loads it."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def _compile(src: str, obj: str) -> tuple[str, str]:
    cmd = [hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    return src, p.stderr


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, err in ex.map(_compile, srcs, objs):
            if verbose:
                print(f"compiled {os.path.basename(src)}", file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-side sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for the
# library's host code: the .cpp sources (entry points, slot-cache policy and
# bookkeeping, profiling, tensor-parallel slicing) are compiled with the
# sanitizers on their host pass only; the kernels' objects are the regular
# build's.  The result loads into a Python process that preloads the ASan
# runtime (asan_runtime()).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "san", "libmoe_mi355x_san.so")


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload)."""
    p = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    if p.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not cands:
            raise RuntimeError("the compiler's shared ASan runtime was not found")
        path = cands[-1]
    return path


def build_host_sanitized(jobs: int | None = None) -> str:
    """libmoe_mi355x_san.so: host code instrumented, kernels as in build()."""
    hip_srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    hip_objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in hip_srcs]
    if not all(os.path.exists(o) and os.path.getmtime(o) >= os.path.getmtime(s) for s, o in zip(hip_srcs, hip_objs)):
        build(jobs=jobs)
    sdir = os.path.dirname(SAN_LIB)
    os.makedirs(sdir, exist_ok=True)
    cpp_srcs = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    cpp_objs = [os.path.join(sdir, os.path.basename(s) + ".o") for s in cpp_srcs]

    def comp(src, obj):
        cmd = [hipcc(), *HIP_FLAGS, "-O1", *SAN_FLAGS, "-c", src, "-o", obj]
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")

    with cf.ThreadPoolExecutor(jobs or min(len(cpp_srcs), 8)) as ex:
        list(ex.map(comp, cpp_srcs, cpp_objs))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libsan", "-o", tmp,
           *cpp_objs, *hip_objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))

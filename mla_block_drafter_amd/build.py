"""Build libdspark.so (HIP for gfx950) in-tree with hipcc.

Every source is compiled with packed-fp32 VALU instructions disabled; hipcc
still forms MFMA and ordinary vector code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdspark.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


# Sources with no kernels: the whole host side of the C ABI (validation,
# layout planning, launch sequencing) and the GEMM planner.
HOST_ONLY_SOURCES = ("dspark_api.hip", "k_gemv.hip")
SAN_DIR = os.path.join(BUILD_DIR, "hostsan")
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def build_host_sanitized(driver_src: str) -> str:
    """Host-side sanitizer build: the kernel-free sources compiled host-only
    with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    regular objects of the kernel sources into libdspark_hostsan.so, and the
    C++ driver `driver_src` built with the same sanitizers against it.
    Returns the driver's path.  (The GPU code is not sanitized: GPU
    sanitizers are not used here.)"""
    os.makedirs(SAN_DIR, exist_ok=True)
    kernel_objs = [os.path.join(BUILD_DIR, os.path.basename(f) + ".o") for f in sources()
                   if os.path.basename(f) not in HOST_ONLY_SOURCES]
    if not all(os.path.exists(o) for o in kernel_objs):
        build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    objs = []
    for name in HOST_ONLY_SOURCES:
        obj = os.path.join(SAN_DIR, name + ".o")
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "--cuda-host-only", "-fPIC",
               "-fno-omit-frame-pointer", *san, "-c", os.path.join(CSRC, name), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized host compile failed on {name}:\n{r.stdout}{r.stderr}")
        objs.append(obj)
    lib = os.path.join(SAN_DIR, "libdspark_hostsan.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, *objs, *kernel_objs, "-o", lib],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}{r.stderr}")
    exe = os.path.join(SAN_DIR, "abi_host_check")
    r = subprocess.run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        driver_src, "-L" + SAN_DIR, "-ldspark_hostsan", "-Wl,-rpath," + SAN_DIR, "-o", exe],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"driver build failed:\n{r.stdout}{r.stderr}")
    return exe


if __name__ == "__main__":
    print(build(verbose=True))

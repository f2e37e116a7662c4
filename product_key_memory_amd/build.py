"""Builds libpkm.so (the HIP kernels and the C ABI of include/pkm.h) in-tree
with hipcc for gfx950.  Run as ``python -m product_key_memory_amd.build``."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkm.so")
SOURCES = ["gemm_f32.hip", "select.hip", "gather.hip", "backward.hip", "batch_norm.hip", "pkm_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


C_DRIVER_SRC = os.path.join(ROOT, "tests", "c_driver", "pkm_forward_main.c")
C_DRIVER = os.path.join(ROOT, "tests", "c_driver", "pkm_forward_main")


def build_c_driver():
    """The plain-C test caller of the library (no torch in its process),
    linked against the in-tree libpkm.so and the HIP runtime."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           C_DRIVER_SRC, "-o", C_DRIVER + ".tmp", "-L", PKG, "-lpkm", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../product_key_memory_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {C_DRIVER_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(C_DRIVER + ".tmp", C_DRIVER)
    return C_DRIVER


def build(verbose=False):
    """Compile every source and link libpkm.so, then the plain-C test
    caller; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    build_c_driver()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the C ABI consumer (tests/c_abi/fckl_c_driver) against the in-tree libfckl.so.

Host code only: it includes include/fckl.h and the HIP runtime and links libfckl.so,
with an rpath to the package directory so that the GPU test can run it in place.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "chunked_top_kl_chunk_amd")
EXE = os.path.join(HERE, "fckl_c_driver")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hipcc = os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = "hipcc"
    cmd = [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "fckl_c_driver.cpp"),
           "-L", PKG, "-lfckl", "-Wl,-rpath,$ORIGIN/../../chunked_top_kl_chunk_amd", "-o", EXE]
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build())

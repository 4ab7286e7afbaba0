"""Builds libresolvent.so (the HIP kernels for gfx950 and the C ABI) in-tree."""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libresolvent.so")

ARCH = "gfx950"
# Packed fp32 VALU instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_library(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    kobjs = []
    for src in ("resolvent_kernels", "chain_kernels", "decode_kernels", "export_kernels",
                "noalloc"):
        kobjs.append(os.path.join(BUILD, src + ".o"))
        _run([hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c",
              os.path.join(CSRC, src + ".hip"), "-o", kobjs[-1]], verbose)
    aobj = os.path.join(BUILD, "resolvent_abi.o")
    rocm_inc = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "include")
    _run([hipcc, *COMMON, "-D__HIP_PLATFORM_AMD__", "-I", rocm_inc, "-x", "c++", "-c",
          os.path.join(CSRC, "resolvent_abi.cpp"), "-o", aobj], verbose)
    tmp = LIBRARY + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *kobjs, aobj, "-o", tmp], verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build_library(verbose=True))

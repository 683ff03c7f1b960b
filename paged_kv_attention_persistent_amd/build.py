"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_attention_persistent_amd.build

The library holds the host runtime (C++) and the gfx950 kernels (HIP) in one
shared object next to this file.  Packed-FP32 instructions are disabled for
the device code (hipcc's host pass warns that it does not know the feature;
that warning is harmless).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = ["pkv_kernels.hip", "pkv_api.cpp", "queue_plan.cpp", "pkv_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"),
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out,
            "-L", os.path.join(os.path.dirname(os.path.dirname(hipcc())), "lib"), "-lrocprofiler-sdk-roctx", *extra]


def build(verbose: bool = False) -> str:
    """Compile every source into libpkv.so (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi", "pkv_c_client.c")
CLIENT = os.path.join(ROOT, "_build", "pkv_c_client")


def build_c_client(verbose: bool = False) -> str:
    """Compile the plain-C consumer of the C ABI (tests/c_abi) with the host C
    compiler, linked against libpkv.so next to this file and the HIP runtime."""
    os.makedirs(os.path.dirname(CLIENT), exist_ok=True)
    rocm = os.path.dirname(os.path.dirname(hipcc()))
    cmd = [shutil.which("gcc") or "gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), CLIENT_SRC,
           "-o", CLIENT, "-L", HERE, "-lpkv", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../paged_kv_attention_persistent_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    return CLIENT


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_client(verbose=True))

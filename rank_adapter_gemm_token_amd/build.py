"""Build liblora.so (HIP kernels for gfx950 + C++ host runtime) in-tree.

    python -m rank_adapter_gemm_token_amd.build [-v]

Each source compiles to an object under _build/ in parallel, then hipcc links
rank_adapter_gemm_token_amd/liblora.so.  Also links libcalibrate.so, the
measurement harness's achievable-peak probes (no part of the library).
Always recompiles.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblora.so")
CALIB_LIB = os.path.join(PKG, "libcalibrate.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "ledger.cpp", "residency.cpp", "route.hip", "pad_copy.hip", "apply_kernels.hip", "gemm_decode.hip",
           "gemm_tiled.hip", "shrink_expand.hip", "scratch.hip"]
CALIB_SOURCES = ["calibrate.hip"]

# Packed-fp32 VALU instructions are kept out of every device object.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CXXFLAGS = ["-std=c++17", "-O3", "-fPIC", "--offload-arch=" + ARCH, "-Wall",
            "-Wno-unused-command-line-argument", "-I" + os.path.join(ROOT, "include")]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CXXFLAGS, *DEVICE_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if os.environ.get("LORA_RESOURCE_USAGE"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is noise.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (src, err))
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

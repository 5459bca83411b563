"""Compile the HIP library (libpkv.so) for gfx950, in-tree.

Every call recompiles all sources (each translation unit in parallel) and
links `paged_kv_cache_430_amd/libpkv.so`. hipcc cross-compiles without a GPU.

`python -m paged_kv_cache_430_amd._build --asan` builds a second library,
`_build_asan/libpkv_asan.so`, whose host-only sources (argument validation,
the allocator, the prefix index) are compiled by g++ with AddressSanitizer;
the kernels are the same objects as in libpkv.so. Run the host tests on it
with the sanitizer runtime preloaded (the interpreter itself is not
instrumented):

    LD_PRELOAD=$(g++ -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
    PKV_LIB=paged_kv_cache_430_amd/_build_asan/libpkv_asan.so \
    python -m pytest tests -m "not gpu"
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"
SOURCES = ["pkv_api.cpp", "allocator.cpp", "prefix.cpp", "kv_append.hip", "decode.hip", "prefill.hip",
           "read_probe.hip", "mfma_probe.hip"]
HOST_SOURCES = ["pkv_api.cpp", "allocator.cpp", "prefix.cpp"]   # no device code
ASAN_DIR = os.path.join(PKG, "_build_asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libpkv_asan.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # hipcc forms packed-fp32 instructions by itself from float code; keep them off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]
# Per-source additions. The prefill kernel keeps its MFMA accumulators in
# ordinary VGPRs (the VGPR form of the MFMA instructions), so the per-tile
# rescale of O does not copy them out of and back into accumulation registers.
# Its scores never hold NaN (rows outside the sequence read as zeros, masked
# scores are −inf), so maxima need no NaN canonicalisation (-fno-honor-nans).
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]}


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libpkv.so")
    return path


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build_asan(verbose=False):
    """libpkv.so's kernels plus AddressSanitizer-instrumented host sources.

    The host sources call the HIP runtime API only, so g++ compiles them
    against the ROCm headers; the kernel objects come from build()."""
    build(verbose=verbose)
    os.makedirs(ASAN_DIR, exist_ok=True)
    gxx = shutil.which("g++")
    if not gxx:
        raise RuntimeError("g++ not found")
    flags = ["-O1", "-g", "-fPIC", "-std=c++17", "-Wall", "-fvisibility=hidden", "-fno-omit-frame-pointer",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")]
    san = "-fsanitize=address"
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(ASAN_DIR, src + ".o")
        _run([gxx, *flags, san, "-c", os.path.join(CSRC, src), "-o", obj], f"g++ (asan) {src}")
        objs.append(obj)
    objs += [os.path.join(BUILD, src + ".o") for src in SOURCES if src not in HOST_SOURCES]
    _run([gxx, "-shared", san, "-o", ASAN_LIB, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], "asan link")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv[1:]:
        build_asan(verbose=True)
    else:
        build(verbose=True)

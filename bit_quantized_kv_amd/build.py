"""Build libkvq.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_quantized_kv_amd.build

Device code is compiled with packed-FP32 instructions disabled and with the
default IEEE fp32 semantics (correctly rounded division and square root, no
denormal flushing) that the bit-exact quantizer relies on.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["kvq_store.hip", "kvq_decode.hip", "kvq_extend.hip", "kvq_bandwidth.hip", "kvq_debug.hip", "kvq_api.cpp"]
ARCH = "gfx950"

COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [_hipcc(), *lang, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


CONVCHECK_SRC = os.path.join(ROOT, "tests", "conv_check.hip")
CONVCHECK_LIB = os.path.join(ROOT, "tests", "libkvq_convcheck.so")


def build_convcheck() -> str:
    """The test suite's exhaustive conversion checks (tests/conv_check.hip), built
    with the library's device flags so the instructions run in the same modes."""
    tmp = CONVCHECK_LIB + ".tmp"
    cmd = [_hipcc(), "-x", "hip", *COMMON, "-shared", CONVCHECK_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for conv_check.hip:\n{r.stderr}")
    os.replace(tmp, CONVCHECK_LIB)
    return CONVCHECK_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

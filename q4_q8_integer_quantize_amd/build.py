"""Build librz.so (the HIP kernels and the C ABI) in-tree for gfx950, the
benchmark's streaming-read helper librz_stream_read.so, and the plain C program
tests/native/abi_consumer that drives librz.so through include/rz.h alone.

    python -m q4_q8_integer_quantize_amd.build

Every source is compiled by hipcc with packed-fp32 instructions disabled, IEEE
fp32 division and no fast-math (the Q8_1 codes depend on correctly rounded
division and ties-to-even rounding).  The fp32-activation kernels also need
fp16 denormals preserved (they take 4-bit weights as fp16 denormals into
v_fma_mix_f32), which is the default for these flags; do not add a flag that
flushes fp16 denormals.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librz.so")
# measurement helper for bench.py (a plain streaming read), outside librz.so
READ_SRC = "stream_read.hip"
READ_LIB = os.path.join(PKG, "librz_stream_read.so")
# a C consumer of the ABI (no Python, no torch), run by the tests
CONSUMER_SRC = os.path.join(ROOT, "tests", "native", "abi_consumer.c")
CONSUMER = os.path.join(ROOT, "tests", "native", "abi_consumer")

SOURCES = ["q8_1_quantize.hip", "q4k_gemv.hip", "q4k_gemv_f32.hip", "q4k_gemm_mfma.hip",
           "q4k_gemv_multi.hip", "q4_0_gemv.hip", "swiglu_ffn.hip", "rmsnorm_q8_1.hip",
           "q4k_gemv_xf32.hip", "topk.hip", "rz_abi.cpp"]
ARCH = os.environ.get("RZ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
        # MFMA results in VGPRs (read by the rescale right away) instead of AGPRs
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link librz.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    _link(objs, LIB)
    _link([_compile(READ_SRC)], READ_LIB)
    build_consumer(CONSUMER)
    if verbose:
        print("built", LIB, READ_LIB, "and", CONSUMER)
    return LIB


def build_consumer(out: str) -> str:
    """Compile tests/native/abi_consumer.c with the host C compiler against
    include/rz.h, librz.so and the HIP runtime; returns ``out``."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    pkg_from_out = os.path.relpath(PKG, os.path.dirname(os.path.abspath(out)))
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", INCLUDE,
           CONSUMER_SRC, "-L", PKG, "-lrz", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/" + pkg_from_out, "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("gcc failed on the ABI consumer:\n%s\n%s" % (" ".join(cmd), res.stderr))
    return out


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, lib)


if __name__ == "__main__":
    build()
    sys.exit(0)

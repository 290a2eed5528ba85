"""Build libqdecode.so (the HIP library) for gfx950 with hipcc.

Sources are compiled in parallel into _build/ and linked into
quantized_decode_q4k_amd/libqdecode.so.  Always rebuilds when called.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqdecode.so")

SOURCES = ["qd_abi.hip", "qd_gemv.hip", "qd_gemv_stream.hip", "qd_gemv_mfma.hip", "qd_gemv_i8.hip", "qd_dequant.hip",
           "qd_prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 arithmetic stays off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


# Per-file device flags: the batch GEMV's products are read by the vector
# ALU right away, so its MFMA results go to ordinary vector registers (no
# accumulation-register copies).
FILE_FLAGS = {"qd_gemv_mfma.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_c_example() -> str:
    """tests/c_abi_example.bin: a plain-C program calling the C ABI (host code
    only, gcc) against the HIP runtime and the C oracle."""
    src = os.path.join(ROOT, "tests", "c_abi_example.c")
    out = os.path.join(ROOT, "tests", "c_abi_example.bin")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-I", os.path.join(rocm, "include"), src,
           os.path.join(ROOT, "oracle", "oracle.c"), "-o", out + ".tmp",
           "-L", HERE, "-lqdecode", "-Wl,-rpath,$ORIGIN/../quantized_decode_q4k_amd",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for c_abi_example.c:\n{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())

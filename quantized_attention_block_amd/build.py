"""Builds libsage.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m quantized_attention_block_amd.build
    python -m quantized_attention_block_amd.build --sanitize

--sanitize builds, for CPU-only checking, the C ABI's host code (argument
validation, workspace sizing, error reporting) with g++ and
-fsanitize=address,undefined against launcher stubs that always fail
(_build/libsage_host_san.so), and the CPU oracle the same way
(_build/liboracle_san.so), then prints the command that runs the CPU test
suite on them (SAGE_LIBRARY / ORACLE_LIBRARY select the libraries, the ASan
runtime is preloaded).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsage.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["quantize.hip", "attn_fwd.hip", "decode.hip", "debug_cvt.hip", "abi.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized() -> tuple:
    os.makedirs(BUILD_DIR, exist_ok=True)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    lib = os.path.join(BUILD_DIR, "libsage_host_san.so")
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC] + san + \
          [os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "host_stubs.cpp"),
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    subprocess.run(cmd, check=True)
    orc = os.path.join(BUILD_DIR, "liboracle_san.so")
    cmd = ["g++", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"] + san + \
          [os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", orc]
    subprocess.run(cmd, check=True)
    return lib, orc


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        lib, orc = build_sanitized()
        asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
        print(f"SAGE_LIBRARY={lib} ORACLE_LIBRARY={orc} LD_PRELOAD={asan} "
              "ASAN_OPTIONS=detect_leaks=0 python -m pytest tests -m 'not gpu' -q")
    else:
        build(verbose=True)
    sys.exit(0)

"""Build libltc.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run from anywhere: `python lossless_tensor_compression_amd/build.py`.
Objects go to _build/ at the repository root; the library is written next
to this file.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libltc.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["ltc_compress.hip", "ltc_decompress.hip", "ltc_crc32.hip", "ltc_api.hip"]
# plain C++ (no device code): the host-side parsing of blob bytes
HOST_SOURCES = ["ltc_host.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
              "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# Packed FP32 instructions (v_pk_*_f32) stay off in device code.  hipcc's
# driver cannot forward -Xclang options to the device pass alone (-Xarch_device
# refuses options that take an argument), so the feature goes to both passes
# and the host pass reports, once per function, that x86 has no such feature;
# that line carries no information and is dropped from the build log.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "".join(line for line in r.stdout.splitlines(keepends=True) if HOST_FEATURE_NOTE not in line)
    if log:
        print(log, end="", flush=True)
    if r.returncode:
        raise subprocess.CalledProcessError(r.returncode, cmd, output=r.stdout)
    return obj


def _compile_host(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs += [_compile_host(s, verbose) for s in HOST_SOURCES]
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

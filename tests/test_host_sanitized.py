"""Sanitizer runs on the CPU (no GPU involved): the library's host code that
reads untrusted blob bytes, and the oracle's pins, under AddressSanitizer and
UndefinedBehaviorSanitizer (lmz README, "Building on lmz", reports its device
code clean under the vendor's memory, race and sync checkers; this is the
host-side counterpart here).

1. tests/host_parse_fuzz.cpp + csrc/ltc_host.cpp (header check, directory
   statistics, host-blob copy groups), built with g++ and
   -fsanitize=address,undefined, fuzzed with truncations, bit flips, random
   byte runs and extreme header fields of oracle-made blobs of every format.
2. oracle/ltc_oracle.c built with gcc and the same sanitizers, loaded in place
   of the plain build (LTC_ORACLE_LIB, libasan preloaded) while the oracle's
   pin tests run in a child process.
Any sanitizer report aborts the program (-fno-sanitize-recover=all,
halt_on_error), which fails the test."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_tensor_compression_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _blobs():
    """Oracle blobs of every kind the host code parses."""
    rng = np.random.default_rng(3)
    x = workloads.c1()[:50000]
    f32 = (rng.standard_normal(7001) * 0.02).astype(np.float32)
    u8 = rng.integers(0, 7, 9000).astype(np.uint8)
    base = x.copy()
    base[::3] ^= 1
    return {
        "v1_bf16": oracle.compress(x, 1, 4096),
        "v1_fp32_ragged": oracle.compress(f32, 3, 1024),
        "v1_fp16": oracle.compress(x.view(np.float16), 2, 2048),
        "v1_u8": oracle.compress(u8, 0, 512),
        "v2_bf16": oracle.compress(x, 1, 4096, shared_tables=True),
        "v2_fp32": oracle.compress(f32, 3, 1024, shared_tables=True),
        "delta_v1": oracle.compress_delta(x, base, 1, 4096),
        "delta_v2": oracle.compress_delta(x, base, 1, 4096, shared_tables=True),
        "top_last_bf16": oracle.compress(x, 1, 4096, top_last=True),
        "top_last_fp32_v2": oracle.compress(f32, 3, 1024, shared_tables=True, top_last=True),
        "top_last_delta": oracle.compress_delta(x, base, 1, 4096, top_last=True),
        "empty": oracle.compress(np.zeros(0, np.uint8), 0, 4096),
        "one_chunk": oracle.compress(x[:100], 1, 131072),
    }


def test_host_parsing_fuzzed_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_parse_fuzz")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_parse_fuzz.cpp"), os.path.join(CSRC, "ltc_host.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    files = []
    for name, b in _blobs().items():
        p = tmp_path / f"{name}.bin"
        b.tofile(p)
        files.append(str(p))
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, *files], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAILED" not in r.stdout and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    fuzzed = int(r.stdout.split()[1])
    accepted = int(r.stdout.split()[3])
    assert fuzzed > 50000 and accepted > 1000, r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("libasan not found")
    lib = str(tmp_path / "libltc_oracle_san.so")
    subprocess.run(["gcc", "-std=c99", "-fPIC", "-shared", "-fopenmp", *SAN,
                    os.path.join(ROOT, "oracle", "ltc_oracle.c"), "-o", lib, "-lm"], check=True)
    pins = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f.endswith(".py"))
    assert len(pins) >= 9
    env = dict(os.environ, LTC_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    # the child checks that it really loaded the sanitized build
    probe = ("import oracle; oracle.lib(); "
             "assert any('libltc_oracle_san' in l for l in open('/proc/self/maps')), 'plain oracle loaded'")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail

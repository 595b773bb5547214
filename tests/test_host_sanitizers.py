"""The library's host C++ under AddressSanitizer and UndefinedBehaviorSanitizer.

pa_api.cpp (argument validation, path choice, workspace layout, stream and
event handling) and block_manager.cpp (free list, tables, prefix cache with
reference counts) are compiled for the CPU with g++ and both sanitizers, the
kernel launchers replaced by stubs that launch nothing
(tests/sanitize/launch_stubs.cpp), and linked into a stand-in library.  A child
process then runs the block manager's tests (hand-worked cases and long random
runs checked against a Python model of the rules) and the C ABI's validation
tests against it.  Any sanitizer report aborts the child, and this test fails.
CPU only: no GPU is touched."""
import os
import shutil
import subprocess
import sys

import pytest

from helpers import ROOT

CSRC = os.path.join(ROOT, "paged_kv_attention_22_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT, "libpa_host_sanitized.so")
SOURCES = [os.path.join(CSRC, "pa_api.cpp"), os.path.join(CSRC, "block_manager.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")]
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def runtime(gxx, name):
    p = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def build(gxx):
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
               "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr}"
        objs.append(obj)
    cmd = [gxx, "-shared", *SAN, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr}"


def test_host_code_is_clean_under_asan_and_ubsan():
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("g++ or the HIP runtime library is not available")
    asan = runtime(gxx, "libasan.so")
    if asan is None:
        pytest.skip("the AddressSanitizer runtime is not available")
    build(gxx)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,                # the ASan runtime must come first
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PA_TEST_LIB": LIB,                # tests/conftest.py loads it in place of libpa.so
        "HIP_VISIBLE_DEVICES": "",         # no GPU in any case
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_block_manager.py"), os.path.join(ROOT, "tests", "test_abi.py"),
           # what needs the real library: its symbol table, its writable data,
           # and pa_decode_noalloc (a HIP source, not part of the host build)
           "-k", "not exports_every_declared_symbol and not keeps_no_mutable_state and not noalloc"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = (r.stdout[-4000:] + "\n" + r.stderr[-8000:])
    assert r.returncode == 0, f"sanitized run failed (rc {r.returncode}):\n{report}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, report
    assert " passed" in r.stdout, report

"""The cache re-layout of jolt_load_cache, built for the CPU alone with the
address and undefined-behaviour sanitizers (tests/cpu/layout_check.cpp):
every residual code read back through the MFMA decode kernel's unpacking
(pairs by mantissa injection, lane chunks and records), every A element at
the kernel's addresses and W2 = B G^T / s, for 2-, 4- and 8-bit residuals,
odd token counts, ranks above 256 and several layers per group.  Needs no
GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_cache_decode_jolt_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = CLANG if os.path.exists(CLANG) else shutil.which("clang++")
    if not cxx:
        pytest.skip("no clang++ for the sanitizer build")
    exe = str(tmp_path_factory.mktemp("layout") / "layout_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D_GLIBCXX_SANITIZE_VECTOR",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "cpu", "layout_check.cpp"),
           os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "rotation.cpp"),
           "-lpthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_layout_under_sanitizers(checker):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([checker], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "layout check OK" in r.stdout

"""The validation and planning code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU).  wq_validate.cpp and wq_plan.cpp, the host code that reads every caller-supplied
descriptor before any device work, are built with g++ and both sanitizers into a library
of their own (the planners' compute-unit query is a host stub), and the descriptor-rule
tests then run against that library in a child process: any out-of-bounds access,
use-after-free, signed overflow, misaligned access or invalid shift aborts it."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_quantized_gemm_amd", "csrc")
SOURCES = [os.path.join(CSRC, "wq_validate.cpp"), os.path.join(CSRC, "wq_plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_stub.cpp")]
# the tests whose library calls are all size queries, status strings or the version
TESTS = ["tests/test_validation.py", "tests/test_packing_layout.py", "tests/test_abi.py"]


def _asan_runtime():
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_validation_under_asan_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("g++ has no AddressSanitizer runtime")
    lib = str(tmp_path / "libwqhost_san.so")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-shared", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         *SOURCES, "-o", lib], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ)
    # the sanitizer runtime goes first; whatever the environment already preloads stays
    env["LD_PRELOAD"] = runtime + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["WQ_HOST_LIBRARY"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in r.stdout

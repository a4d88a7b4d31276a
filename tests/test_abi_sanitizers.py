"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

``fa_api.cpp`` (every entry point's checks) and ``fa_sizes.cpp`` (the workspace and grid size
arithmetic) are built for the host with g++ and the two sanitizers, linked with stand-in
launchers (``tests/abi_host/stub_launch.cpp``) instead of the kernels, and driven through every
validation path by ``tests/abi_host/validate_main.cpp``: rejected calls must return their status
without reaching a launcher, accepted ones must reach the right launcher, and extreme sizes must
not overflow.  Any sanitizer report fails the run.  No GPU code is built or run.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_attention_02_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "abi_host")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP host headers")
def test_validation_is_clean_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory(prefix="fa_abi_san_") as tmp:
        exe = os.path.join(tmp, "validate")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, "-I", HOST,
               os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_sizes.cpp"),
               os.path.join(HOST, "stub_launch.cpp"), os.path.join(HOST, "validate_main.cpp"),
               "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        # The process environment is passed on unchanged; ASan is told not to insist on being
        # the first library loaded.
        env = dict(os.environ,
                   ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out
        assert "all validation checks hold" in out
        assert "runtime error" not in out and "AddressSanitizer" not in out, out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP host headers")
def test_prefill_plan_invariants_under_asan_and_ubsan():
    """The chunked prefill's work plan (``fa_prefill_plan.h``, the same functions the plan kernel
    runs) executed on the host by ``tests/abi_host/plan_main.cpp`` for the benchmark mix, short-
    chunk mixes, edge cases and random mixes: full coverage of every output row and key range,
    every index inside its buffer, totals within the workspace bounds."""
    with tempfile.TemporaryDirectory(prefix="fa_plan_san_") as tmp:
        exe = os.path.join(tmp, "plan")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, os.path.join(CSRC, "fa_sizes.cpp"), os.path.join(HOST, "plan_main.cpp"),
               "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        env = dict(os.environ,
                   ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out
        assert "plan checks hold" in out, out
        assert "runtime error" not in out and "AddressSanitizer" not in out, out

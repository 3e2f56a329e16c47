"""The CPU-side code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds, with g++ and -fsanitize=address,undefined:
  * the oracle (oracle/spear_oracle.cpp);
  * the ABI's host code: csrc/api.hip compiled as host C++ (it holds no
    kernels), csrc/scheduler.cpp, and launch stubs (tests/sanitize_stubs.cpp)
    in place of the kernel files;
  * the decode work-split check (tests/partition_check.cpp);
then reruns the CPU test files that exercise them (oracle pins, scheduler,
ABI validation, work split) in a child interpreter with the sanitizer runtime
preloaded and those builds selected (SPEAR_ORACLE_LIB, SPEAR_EC_LIB,
SPEAR_SANITIZE_CXXFLAGS).  Any sanitizer report fails the run.  No GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantization_error_compensation_amd", "csrc")
OUT = os.path.join(ROOT, "tests", "_build")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g",
       "-O1"]


def _gxx(args):
    subprocess.check_call(["g++", "-std=c++17", "-shared", "-fPIC", *SAN, *args])


@pytest.fixture(scope="module")
def builds():
    os.makedirs(OUT, exist_ok=True)
    oracle_so = os.path.join(OUT, "libspear_oracle_san.so")
    _gxx(["-ffp-contract=off", "-fno-fast-math", os.path.join(ROOT, "oracle", "spear_oracle.cpp"),
          "-o", oracle_so])
    api_so = os.path.join(OUT, "libspear_ec_host_san.so")
    _gxx(["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
          "-I", CSRC, "-x", "c++", os.path.join(CSRC, "api.hip"), "-x", "none",
          os.path.join(CSRC, "scheduler.cpp"), os.path.join(ROOT, "tests", "sanitize_stubs.cpp"),
          "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", api_so])
    return oracle_so, api_so


def test_cpu_code_is_clean_under_asan_and_ubsan(builds):
    oracle_so, api_so = builds
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    env = dict(os.environ, LD_PRELOAD=asan, SPEAR_ORACLE_LIB=oracle_so, SPEAR_EC_LIB=api_so,
               SPEAR_SANITIZE_CXXFLAGS=" ".join(SAN),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    files = ["tests/test_oracle_pins.py", "tests/test_scheduler.py", "tests/test_abi_host.py",
             "tests/test_partition.py"]
    res = subprocess.run([sys.executable, "-m", "pytest", *files, "-m", "not gpu", "-q", "-x",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "LeakSanitizer"):
        assert marker not in out, out[-4000:]
    assert " passed" in out

"""The fp64 oracle and the C ABI's host-side validation, built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU (no GPU, no kernel launch).

tests/c/oracle_check.c runs the oracle through every input type, both variants, snapshots,
several thread counts and the decode step, checking exact properties of the recurrence as it
goes.  tests/c/api_check.cpp sends every entry point of include/gdn.h arguments that the host
validation must reject, and checks the status codes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    subprocess.run(["gcc", "-std=c11", *SAN, "-pthread", "-Wall", "-Wextra",
                    os.path.join(ROOT, "tests", "c", "oracle_check.c"), os.path.join(ROOT, "oracle", "gdn_oracle.c"),
                    "-lm", "-o", exe], check=True)
    _run(exe)


def _library_objects():
    build_dir = os.path.join(ROOT, "gated_deltanet_state_amd", "_build")
    names = ["gdn_decode.o", "gdn_chunk_valu.o", "gdn_chunk_mfma.o", "kda_chunk_mfma.o"]
    objs = [os.path.join(build_dir, n) for n in names]
    if not all(os.path.exists(o) for o in objs):
        subprocess.run(["python", os.path.join(ROOT, "gated_deltanet_state_amd", "build.py")], check=True)
    return objs


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers are missing")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_check")
    # the kernels' objects are linked as built (device code untouched); the validation code and
    # the driver are compiled for the host with the sanitizers
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN,
                    os.path.join(ROOT, "tests", "c", "api_check.cpp"),
                    os.path.join(ROOT, "gated_deltanet_state_amd", "csrc", "gdn_api.cpp"), *_library_objects(),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
    _run(exe)

"""The host ABI checks of test_abi_host.py, run against the C-ABI layer built
with AddressSanitizer and UndefinedBehaviorSanitizer.

mosaic_bsa_api.cpp holds all host-side validation, workspace carving and
error reporting.  It is compiled here by g++ on its own, with
-fsanitize=address,undefined, and linked with launch stubs
(tests/sanitize/launch_stubs.cpp) in place of the kernels: every argument
set the ABI tests pass is rejected during validation, so a stub that is
reached reports a HIP error and the test expecting another status fails.
The test module then runs in a child interpreter with the sanitizer runtime
preloaded; any report aborts it.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT, "libmosaic_bsa_host_asan.so")
ROCM = "/opt/rocm"


def _build() -> str:
    os.makedirs(OUT, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "spherical_block_sparse_amd", "csrc"),
           os.path.join(ROOT, "spherical_block_sparse_amd", "csrc", "mosaic_bsa_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"sanitizer build failed:\n{' '.join(cmd)}\n{r.stderr}"
    return LIB


def _runtime(name: str) -> str:
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else ""


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_checks_under_address_and_ub_sanitizers():
    lib = _build()
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan:
        pytest.skip("libasan.so not found")
    env = dict(os.environ)
    env["MOSAIC_ABI_TEST_LIB"] = lib
    env["LD_PRELOAD"] = ":".join(p for p in (asan, ubsan) if p)
    # the interpreter and torch are not built with the sanitizer: leak
    # tracking and allocator-mismatch reports would be about them
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:new_delete_type_mismatch=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail

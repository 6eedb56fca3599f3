"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU oracle (oracle/vq_oracle.c) runs seeded encode / top-2 / decode /
  smoothing / packing calls over every bit pattern of both element types,
  checking invariants that need no second implementation
  (tests/sanitize/oracle_driver.c).
* The C ABI's argument checks (product_vq_kv_amd/csrc/vq_capi.cpp) run on
  200,000 valid, invalid and extreme argument combinations, with the kernel
  launchers replaced by host stand-ins (tests/sanitize/capi_stubs.cpp), so no
  GPU is needed; every status must be one the header defines
  (tests/sanitize/capi_driver.cpp).
Both are built with the host compilers (gcc, g++), never for the GPU; any
overflow, out-of-bounds access or leak aborts the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr and "cannot find" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    print(run.stdout)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    return run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    out = _build_and_run(["gcc", "-std=c11", "-ffp-contract=off", *SAN,
                          os.path.join(ROOT, "oracle", "vq_oracle.c"),
                          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm",
                          "-o", exe], exe)
    assert "0 invariant failures" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_capi_argument_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "capi_san")
    out = _build_and_run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN,
                          "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
                          "-I" + os.path.join(ROOT, "product_vq_kv_amd", "csrc"),
                          os.path.join(ROOT, "product_vq_kv_amd", "csrc", "vq_capi.cpp"),
                          os.path.join(ROOT, "tests", "sanitize", "capi_stubs.cpp"),
                          os.path.join(ROOT, "tests", "sanitize", "capi_driver.cpp"),
                          "-o", exe], exe)
    assert "0 unknown statuses" in out

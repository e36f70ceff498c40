"""AddressSanitizer + UndefinedBehaviorSanitizer build of the library's host
code (csrc/host_pack.cpp: sizes, quantiser, packer, unpacker, split plans) and
of the CPU oracle (oracle/oracle.c), driven by tests/sanitize_driver.cpp over
every weight format and a spread of shapes. CPU only: the HIP kernels are not
part of this build, and no GPU code is built with a sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]


def _compile(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]


@pytest.mark.timeout(600)
def test_host_code_and_oracle_under_asan_ubsan(tmp_path):
    if not (shutil.which("g++") and shutil.which("gcc")):
        pytest.skip("gcc/g++ not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "weight_quantized_gemm_amd", "csrc"), "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__"]
    d = str(tmp_path)
    _compile(["gcc", "-std=c11", *SAN, "-c", os.path.join(ROOT, "oracle", "oracle.c"),
              "-o", "oracle.o"], d)
    _compile(["g++", "-std=c++17", *SAN, *inc, "-c",
              os.path.join(ROOT, "weight_quantized_gemm_amd", "csrc", "host_pack.cpp"),
              "-o", "host_pack.o"], d)
    _compile(["g++", "-std=c++17", *SAN, *inc, "-c",
              os.path.join(ROOT, "tests", "sanitize_driver.cpp"), "-o", "driver.o"], d)
    _compile(["g++", *SAN, "driver.o", "host_pack.o", "oracle.o", "-lm", "-o", "driver"], d)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([os.path.join(d, "driver")], cwd=d, capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) > 300
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr

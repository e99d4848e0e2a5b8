"""The C-ABI host layer under AddressSanitizer and UBSan (CPU only).

Builds libswa with the sanitizers on its host code (device code is built
as usual) and tests/capi_host_checks.c against it, then runs the program:
every call is rejected by the library's argument checks before any launch,
so no GPU is needed.  Any memory error or undefined behaviour in the
descriptor checks, the split plan or the workspace arithmetic fails the
test.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

from tests.conftest import ROOT

ROCM = "/opt/rocm"
CSRC = os.path.join(ROOT, "sliding_window_attention_ring_amd", "csrc")
SOURCES = ["swa_capi.hip", "swa_append.hip", "swa_decode.hip", "swa_decode_int8.hip", "swa_reuse.hip"]


@pytest.mark.slow
def test_host_layer_under_sanitizers():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    tmp = tempfile.mkdtemp(prefix="swa_san_")
    try:
        lib = os.path.join(tmp, "libswa_san.so")
        # sanitizers on the host pass only: each flag follows -Xarch_host
        host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer"]
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san + \
              ["-I", os.path.join(ROOT, "include")] + [os.path.join(CSRC, f) for f in SOURCES] + ["-o", lib]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, r.stderr[-2000:]
        exe = os.path.join(tmp, "host_checks")
        c_flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__"]
        c_flags.append("-fsanitize=address,undefined")  # host C program, no device code
        r = subprocess.run([clang] + c_flags + ["-I", os.path.join(ROOT, "include"),
                                                os.path.join(ROOT, "tests", "capi_host_checks.c"), "-o", exe,
                                                "-L", tmp, "-lswa_san", "-Wl,-rpath," + tmp],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0 and "host checks ok" in r.stdout, (r.stdout + r.stderr)[-3000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)

"""The C ABI used from plain C: csrc/swa_example.c (built next to libswa.so)
allocates with hipMalloc, appends, decodes and validates through
include/swa.h only, and checks closed forms (one visible token -> its value
row exactly; identical keys -> mean of the values) and an error code."""

import os
import subprocess

import pytest

from tests.conftest import ROOT
from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def test_c_program_through_the_abi():
    require_gpu()
    exe = os.path.join(ROOT, "sliding_window_attention_ring_amd", "swa_example")
    assert os.path.exists(exe), "swa_example is not built: run the build first"
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "swa_example ok" in res.stdout

"""Build ``libswa.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m sliding_window_attention_ring_amd.build``.  hipcc
cross-compiles the device code, so no GPU is needed to build.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libswa.so")
EXAMPLE = os.path.join(PKG, "swa_example")
SOURCES = ["swa_capi.hip", "swa_append.hip", "swa_decode.hip", "swa_decode_int8.hip", "swa_reuse.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def command(out: str = LIB, defines=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        *[f"-D{d}" for d in defines],
        # packed fp32 instructions stay off: plain v_fma/v_add only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"),
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build_example(verbose: bool = True) -> str:
    """Compile csrc/swa_example.c, a plain C program that uses libswa.so
    through include/swa.h only."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           os.path.join(CSRC, "swa_example.c"), "-o", EXAMPLE,
           "-L", PKG, "-lswa", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"building the C example failed:\n{res.stderr}")
    return EXAMPLE


def build(verbose: bool = True, out: str = LIB, defines=()) -> str:
    """Compile every source into ``libswa.so`` next to this file (always rebuilds).

    ``defines`` (e.g. ``["SWA_INT8_UB=4"]``) override the kernels' tuning
    constants; ``out`` writes the library elsewhere (load it with SWA_LIB).
    """
    tmp = out + ".tmp"
    cmd = command(tmp, defines)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln and "(ignoring feature)" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    a = ap.parse_args()
    build(out=a.out, defines=a.defines)
    if a.out == LIB:
        build_example()

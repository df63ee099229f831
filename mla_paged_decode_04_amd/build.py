"""Build step: compile the HIP sources for gfx950 into in-tree shared libraries.

    python -m mla_paged_decode_04_amd.build

produces ``mla_paged_decode_04_amd/libmla_decode.so`` (host C ABI + device
code objects for gfx950) and ``libmla_probe.so`` (the achievable-peak probe,
include/mla_probe.h). hipcc cross-compiles without a GPU present.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# host C ABI + planner + combine, one file per decode kernel, the cache append
# and the absorbed projections
SRCS = [os.path.join(CSRC, f) for f in ("mla_decode.hip", "mla_narrow.hip", "mla_wide.hip", "mla_wide128.hip", "mla_append.hip",
                                        "mla_absorb.hip")]
LIB = os.path.join(PKG, "libmla_decode.so")
PROBE_SRCS = [os.path.join(CSRC, "mla_probe.hip")]
PROBE_LIB = os.path.join(PKG, "libmla_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed fp32 VALU forms (v_pk_{add,mul,fma}_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _compile(srcs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile both libraries (always; a stale build is never reused).
    Returns the decode library's path."""
    _compile(SRCS, LIB, verbose)
    _compile(PROBE_SRCS, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Compiles the gfx950 scan library (libssd.so) in place with hipcc.

    python -m complex_chunkwise_ssd_amd.build
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssd.so")
ARCH = "gfx950"


def hipcc_command(out: str, extra=()):
    return [
        "hipcc", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep hipcc from forming packed fp32 instructions on its own
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I" + INCLUDE, "-I" + CSRC, *extra,
        os.path.join(CSRC, "ssd_api.hip"), "-o", out,
    ]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed for libssd.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

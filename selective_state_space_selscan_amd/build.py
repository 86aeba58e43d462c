"""Build libselscan.so (HIP, gfx950) in place.

    python -m selective_state_space_selscan_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).  The host pass warns
that it does not know that feature; the warning is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libselscan.so")
ARCH = os.environ.get("SELSCAN_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIP_FLAGS, *extra_flags, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (proc.returncode, proc.stdout))
    if verbose and out:
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

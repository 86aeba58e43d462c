"""Build libselscan.so (HIP, gfx950) in place.

    python -m selective_state_space_selscan_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).  The host pass warns
that it does not know that feature; the warning is harmless.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "--hip-link" not in l and l.strip())
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed (%d): %s\n%s" % (proc.returncode, " ".join(cmd),
                                                          proc.stdout))
    if verbose and out:
        print(out)


def build(verbose: bool = False, extra_flags=(), jobs: int = 0) -> str:
    """Compile every csrc/*.hip to an object (in parallel), then link."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if jobs <= 0:
        try:
            jobs = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            jobs = os.cpu_count() or 1
        jobs = max(1, min(jobs, 16))
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="selscan_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in sources()]
        cmds = [[hipcc, *compile_flags, *extra_flags, "-c", src, "-o", obj]
                for src, obj in zip(sources(), objs)]
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

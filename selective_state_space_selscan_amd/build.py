"""Build libselscan.so (HIP, gfx950) in place.

    python -m selective_state_space_selscan_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).  The host pass warns
that it does not know that feature; the warning is harmless.
"""
from __future__ import annotations

import concurrent.futures
import glob
import hashlib
import os
import shutil
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


# Units that take the longest to compile (the N = 64 and N = 32 variant
# instantiations, the look-back plan, the default forward and its
# checkpoint-keeping twin), started first so
# that a parallel build does not end waiting on one of them.
SLOW_UNITS = ("_n64", "fwd_lookback", "fwd_stream.hip", "fwd_stream_keep", "_n32",
              "bwd_stream_zoh")


def sources():
    def rank(path):
        name = os.path.basename(path)
        for i, key in enumerate(SLOW_UNITS):
            if key in name:
                return (i, name)
        return (len(SLOW_UNITS), name)
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")), key=rank)


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


# Object cache of incremental builds (git-ignored): one object per source,
# keyed by the source, the repository headers it includes and the flags.
CACHE = os.path.join(os.path.dirname(PKG), "_build", "objs")


def _local_includes(path, seen):
    """The repository headers ``path`` includes, transitively (quoted
    includes resolved against the including file's directory)."""
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#include \""):
                inc = os.path.normpath(os.path.join(os.path.dirname(path), line.split('"')[1]))
                if os.path.exists(inc) and inc not in seen:
                    seen.add(inc)
                    _local_includes(inc, seen)
    return seen


def _unit_key(src, flags):
    h = hashlib.sha256()
    h.update(" ".join(flags).encode())
    for path in [src] + sorted(_local_includes(src, set())):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:24]


def build(verbose: bool = False, extra_flags=(), jobs: int = 0, incremental: bool = False) -> str:
    """Compile every csrc/*.hip to an object (in parallel), then link.  With
    ``incremental``, objects whose source, headers and flags are unchanged
    come from the object cache (the default compiles everything)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if jobs <= 0:
        try:
            jobs = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            jobs = os.cpu_count() or 1
        jobs = max(1, min(jobs, 16))
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    flags = [*compile_flags, *extra_flags]
    with tempfile.TemporaryDirectory(prefix="selscan_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in sources()]
        cmds, cached = [], []
        for src, obj in zip(sources(), objs):
            key = os.path.join(CACHE, "%s.%s.o" % (os.path.basename(src), _unit_key(src, flags)))
            if incremental and os.path.exists(key):
                shutil.copyfile(key, obj)
                continue
            cmds.append([hipcc, *flags, "-c", src, "-o", obj])
            cached.append((obj, key))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        os.makedirs(CACHE, exist_ok=True)
        for obj, key in cached:
            shutil.copyfile(obj, key)
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
    sys.exit(0)

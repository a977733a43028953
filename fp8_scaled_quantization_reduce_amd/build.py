"""Build libfp8q.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8q.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops keeps the compiler from forming packed fp32 instructions.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _jobs() -> int:
    try:
        return max(1, int(os.environ.get("MAX_JOBS", "")))
    except ValueError:
        return max(1, min(os.cpu_count() or 4, 16))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one object each, in parallel) and link them
    into one shared library, in-tree."""
    tmp = LIB + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="fp8q_build_") as objdir:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + ".o")
            objs.append(obj)
            cmds.append([HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])
        with ThreadPoolExecutor(max_workers=min(_jobs(), len(cmds))) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

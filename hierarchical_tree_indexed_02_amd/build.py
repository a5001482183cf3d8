"""Compiles the HIP sources into the in-tree shared library libzha.so (gfx950).

Each source is compiled to its own object in parallel (the kernels of one file do not
depend on another file's device code), then the objects are linked into the library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzha.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-ffp-contract=fast",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _quiet(stderr: str) -> str:
    return "\n".join(l for l in (stderr or "").splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    """Always recompiles; writes libzha.so atomically."""
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="zha_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(pair):
            src, obj = pair
            cmd = [HIPCC, *FLAGS, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            return src, subprocess.run(cmd, capture_output=True, text=True)

        workers = max(1, min(len(srcs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(compile_one, zip(srcs, objs)))
        for src, res in results:
            errs = _quiet(res.stderr)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({res.returncode}):\n{errs}")
            if verbose and errs.strip():
                print(errs, file=sys.stderr)
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{_quiet(res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

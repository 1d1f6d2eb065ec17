"""Build the gfx950 HIP library (libgla_mi355x.so) in-tree with hipcc.

The library holds the kernels and the C ABI declared in include/gla.h; it
links only the HIP runtime (no torch). Each translation unit compiles in its
own hipcc process (in parallel), then one link produces the library.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgla_mi355x.so")
SOURCES = ["gla_kernels.hip", "gla_gated.hip", "gla_runs.hip", "ssw_kernels.hip", "gla_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops stay off: the compiler must not emit v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmpdir = tempfile.mkdtemp(prefix="gla_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            subprocess.run(cmd, check=True)
            return obj

        workers = min(len(SOURCES), max(1, (os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

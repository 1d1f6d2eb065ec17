"""The C ABI from a plain C program (tests/c_caller/gla_c_caller.c): no
Python, no torch between the caller and the library.

CPU: include/gla.h compiles on its own as strict C99; the caller compiles
and links against the built library and its host-side checks pass (version,
status strings, workspace sizes, argument errors before any launch).
GPU: the caller runs gla_fwd on seeded inputs written by the workload
generator and its output matches the float64 oracle (bar 5e-3).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_caller", "gla_c_caller.c")
PKG = os.path.join(ROOT, "recurrent_vision_token_gla_amd")
LIB = os.path.join(PKG, "libgla_mi355x.so")
ROCM = "/opt/rocm"


def _build(out_dir):
    if not os.path.exists(LIB):
        pytest.skip("the HIP library is not built")
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = os.path.join(out_dir, "gla_c_caller")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"), SRC,
           "-L", PKG, "-lgla_mi355x", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + PKG, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_header_is_strict_c99():
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                        "-x", "c", os.path.join(ROOT, "include", "gla.h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_caller_host_checks(tmp_path):
    exe = _build(str(tmp_path))
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "host ok" in r.stdout, r.stdout + r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,gh,gw,dk,dv,chunk,dirs", [
    (1, 6, 40, 40, 64, 64, 64, [2]),          # the 640x640 image regime, top to bottom
    (2, 2, 9, 17, 32, 64, 16, [1, 3]),        # ragged tail, per-batch directions, dk 32 / dv 64
])
def test_c_caller_forward_matches_oracle(tmp_path, B, H, gh, gw, dk, dv, chunk, dirs):
    import oracle
    from gpu_util import TOL, rel_err, say
    from recurrent_vision_token_gla_amd import workloads as W

    exe = _build(str(tmp_path))
    x = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=480 + gh + dk)
    for name, a in zip(("q", "k", "v", "gk"), x):
        a.tofile(os.path.join(str(tmp_path), name + ".bin"))
    say(f"c caller B={B} H={H} grid={gh}x{gw} dk={dk} dv={dv} chunk={chunk} dirs={dirs}")
    args = [exe, "run", str(tmp_path), str(B), str(H), str(gh), str(gw), str(dk), str(dv), str(chunk)]
    r = subprocess.run(args + [str(d) for d in dirs], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "run ok" in r.stdout, r.stdout + r.stderr
    o = np.fromfile(os.path.join(str(tmp_path), "o.bin"), dtype=np.float16).reshape(B, gh * gw, H, dv)
    err = rel_err(o.astype(np.float64), oracle.gla_forward(*x, gh, gw, dirs))
    say(f"  {r.stdout.strip()}  rel_err={err:.2e}")
    assert err <= TOL

"""Token-by-token fp64 recurrence: the oracle's definition of the forward.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The forward (GTR project page, "How GTR Works" and "A Kernel That Makes
Recurrence Fast"; ai.info summary of GTR, "Methodology in Plain English"):
key-only gated linear attention with a zero initial state, run along one scan
order of the patch grid, output put back in raster order:

    S_0 = 0,   S_t = diag(exp(g_t)) S_{t-1} + k_t^T v_t,   o_t = q_t S_t.

The carried-state form (ai.info summary of GTR, "Future Directions": the
state carried across frames) starts from a given S_0 [B, H, dk, dv] and can
also return the state after the last token, S_T.

Two implementations of the same loop are kept: the C one (gla_oracle.c,
OpenMP over independent value columns) for speed, and a numpy twin that is
vectorised over (batch, head) and used to cross-check it.
"""
from __future__ import annotations

import ctypes
from typing import Sequence

import numpy as np

from . import build as _build
from .scan_order import to_raster, to_scan

_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(_build.ensure_built())
        lib.gla_oracle_recurrence.restype = ctypes.c_int
        lib.gla_oracle_recurrence.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5
        lib.gla_oracle_recurrence_state.restype = ctypes.c_int
        lib.gla_oracle_recurrence_state.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 5
        lib.gla_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def oracle_threads() -> int:
    """Threads the C oracle's OpenMP loop uses."""
    return int(_load().gla_oracle_max_threads())


def _f64(a) -> np.ndarray:
    # exact upcast of the values the GPU receives (f16/f32 -> f64 is exact)
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def recurrence_c(q, k, v, g, s0=None, return_state: bool = False):
    """Scan-ordered [B, T, H, D] inputs -> scan-ordered o, in float64 (C).

    s0 is the state before the first token ([B, H, dk, dv], None for zero);
    with return_state the state after the last token is returned as well.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv), np.float64)
    lib = _load()
    if s0 is None and not return_state:
        rc = lib.gla_oracle_recurrence(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                       g.ctypes.data, o.ctypes.data, B, T, H, dk, dv)
    else:
        s0a = None if s0 is None else _f64(s0)
        if s0a is not None and s0a.shape != (B, H, dk, dv):
            raise ValueError("s0 must be [B, H, dk, dv]")
        sT = np.zeros((B, H, dk, dv), np.float64)
        rc = lib.gla_oracle_recurrence_state(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data,
            None if s0a is None else s0a.ctypes.data, o.ctypes.data, sT.ctypes.data,
            B, T, H, dk, dv)
    if rc != 0:
        raise ValueError("gla_oracle_recurrence rejected its arguments")
    if return_state:
        return o, sT
    return o


def recurrence_numpy(q, k, v, g, s0=None, return_state: bool = False):
    """Same recurrence as recurrence_c, looped over t, vectorised over (B, H)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        S = np.exp(g[:, t])[..., None] * S + k[:, t][..., None] * v[:, t][:, :, None, :]
        o[:, t] = np.einsum("bhd,bhde->bhe", q[:, t], S)
    if return_state:
        return o, S
    return o


def gla_forward(q, k, v, gk, grid_h: int, grid_w: int, dirs: Sequence[int],
                impl: str = "c", s0=None, return_state: bool = False):
    """Raster-ordered [B, T, H, D] inputs -> raster-ordered o (float64).

    dirs holds one direction code per batch element (0 L2R, 1 R2L, 2 T2B,
    3 B2T). The inputs are upcast exactly to float64, gathered into scan
    order, run through the recurrence, and scattered back. s0 / return_state
    as in recurrence_c; the states belong to the scan, so they carry no
    spatial order.
    """
    q, k, v, gk = _f64(q), _f64(k), _f64(v), _f64(gk)
    if q.shape[1] != grid_h * grid_w:
        raise ValueError("T must equal grid_h * grid_w")
    if len(dirs) != q.shape[0]:
        raise ValueError("one direction per batch element")
    run = recurrence_c if impl == "c" else recurrence_numpy
    s = lambda x: to_scan(x, grid_h, grid_w, dirs)
    res = run(s(q), s(k), s(v), s(gk), s0=s0, return_state=return_state)
    if return_state:
        return to_raster(res[0], grid_h, grid_w, dirs), res[1]
    return to_raster(res, grid_h, grid_w, dirs)

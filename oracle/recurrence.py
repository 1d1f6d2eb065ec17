"""Token-by-token fp64 recurrence: the oracle's definition of the forward.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The forward (GTR project page, "How GTR Works" and "A Kernel That Makes
Recurrence Fast"; ai.info summary of GTR, "Methodology in Plain English"):
key-only gated linear attention with a zero initial state, run along one scan
order of the patch grid, output put back in raster order:

    S_0 = 0,   S_t = diag(exp(g_t)) S_{t-1} + k_t^T v_t,   o_t = q_t S_t.

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
        lib.gla_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def oracle_threads() -> int:
    """Threads the C oracle's OpenMP loop uses."""
    return int(_load().gla_oracle_max_threads())


def _f64(a) -> np.ndarray:
    # exact upcast of the values the GPU receives (f16/f32 -> f64 is exact)
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def recurrence_c(q, k, v, g) -> np.ndarray:
    """Scan-ordered [B, T, H, D] inputs -> scan-ordered o, in float64 (C)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv), np.float64)
    rc = _load().gla_oracle_recurrence(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                       g.ctypes.data, o.ctypes.data, B, T, H, dk, dv)
    if rc != 0:
        raise ValueError("gla_oracle_recurrence rejected its arguments")
    return o


def recurrence_numpy(q, k, v, g) -> np.ndarray:
    """Same recurrence as recurrence_c, looped over t, vectorised over (B, H)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        S = np.exp(g[:, t])[..., None] * S + k[:, t][..., None] * v[:, t][:, :, None, :]
        o[:, t] = np.einsum("bhd,bhde->bhe", q[:, t], S)
    return o


def gla_forward(q, k, v, gk, grid_h: int, grid_w: int, dirs: Sequence[int],
                impl: str = "c") -> np.ndarray:
    """Raster-ordered [B, T, H, D] inputs -> raster-ordered o (float64).

    dirs holds one direction code per batch element (0 L2R, 1 R2L, 2 T2B,
    3 B2T). The inputs are upcast exactly to float64, gathered into scan
    order, run through the recurrence, and scattered back.
    """
    q, k, v, gk = _f64(q), _f64(k), _f64(v), _f64(gk)
    if q.shape[1] != grid_h * grid_w:
        raise ValueError("T must equal grid_h * grid_w")
    if len(dirs) != q.shape[0]:
        raise ValueError("one direction per batch element")
    run = recurrence_c if impl == "c" else recurrence_numpy
    s = lambda x: to_scan(x, grid_h, grid_w, dirs)
    o_scan = run(s(q), s(k), s(v), s(gk))
    return to_raster(o_scan, grid_h, grid_w, dirs)

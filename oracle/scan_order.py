"""Scan orders over the patch grid, built from plain numpy grid operations.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Each GTR block scans the stride-16 patch grid in exactly one order -- left to
right, right to left, top to bottom or bottom to top -- and the output is put
back in spatial order afterwards (GTR project page, "How GTR Works"; ai.info
summary of GTR, "Methodology in Plain English").

Reading taken where the pages are silent: tokens are stored in raster
(row-major) order; left->right is that raster order; top->bottom walks the
columns left to right, each column top to bottom; right->left and
bottom->top are the full reversals of those two sequences, so reversing the
direction is the same as reversing the token sequence.

scan_order(...)[t] is the raster index of the token visited at scan position t.
"""
from __future__ import annotations

import numpy as np

L2R, R2L, T2B, B2T = 0, 1, 2, 3


def scan_order(grid_h: int, grid_w: int, direction: int) -> np.ndarray:
    if grid_h <= 0 or grid_w <= 0:
        raise ValueError("grid sides must be positive")
    raster = np.arange(grid_h * grid_w, dtype=np.int64).reshape(grid_h, grid_w)
    if direction == L2R:
        return raster.ravel().copy()
    if direction == R2L:
        return raster.ravel()[::-1].copy()
    if direction == T2B:
        return raster.T.ravel().copy()
    if direction == B2T:
        return raster.T.ravel()[::-1].copy()
    raise ValueError(f"unknown direction {direction}")


def to_scan(x: np.ndarray, grid_h: int, grid_w: int, dirs) -> np.ndarray:
    """Gather [B, T, ...] raster-ordered x into per-batch scan order."""
    out = np.empty_like(x)
    for b, d in enumerate(dirs):
        out[b] = x[b][scan_order(grid_h, grid_w, int(d))]
    return out


def to_raster(y: np.ndarray, grid_h: int, grid_w: int, dirs) -> np.ndarray:
    """Scatter [B, T, ...] scan-ordered y back to raster order."""
    out = np.empty_like(y)
    for b, d in enumerate(dirs):
        out[b][scan_order(grid_h, grid_w, int(d))] = y[b]
    return out

"""Float64 oracle of the GLA block's output epilogue and of the Spatial SwiGLU
channel mixer. TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Output gate (ai.info summary of GTR, "Methodology in Plain English": a
data-dependent output gate applied to the RMS-normalised output). The pages
give no formula; the plain reading, the gated-RMSNorm epilogue of the GLA
paper the pages cite (mlsanity reference list), per (batch, token, head):

    y = o / sqrt(mean_e(o_e^2) + eps) * w * silu(z),   silu(z) = z / (1 + exp(-z))

with o the GLA output row (dv values), z the caller's gate row (dv values,
computed from the block input by the caller) and w a learned weight of dv
values shared by the heads.

Spatial SwiGLU (ai.info summary, "Methodology in Plain English"; project
page, "How GTR Works"): a SwiGLU mixer whose non-gated input path is
filtered per channel by a 3x3 kernel over the 2-D patch grid before the
gating product, with tokens back in sequence order afterwards. With a = W1 x (gate branch) and u = W3 x (value branch)
already projected by the caller, per token (y, x) of the grid and channel c:

    h[y, x, c] = silu(a[y, x, c]) * (bias[c] + sum_{i, j in 0..2}
                 weight[c, i, j] * u[y + i - 1, x + j - 1, c])

with zero padding outside the grid (same-size output) and the weight read as
a cross-correlation, the deep-learning convention; the output projection W2
is the caller's. Tokens are in raster order: token index = y * grid_w + x.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(z) -> np.ndarray:
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def rmsnorm_gate(o, gate, weight, eps: float) -> np.ndarray:
    """[..., dv] rows: o / sqrt(mean(o^2) + eps) * weight * silu(gate)."""
    o = _f64(o)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + float(eps))
    return o / rms * _f64(weight) * silu(gate)


def spatial_swiglu(a, u, weight, bias, grid_h: int, grid_w: int) -> np.ndarray:
    """a, u: [B, T, F] with T = grid_h * grid_w in raster order; weight
    [F, 3, 3]; bias [F] or None. Returns h [B, T, F] in float64."""
    a, u, w = _f64(a), _f64(u), _f64(weight)
    B, T, F = u.shape
    if T != grid_h * grid_w:
        raise ValueError("T must equal grid_h * grid_w")
    g = u.reshape(B, grid_h, grid_w, F)
    pad = np.zeros((B, grid_h + 2, grid_w + 2, F))
    pad[:, 1:-1, 1:-1] = g
    conv = np.zeros((B, grid_h, grid_w, F)) if bias is None else np.broadcast_to(
        _f64(bias), (B, grid_h, grid_w, F)).copy()
    for i in range(3):
        for j in range(3):
            conv += w[:, i, j] * pad[:, i:i + grid_h, j:j + grid_w]
    return silu(a) * conv.reshape(B, T, F)

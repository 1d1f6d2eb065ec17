"""Seeded synthetic workloads for the key-only GLA forward.

This module only draws inputs. It holds none of the forward's arithmetic, so
both the HIP path and the CPU oracle can take their inputs from here without
sharing any of the computation.

Workload shapes follow the pages' image regimes: a stride-16 patch grid, so a
640x640 image gives a 40x40 grid of 1,600 tokens and 1280x1280 gives 80x80 =
6,400 tokens (ai.info summary of GTR, "Main Findings", kernel-level speedups;
project page, "Accuracy Scales with Input Resolution"). The pages give no
activation statistics; the value distributions below are a stated synthetic
recipe (q, k, v standard normal, q scaled by dk^-1/2, log-gates from a
log-sigmoid of a normal draw), and they stand in for GTR activations on COCO
images, which are not used.

Layout of every tensor: [B, T, H, D], raster (row-major) token order,
contiguous. Direction codes: 0 left->right, 1 right->left, 2 top->bottom,
3 bottom->top.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

L2R, R2L, T2B, B2T = 0, 1, 2, 3
DIRECTION_NAMES = {L2R: "L2R", R2L: "R2L", T2B: "T2B", B2T: "B2T"}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a sequence of forward calls of one shape."""

    index: int  # 0-based position in WORKLOADS
    name: str
    B: int
    H: int
    grid_h: int
    grid_w: int
    dk: int
    dv: int
    chunk: int
    dtype: str  # "f16" or "f32": the type of q, k, v, gk and o
    gate: str  # "plain": logsigmoid(N(0,1))/16; "mixed": per-channel mix
    calls: int  # forward calls in one pass of the workload
    dir_mode: str  # "fixed_l2r", "each", "per_batch", "cycle_calls"

    @property
    def T(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def np_dtype(self):
        return np.float16 if self.dtype == "f16" else np.float32

    def directions(self, call: int) -> List[int]:
        """Per-batch direction codes (length B) of forward call `call`."""
        if self.dir_mode == "fixed_l2r":
            return [L2R] * self.B
        if self.dir_mode in ("each", "cycle_calls"):
            # one call per scan order, cycling L2R, R2L, T2B, B2T
            return [call % 4] * self.B
        if self.dir_mode == "per_batch":
            return [b % 4 for b in range(self.B)]
        raise ValueError(self.dir_mode)

    def tokens_per_call(self) -> int:
        return self.B * self.T


WORKLOADS = [
    Workload(0, "tiny_8x8_fp32", B=1, H=1, grid_h=8, grid_w=8, dk=32, dv=32,
             chunk=16, dtype="f32", gate="plain", calls=1, dir_mode="fixed_l2r"),
    Workload(1, "img640_40x40_h6", B=1, H=6, grid_h=40, grid_w=40, dk=64, dv=64,
             chunk=64, dtype="f16", gate="plain", calls=4, dir_mode="each"),
    Workload(2, "img1280_80x80_h6", B=1, H=6, grid_h=80, grid_w=80, dk=64, dv=64,
             chunk=64, dtype="f16", gate="plain", calls=4, dir_mode="each"),
    Workload(3, "batched_b8_40x40_h12", B=8, H=12, grid_h=40, grid_w=40, dk=64,
             dv=64, chunk=64, dtype="f16", gate="plain", calls=1,
             dir_mode="per_batch"),
    Workload(4, "stack12_b4_80x80_h16", B=4, H=16, grid_h=80, grid_w=80, dk=64,
             dv=64, chunk=64, dtype="f16", gate="mixed", calls=12,
             dir_mode="cycle_calls"),
]


def _log_sigmoid(x: np.ndarray) -> np.ndarray:
    # numerically stable log(1 / (1 + exp(-x))) in float64
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def seed_for(workload_index: int, call: int) -> int:
    return 1000 * (workload_index + 1) + call


def make_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype,
                seed: int, gate: str = "plain",
                gate_override: Optional[np.ndarray] = None):
    """Draw q, k, v, gk of shape [B, T, H, D] in `dtype` (numpy float16/32).

    Draw order: q, k, v, [channel mask for the mixed gate], gate normals.
    Values are drawn in float64, scaled, then rounded once to `dtype`.
    gate == "plain":  gk = logsigmoid(N(0,1)) / 16.
    gate == "mixed":  each (b, h, key-dim) channel picks, by a fair coin, a
                      near-zero regime logsigmoid(N(4,1))/16 or a strong regime
                      logsigmoid(N(-4,1)); every token draws from its channel's
                      regime.
    gate_override, if given, is broadcast to [B, T, H, dk] and used as gk.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk)) * (dk ** -0.5)
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    if gate_override is not None:
        g = np.broadcast_to(np.asarray(gate_override, np.float64), (B, T, H, dk))
    elif gate == "plain":
        g = _log_sigmoid(rng.standard_normal((B, T, H, dk))) / 16.0
    elif gate == "mixed":
        strong = rng.random((B, 1, H, dk)) < 0.5
        z = rng.standard_normal((B, T, H, dk))
        near = _log_sigmoid(z + 4.0) / 16.0
        hard = _log_sigmoid(z - 4.0)
        g = np.where(strong, hard, near)
    else:
        raise ValueError(gate)
    cast = lambda a: np.ascontiguousarray(a.astype(dtype))
    return cast(q), cast(k), cast(v), cast(g)


def workload_inputs(w: Workload, call: int):
    """Inputs of forward call `call` of workload `w` (fresh draw per call)."""
    return make_inputs(w.B, w.T, w.H, w.dk, w.dv, w.np_dtype,
                       seed_for(w.index, call), gate=w.gate)



# ---------------------------------------------------------------------------
# Block epilogue and channel-mixer inputs. The pages give no widths for the
# channel mixer; SSW_WORKLOADS use F = 2048, the SwiGLU hidden width of a
# 768-wide block at the usual 8/3 ratio, on the same 40x40 and 80x80 grids.
# Draws (all standard normal unless stated): output-gate rows z; RMSNorm
# weight 1 + 0.1 N(0,1); gate branch a; value branch u; depthwise weights
# N(0,1)/3 (fan-in 9); bias 0.1 N(0,1).

@dataclasses.dataclass(frozen=True)
class SswWorkload:
    name: str
    B: int
    grid_h: int
    grid_w: int
    F: int
    dtype: str = "f16"

    @property
    def T(self) -> int:
        return self.grid_h * self.grid_w


SSW_WORKLOADS = [
    SswWorkload("ssw_img640_40x40_f2048", B=1, grid_h=40, grid_w=40, F=2048),
    SswWorkload("ssw_img1280_80x80_f2048", B=1, grid_h=80, grid_w=80, F=2048),
]

GATE_EPS = 1e-6


def make_gate_inputs(B: int, T: int, H: int, dv: int, dtype, seed: int):
    """Output-gate rows z [B, T, H, dv] in `dtype` and the RMSNorm weight
    [dv] in float32."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((B, T, H, dv))
    w = 1.0 + 0.1 * rng.standard_normal(dv)
    return np.ascontiguousarray(z.astype(dtype)), np.ascontiguousarray(w.astype(np.float32))


def make_ssw_inputs(B: int, T: int, F: int, dtype, seed: int, with_bias: bool = True):
    """a, u [B, T, F] in `dtype`; weight [F, 3, 3] and bias [F] (or None) in
    float32."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((B, T, F))
    u = rng.standard_normal((B, T, F))
    w = rng.standard_normal((F, 3, 3)) / 3.0
    bias = 0.1 * rng.standard_normal(F) if with_bias else None
    cast = lambda x: np.ascontiguousarray(x.astype(dtype))
    return (cast(a), cast(u), np.ascontiguousarray(w.astype(np.float32)),
            None if bias is None else np.ascontiguousarray(bias.astype(np.float32)))

"""Pins for the epilogue oracles (output gate, Spatial SwiGLU): checks that tie
them to the hand-derived fixtures, to independent torch CPU library routines
(F.rms_norm, F.silu, grouped F.conv2d, all in float64) and to properties.

  gate -- callable (o, z, w, eps) -> y over [..., dv] rows
  ssw  -- callable (a, u, weight, bias, grid_h, grid_w) -> h, [B, T, F]
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

from pins import load_golden


def _t(x):
    return torch.from_numpy(np.asarray(x, np.float64))


def check_golden_gate(gate):
    for case in load_golden("epilogue_cases.json")["rmsnorm_gate"]:
        y = gate(np.array(case["o"]), np.array(case["z"]), np.array(case["w"]), case["eps"])
        np.testing.assert_allclose(y, case["y"], rtol=1e-12, atol=1e-12, err_msg=case["name"])


def check_gate_against_torch(gate, seed=30):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((2, 5, 3, 8))
    z = rng.standard_normal((2, 5, 3, 8)) * 3
    w = rng.standard_normal(8)
    for eps in (0.0, 1e-6, 0.5):
        ref = F.rms_norm(_t(o), (8,), weight=_t(w), eps=eps) * F.silu(_t(z))
        np.testing.assert_allclose(gate(o, z, w, eps), ref.numpy(), rtol=1e-12, atol=1e-12)


def check_gate_properties(gate, seed=31):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((4, 6))
    z = rng.standard_normal((4, 6))
    w = rng.standard_normal(6)
    y = gate(o, z, w, 0.0)
    np.testing.assert_allclose(gate(7.5 * o, z, w, 0.0), y, rtol=1e-12, atol=1e-12)  # scale-free
    assert np.all(gate(o, np.zeros_like(z), w, 0.0) == 0)                             # silu(0) = 0
    o2 = o.copy()
    o2[1] *= -3.0                                    # rows are independent
    y2 = gate(o2, z, w, 0.0)
    np.testing.assert_allclose(y2[[0, 2, 3]], y[[0, 2, 3]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(y2[1], -y[1], rtol=1e-12, atol=1e-12)


def check_golden_ssw(ssw):
    for case in load_golden("epilogue_cases.json")["spatial_swiglu"]:
        a = np.array(case["a"])[None]
        u = np.array(case["u"])[None]
        h = ssw(a, u, np.array(case["weight"], np.float64), np.array(case["bias"]),
                case["grid_h"], case["grid_w"])
        np.testing.assert_allclose(h[0], case["h"], rtol=1e-12, atol=1e-12, err_msg=case["name"])


def check_ssw_against_torch(ssw, seed=32):
    rng = np.random.default_rng(seed)
    for (B, gh, gw, Fc) in [(1, 5, 7, 3), (2, 4, 4, 6), (1, 1, 9, 2), (1, 8, 1, 2)]:
        a = rng.standard_normal((B, gh * gw, Fc)) * 2
        u = rng.standard_normal((B, gh * gw, Fc))
        w = rng.standard_normal((Fc, 3, 3))
        bias = rng.standard_normal(Fc)
        x = _t(u).reshape(B, gh, gw, Fc).permute(0, 3, 1, 2)
        conv = F.conv2d(x, _t(w)[:, None], _t(bias), padding=1, groups=Fc)
        ref = (F.silu(_t(a)) * conv.permute(0, 2, 3, 1).reshape(B, gh * gw, Fc)).numpy()
        np.testing.assert_allclose(ssw(a, u, w, bias, gh, gw), ref, rtol=1e-12, atol=1e-12)


def check_ssw_properties(ssw, seed=33):
    rng = np.random.default_rng(seed)
    gh, gw, Fc = 4, 5, 3
    a = rng.standard_normal((1, gh * gw, Fc))
    u = rng.standard_normal((1, gh * gw, Fc))
    delta = np.zeros((Fc, 3, 3))
    delta[:, 1, 1] = 1.0                                 # identity kernel
    sil = a / (1 + np.exp(-a))
    np.testing.assert_allclose(ssw(a, u, delta, None, gh, gw), sil * u, rtol=1e-12, atol=1e-12)
    ones = np.ones((Fc, 3, 3))                           # counts the in-grid taps
    big = np.full_like(a, 50.0)                          # silu(50) = 50 to double precision
    h = ssw(big, np.ones_like(u), ones, None, gh, gw)[0, :, 0] / 50.0
    y, x = np.divmod(np.arange(gh * gw), gw)
    taps = (3 - (y == 0) - (y == gh - 1)) * (3 - (x == 0) - (x == gw - 1))
    np.testing.assert_allclose(h, taps, rtol=1e-12)

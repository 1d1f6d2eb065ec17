"""GPU parity of the Spatial SwiGLU core against the float64 oracle.

Bar: max|h - h_ref| / max|h_ref| <= 5e-3, h_ref computed from exactly the
values the GPU receives (half inputs upcast, float weights).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, rel_err, say, to_dev
from recurrent_vision_token_gla_amd import gla
from recurrent_vision_token_gla_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gla.load()
    yield


def _run(a, u, w, bias, gh, gw):
    ta, tu, tw = to_dev(a, u, w)
    tb = None if bias is None else to_dev(bias)[0]
    h = gla.spatial_swiglu(ta, tu, tw, tb, gh, gw)
    torch.cuda.synchronize()
    return h.double().cpu().numpy()


@pytest.mark.parametrize("B,gh,gw,F", [(1, 1, 1, 8), (1, 3, 5, 8), (2, 9, 17, 40), (1, 8, 16, 64),
                                       (1, 17, 33, 72), (3, 10, 7, 136), (1, 40, 40, 256),
                                       (1, 1, 50, 16), (1, 50, 1, 16)])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_spatial_swiglu_shapes(B, gh, gw, F, dtype):
    a, u, w, bias = W.make_ssw_inputs(B, gh * gw, F, dtype, seed=500 + gh * gw + F)
    say(f"ssw B={B} grid={gh}x{gw} F={F} {np.dtype(dtype).name}")
    h = _run(a, u, w, bias, gh, gw)
    ref = oracle.spatial_swiglu(a, u, w, bias, gh, gw)
    assert rel_err(h, ref) <= TOL


def test_spatial_swiglu_no_bias_and_delta_kernel():
    gh, gw, F = 12, 20, 64
    a, u, w, _ = W.make_ssw_inputs(2, gh * gw, F, np.float16, seed=510, with_bias=False)
    h = _run(a, u, w, None, gh, gw)
    assert rel_err(h, oracle.spatial_swiglu(a, u, w, None, gh, gw)) <= TOL
    delta = np.zeros_like(w)
    delta[:, 1, 1] = 1.0
    h = _run(a, u, delta, None, gh, gw)
    assert rel_err(h, oracle.silu(a) * u.astype(np.float64)) <= TOL


@pytest.mark.parametrize("wi", [0, 1])
def test_spatial_swiglu_workloads(wi):
    w = W.SSW_WORKLOADS[wi]
    a, u, wt, bias = W.make_ssw_inputs(w.B, w.T, w.F, np.float16, seed=520 + wi)
    say(f"ssw workload {w.name}")
    h = _run(a, u, wt, bias, w.grid_h, w.grid_w)
    ref = oracle.spatial_swiglu(a, u, wt, bias, w.grid_h, w.grid_w)
    err = rel_err(h, ref)
    say(f"  rel_err={err:.2e}")
    assert err <= TOL


def test_spatial_swiglu_argument_errors():
    a = torch.zeros((1, 16, 12), dtype=torch.float16, device="cuda")
    with pytest.raises(gla.GLAError):  # F not a multiple of 8
        gla.spatial_swiglu(a, a.clone(), torch.zeros((12, 3, 3), device="cuda"), None, 4, 4)
    b = torch.zeros((1, 16, 16), dtype=torch.float16, device="cuda")
    with pytest.raises(gla.GLAError):  # output aliases an input
        gla.spatial_swiglu(b, b.clone(), torch.zeros((16, 3, 3), device="cuda"), None, 4, 4, out=b)


def test_spatial_swiglu_wide_grid_grid_per_tile_kernel():
    """A grid so wide that ten rows of the value tensor pass 2^31 bytes takes
    the grid-per-tile kernel (the persistent one addresses a unit's halo
    rows with 32-bit offsets). Checked on column windows: the oracle runs on
    each window plus its neighbour columns, and the window's tokens, whose
    3x3 neighbourhoods lie inside, are compared."""
    gh, gw, F = 1, 1 << 17, 1024
    assert 10 * gw * F * 2 >= 1 << 31
    a, u, w, bias = W.make_ssw_inputs(1, gh * gw, F, np.float16, seed=530)
    h = _run(a, u, w, bias, gh, gw)
    worst = 0.0
    for x0 in (0, 5000, gw // 2 + 3, gw - 40):
        lo, hi = max(0, x0 - 1), min(gw, x0 + 40 + 1)
        ref = oracle.spatial_swiglu(a[:, lo:hi], u[:, lo:hi], w, bias, gh, hi - lo)
        s = slice(x0 - lo, x0 - lo + 40)
        err = rel_err(h[:, x0:x0 + 40], ref[:, s])
        say(f"ssw wide grid window x0={x0}: rel_err={err:.3e}")
        worst = max(worst, err)
    assert worst <= TOL

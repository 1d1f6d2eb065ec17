"""GPU parity of the forward with the fused output gate,
y = RMSNorm(o) * w * silu(z), against the float64 oracle (forward, then
oracle.rmsnorm_gate), on both schedules.

Bar: max|y - y_ref| / max|y_ref| <= 5e-3.
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


def _ref(x, z, w, gh, gw, dirs, s0=None):
    o = oracle.gla_forward(*x, gh, gw, dirs, s0=s0)
    return oracle.rmsnorm_gate(o, z, w, W.GATE_EPS)


def _run(x, z, w, gh, gw, dirs, chunk, s0=None):
    tq, tk, tv, tg, tz = to_dev(*x, z)
    tw = to_dev(w)[0]
    ts0 = None if s0 is None else to_dev(s0)[0]
    B, T, H, dk = x[0].shape
    dv = x[2].shape[-1]
    ws = gla.alloc_workspace(B, H, gh, gw, dk, dv, chunk)
    y = gla.fwd_gated(tq, tk, tv, tg, tz, tw, W.GATE_EPS, gh, gw, list(dirs), chunk=chunk,
                      s0=ts0, workspace=ws)
    torch.cuda.synchronize()
    return y.double().cpu().numpy()


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_gated_shapes(dk, dv, chunk, dtype):
    gh, gw, B, H = 9, 17, 2, 2
    x = W.make_inputs(B, gh * gw, H, dk, dv, dtype, seed=600 + dk + dv + chunk)
    z, w = W.make_gate_inputs(B, gh * gw, H, dv, dtype, seed=601 + dk)
    say(f"gated dk={dk} dv={dv} chunk={chunk} {np.dtype(dtype).name}")
    y = _run(x, z, w, gh, gw, [1, 2], chunk)
    assert rel_err(y, _ref(x, z, w, gh, gw, [1, 2])) <= TOL


@pytest.mark.parametrize("wi", [1, 2])
def test_gated_workload_shapes_both_schedules(wi):
    """640^2 takes the single pass and 1280^2 the three phases."""
    wl = W.WORKLOADS[wi]
    x = W.workload_inputs(wl, 0)
    z, w = W.make_gate_inputs(wl.B, wl.T, wl.H, wl.dv, np.float16, seed=610 + wi)
    dirs = wl.directions(2)
    say(f"gated {wl.name} schedule {gla.auto_schedule(wl.B, wl.H, wl.grid_h, wl.grid_w, 64, 64, 64)}")
    y = _run(x, z, w, wl.grid_h, wl.grid_w, dirs, wl.chunk)
    err = rel_err(y, _ref(x, z, w, wl.grid_h, wl.grid_w, dirs))
    say(f"  rel_err={err:.2e}")
    assert err <= TOL


def test_gated_with_carried_state():
    gh, gw, B, H = 16, 20, 1, 3
    x = W.make_inputs(B, gh * gw, H, 64, 64, np.float16, seed=620)
    z, w = W.make_gate_inputs(B, gh * gw, H, 64, np.float16, seed=621)
    s0 = np.random.default_rng(6).standard_normal((B, H, 64, 64)).astype(np.float32)
    y = _run(x, z, w, gh, gw, [3], 64, s0=s0)
    assert rel_err(y, _ref(x, z, w, gh, gw, [3], s0=s0)) <= TOL


def test_gated_equals_ungated_then_gate():
    """The fused epilogue equals the plain forward followed by the gate formula
    evaluated on the GPU output (same o, rounded once)."""
    gh, gw, B, H = 12, 12, 2, 2
    x = W.make_inputs(B, gh * gw, H, 64, 64, np.float16, seed=630)
    z, w = W.make_gate_inputs(B, gh * gw, H, 64, np.float16, seed=631)
    tq, tk, tv, tg = to_dev(*x)
    o = gla.fwd(tq, tk, tv, tg, gh, gw, [0, 1], 64).double().cpu().numpy()
    y = _run(x, z, w, gh, gw, [0, 1], 64)
    assert rel_err(y, oracle.rmsnorm_gate(o, z, w, W.GATE_EPS)) <= 2e-3

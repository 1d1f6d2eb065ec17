"""GPU parity at the edges of the half range, and the workspace contract.

Inputs here are built so that the exact outputs stay well inside the half
range while intermediate quantities do not: score entries of q.k beyond
65504, diagonal-block factors that exceed the half range when the decay of
a 16-token block is concentrated in one half of it, and boundary states that
grow past 65504 under biased, correlated k and v with almost no decay. Each
case is checked against the float64 oracle on exactly the half values the
GPU receives, on both schedules.

Bar: max|o - o_ref| / max|o_ref| <= 5e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, rel_err, say, to_dev
from recurrent_vision_token_gla_amd import gla
from recurrent_vision_token_gla_amd import workloads as W

pytestmark = pytest.mark.gpu
SCHEDS = {"single": gla.SCHED_SINGLE_PASS, "three": gla.SCHED_THREE_PHASE,
          "runs": gla.SCHED_RUNS}  # runs: chunk 64 only


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gla.load()
    yield


def _half(x):
    return np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float16))


def _run(x, gh, gw, dirs, chunk, sched, s0=None):
    tq, tk, tv, tg = to_dev(*x)
    ts0 = None if s0 is None else to_dev(s0)[0]
    o, sT = gla.fwd_state(tq, tk, tv, tg, gh, gw, list(dirs), chunk=chunk, s0=ts0, schedule=sched)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), sT.double().cpu().numpy()


def _check(x, gh, gw, dirs, chunk, sched, s0=None):
    o, sT = _run(x, gh, gw, dirs, chunk, sched, s0)
    ro, rs = oracle.gla_forward(*x, gh, gw, dirs, s0=s0, return_state=True)
    eo, es = rel_err(o, ro), rel_err(sT, rs)
    say(f"  max|o_ref| {np.max(np.abs(ro)):.3g}  max|S_T| {np.max(np.abs(rs)):.3g}  "
        f"o err {eo:.2e}  S_T err {es:.2e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(sT))
    assert eo <= TOL and es <= TOL


def concentrated_decay(B, T, H, dk, per_token=1.0):
    """gk that decays by 2^-per_token on tokens 8..15 of every 16-token block
    of the scan (and not at all on tokens 0..7): the block's decay range is
    8 * per_token in log2, all of it in the second half."""
    t = np.arange(T) % 16
    g = np.where(t >= 8, -np.log(2.0) * per_token, 0.0)
    return np.broadcast_to(g[None, :, None, None], (B, T, H, dk)).copy()


@pytest.mark.parametrize("sched", sorted(SCHEDS))
@pytest.mark.parametrize("qk_scale", [300.0, 1000.0])
def test_large_q_k_with_concentrated_decay(sched, qk_scale):
    """|q|, |k| of several hundred to a thousand with the decay of each block
    in its second half: the diagonal factors q 2^(s_i - s_7), k 2^(s_7 - s_j)
    reach |k| 2^8, and the scores q.k reach about 1e7; v is small so that the
    outputs stay near 1e3."""
    gh, gw, B, H, dk, dv = 16, 20, 2, 2, 64, 64
    T = gh * gw
    rng = np.random.default_rng(int(qk_scale))
    # the scan order is the raster order for direction 0: the decay pattern
    # follows the scan positions
    x = (_half(rng.standard_normal((B, T, H, dk)) * qk_scale),
         _half(rng.standard_normal((B, T, H, dk)) * qk_scale),
         _half(rng.standard_normal((B, T, H, dv)) * 1e-4),
         _half(concentrated_decay(B, T, H, dk)))
    say(f"{sched} |q|,|k| ~ {qk_scale}")
    _check(x, gh, gw, [0, 0], 64, SCHEDS[sched])


@pytest.mark.parametrize("sched", ["single", "three"])  # chunk 32 below: no runs schedule
@pytest.mark.parametrize("per_token", [0.5, 2.0, 20.0])
def test_decay_ranges_with_large_keys(sched, per_token):
    """The same concentrated decay at block ranges of 4, 16 and 160 (log2),
    with |k| about 200 and moderate q, v: every diagonal arithmetic."""
    gh, gw, B, H, dk, dv = 12, 16, 1, 3, 64, 32
    T = gh * gw
    rng = np.random.default_rng(11)
    x = (_half(rng.standard_normal((B, T, H, dk)) * 0.125),
         _half(rng.standard_normal((B, T, H, dk)) * 200.0),
         _half(rng.standard_normal((B, T, H, dv))),
         _half(concentrated_decay(B, T, H, dk, per_token)))
    say(f"{sched} per-token decay 2^-{per_token} on half of each block")
    _check(x, gh, gw, [0], 32, SCHEDS[sched])


@pytest.mark.parametrize("sched", sorted(SCHEDS))
def test_states_beyond_the_half_range(sched):
    """Biased, correlated k and v (both about 4) with almost no decay on an
    80x80 grid: the boundary states grow to about 1e5, beyond 65504, while q
    is small enough that the outputs stay near 1e3."""
    gh, gw, B, H, dk, dv = 80, 80, 1, 2, 64, 64
    T = gh * gw
    rng = np.random.default_rng(21)
    common = rng.standard_normal((B, T, H, 1))
    x = (_half(rng.standard_normal((B, T, H, dk)) * 1e-3),
         _half(4.0 + 0.5 * common + 0.25 * rng.standard_normal((B, T, H, dk))),
         _half(4.0 + 0.5 * common + 0.25 * rng.standard_normal((B, T, H, dv))),
         _half(np.full((B, T, H, dk), -1e-5)))
    say(f"{sched} 80x80, k, v ~ 4, decay 1e-5")
    _check(x, gh, gw, [2], 64, SCHEDS[sched])


@pytest.mark.parametrize("sched", sorted(SCHEDS))
def test_large_carried_state(sched):
    """A carried state of about 1e6 (float) with weak decay: the state rows
    are scaled in half through the whole chain; q is small enough that the
    outputs stay near 1e4."""
    gh, gw, B, H, dk, dv = 40, 40, 1, 2, 64, 64
    q, k, v, g = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=31,
                               gate_override=np.float16(-2e-4))
    x = (_half(q.astype(np.float64) * 2e-3), k, v, g)
    s0 = (np.random.default_rng(3).standard_normal((B, H, dk, dv)) * 1e6).astype(np.float32)
    say(f"{sched} |s0| ~ 1e6")
    _check(x, gh, gw, [1], 64, SCHEDS[sched], s0=s0)


def test_unprepared_workspace_of_any_contents():
    """A workspace that gla_workspace_init has not prepared, filled with 0xFF
    (every control word set): gla_fwd runs the three phases and is correct;
    the single pass is refused."""
    w = W.WORKLOADS[1]
    x = W.workload_inputs(w, 0)
    tq, tk, tv, tg = to_dev(*x)
    ws = gla.alloc_workspace(w.B, w.H, w.grid_h, w.grid_w, w.dk, w.dv, w.chunk, prepare=False)
    ws.fill_(0xFF)
    assert not gla.is_prepared(ws)
    o = gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, w.directions(0), w.chunk, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.gla_forward(*x, w.grid_h, w.grid_w, w.directions(0))
    assert rel_err(o.double().cpu().numpy(), ref) <= TOL
    with pytest.raises(gla.GLAError) as e:
        gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, w.directions(0), w.chunk, workspace=ws,
                schedule=gla.SCHED_SINGLE_PASS)
    assert e.value.status == gla.E_UNPREPARED
    # once prepared, the single pass runs on it
    gla.workspace_init(ws)
    assert gla.is_prepared(ws)
    o1 = gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, w.directions(0), w.chunk, workspace=ws,
                 schedule=gla.SCHED_SINGLE_PASS)
    torch.cuda.synchronize()
    assert rel_err(o1.double().cpu().numpy(), ref) <= TOL
    assert gla.workspace_error(ws) == 0
    gla.workspace_release(ws)
    assert not gla.is_prepared(ws)


@pytest.mark.parametrize("gh,gw,chunk", [(80, 80, 16), (80, 80, 64), (40, 40, 64)])
def test_in_place_state_update_on_long_chains(gh, gw, chunk):
    """s_final == s0 on chains of 25 to 400 chunks (many single-pass
    segments): the call takes the three phases and equals the oracle; the
    single pass refuses it."""
    B, H, dk, dv = 1, 3, 64, 64
    x = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=40 + gh + chunk)
    s0 = (np.random.default_rng(9).standard_normal((B, H, dk, dv)) * 3).astype(np.float32)
    tq, tk, tv, tg = to_dev(*x)
    st = to_dev(s0)[0]
    o, sT = gla.fwd_state(tq, tk, tv, tg, gh, gw, [3], chunk=chunk, s0=st, s_final=st)
    torch.cuda.synchronize()
    assert sT.data_ptr() == st.data_ptr()
    ro, rs = oracle.gla_forward(*x, gh, gw, [3], s0=s0, return_state=True)
    assert rel_err(o.double().cpu().numpy(), ro) <= TOL
    assert rel_err(st.double().cpu().numpy(), rs) <= TOL
    with pytest.raises(gla.GLAError) as e:
        gla.fwd_state(tq, tk, tv, tg, gh, gw, [3], chunk=chunk, s0=st, s_final=st,
                      schedule=gla.SCHED_SINGLE_PASS)
    assert e.value.status == gla.E_UNSUPPORTED


@pytest.mark.parametrize("call", [1, 2, 3])
def test_stack_right_to_left_top_to_bottom_bottom_to_top_full(call):
    """Calls 1, 2 and 3 of the 12-block stack (R2L, T2B, B2T; 4 x 80x80, 16
    heads, mixed gates) compared in full against the oracle."""
    w = W.WORKLOADS[4]
    x = W.workload_inputs(w, call)
    dirs = w.directions(call)
    say(f"stack call {call} dirs={dirs}")
    tq, tk, tv, tg = to_dev(*x)
    o = gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, dirs, w.chunk)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    del tq, tk, tv, tg
    ref = oracle.gla_forward(*x, w.grid_h, w.grid_w, dirs)
    err = rel_err(o, ref)
    say(f"  rel_err={err:.3e}")
    assert np.all(np.isfinite(o)) and err <= TOL

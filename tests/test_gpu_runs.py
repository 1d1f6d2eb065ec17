"""GPU parity of the runs schedule (one workgroup per run of 64-token chunks,
four for half inputs and three for float, one group of four waves per chunk;
decoupled look-back between runs) against the float64 oracle.

Bar: max|x - x_ref| / max|x_ref| <= 5e-3 for outputs and final states.
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


def _run(x, gh, gw, dirs, s0=None, ws=None):
    tq, tk, tv, tg = to_dev(*x)
    ts0 = None if s0 is None else to_dev(s0)[0]
    o, sT = gla.fwd_state(tq, tk, tv, tg, gh, gw, list(dirs), chunk=64, s0=ts0,
                          schedule=gla.SCHED_RUNS, workspace=ws)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), sT.double().cpu().numpy()


def _check(x, gh, gw, dirs, s0=None, ws=None):
    o, sT = _run(x, gh, gw, dirs, s0, ws)
    ro, rs = oracle.gla_forward(*x, gh, gw, dirs, s0=s0, return_state=True)
    eo, es = rel_err(o, ro), rel_err(sT, rs)
    say(f"  o err {eo:.2e}  S_T err {es:.2e}")
    assert np.all(np.isfinite(o)) and eo <= TOL and es <= TOL
    return o


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("gh,gw", [(5, 7), (8, 8), (9, 17), (16, 17), (21, 20), (40, 40)])
def test_runs_shapes_chain_lengths_and_tails(dk, dv, gh, gw):
    """Chains of 1 to 25 chunks: a single run, runs shorter than four
    chunks, ragged last chunks."""
    B, H = 2, 2
    x = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=600 + dk + dv + gh * gw)
    say(f"runs dk={dk} dv={dv} grid={gh}x{gw} N={-(-gh * gw // 64)}")
    _check(x, gh, gw, [1, 2])


@pytest.mark.parametrize("wi", [1, 2, 3])
def test_runs_on_workloads(wi):
    w = W.WORKLOADS[wi]
    x = W.workload_inputs(w, 0)
    say(f"runs {w.name}")
    _check(x, w.grid_h, w.grid_w, w.directions(0))


def test_runs_stack_call_mixed_gates():
    w = W.WORKLOADS[4]
    for call in (0, 3):
        x = W.workload_inputs(w, call)
        say(f"runs {w.name} call {call}")
        _check(x, w.grid_h, w.grid_w, w.directions(call))


@pytest.mark.parametrize("gh,gw", [(8, 8), (40, 40), (80, 80), (128, 128)])
def test_runs_carried_state(gh, gw):
    B, H = 1, 3
    x = W.make_inputs(B, gh * gw, H, 64, 64, np.float16, seed=610 + gh)
    s0 = (np.random.default_rng(6).standard_normal((B, H, 64, 64)) * 3).astype(np.float32)
    say(f"runs with s0 grid={gh}x{gw}")
    _check(x, gh, gw, [3], s0=s0)


def test_runs_fp32_inputs():
    x = W.make_inputs(2, 20 * 20, 3, 64, 64, np.float32, seed=620)
    _check(x, 20, 20, [0, 1])


def test_runs_strong_and_mixed_decay():
    x = W.make_inputs(2, 32 * 32, 3, 64, 64, np.float16, seed=630, gate="mixed")
    _check(x, 32, 32, [2, 3])
    g = np.full((1, 24 * 24, 2, 64), -1e4, np.float16)
    q, k, v, _ = W.make_inputs(1, 24 * 24, 2, 64, 64, np.float16, seed=631)
    _check((q, k, v, g), 24, 24, [0])


def test_runs_states_beyond_the_half_range():
    gh, gw, B, H = 80, 80, 1, 2
    T = gh * gw
    rng = np.random.default_rng(21)
    common = rng.standard_normal((B, T, H, 1))
    h = lambda a: np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float16))
    x = (h(rng.standard_normal((B, T, H, 64)) * 1e-3),
         h(4.0 + 0.5 * common + 0.25 * rng.standard_normal((B, T, H, 64))),
         h(4.0 + 0.5 * common + 0.25 * rng.standard_normal((B, T, H, 64))),
         h(np.full((B, T, H, 64), -1e-5)))
    _check(x, gh, gw, [2])


def test_runs_many_chains_and_long_chains():
    """More runs than the GPU holds at once (run-major dispatch, look-backs
    across waves of workgroups), and a 256-chunk chain."""
    x = W.make_inputs(16, 24 * 24, 16, 64, 32, np.float16, seed=640)
    dirs = [b % 4 for b in range(16)]
    _check(x, 24, 24, dirs)
    x = W.make_inputs(1, 128 * 128, 2, 32, 64, np.float16, seed=641)
    _check(x, 128, 128, [1])


def test_runs_control_words_clean_and_replays_exact():
    gh, gw, B, H = 40, 40, 2, 6
    x = W.make_inputs(B, gh * gw, H, 64, 64, np.float16, seed=650)
    tq, tk, tv, tg = to_dev(*x)
    ws = gla.alloc_workspace(B, H, gh, gw, 64, 64, 64)
    eager = gla.fwd(tq, tk, tv, tg, gh, gw, [0, 3], workspace=ws, schedule=gla.SCHED_RUNS)
    torch.cuda.synchronize()
    eager = eager.clone()
    assert not ws[:gla.CTRL_BYTES].any().item()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gla.fwd(tq, tk, tv, tg, gh, gw, [0, 3], out=out, workspace=ws, stream=s,
                schedule=gla.SCHED_RUNS)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            gla.fwd(tq, tk, tv, tg, gh, gw, [0, 3], out=out, workspace=ws, stream=s,
                    schedule=gla.SCHED_RUNS)
    torch.cuda.synchronize()
    for i in range(5):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        _ = (tq.float() * 2).sum().item()
    assert not ws[:gla.CTRL_BYTES].any().item()
    assert gla.workspace_error(ws) == 0
    assert rel_err(eager.double().cpu().numpy(), oracle.gla_forward(*x, gh, gw, [0, 3])) <= TOL

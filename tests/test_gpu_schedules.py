"""GPU parity of both kernel schedules (single pass and three phases) against
the CPU oracle, their agreement, and the single pass's control words.

Bar: max|o - o_ref| / max|o_ref| <= 5e-3 against the float64 recurrence.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, rel_err, say, to_dev
from recurrent_vision_token_gla_amd import gla
from recurrent_vision_token_gla_amd import workloads as W

pytestmark = pytest.mark.gpu
SCHEDS = {"single": gla.SCHED_SINGLE_PASS, "three": gla.SCHED_THREE_PHASE}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gla.load()
    yield


def _run(x, gh, gw, dirs, chunk, sched, s0=None, ws=None):
    tq, tk, tv, tg = to_dev(*x)
    ts0 = None if s0 is None else to_dev(s0)[0]
    o, sT = gla.fwd_state(tq, tk, tv, tg, gh, gw, list(dirs), chunk=chunk, s0=ts0,
                          schedule=sched, workspace=ws)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), sT.double().cpu().numpy()


@pytest.mark.parametrize("sched", sorted(SCHEDS))
@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_schedule_shapes_and_ragged_tail(sched, dk, dv, chunk):
    gh, gw, B, H = 9, 17, 2, 2  # 153 tokens: several chunks and a ragged tail
    x = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=400 + dk + dv + chunk)
    say(f"{sched} dk={dk} dv={dv} chunk={chunk}")
    o, _ = _run(x, gh, gw, [0, 3], chunk, SCHEDS[sched])
    assert rel_err(o, oracle.gla_forward(*x, gh, gw, [0, 3])) <= TOL


@pytest.mark.parametrize("H", [8, 10])
@pytest.mark.parametrize("dv", [32, 64])
def test_single_pass_value_split_both_sides(H, dv):
    # 40x40 grid: H 8 is 200 chunk-heads (dv = 64 splits its value columns
    # over two workgroups per chunk-head), H 10 is 250 (no split); with a
    # carried state in and out, against the oracle
    g, B = 40, 1
    x = W.make_inputs(B, g * g, H, 64, dv, np.float16, seed=950 + H + dv)
    s0 = np.random.default_rng(7).standard_normal((B, H, 64, dv)).astype(np.float32)
    dirs = [2]
    say(f"single pass H={H} dv={dv}")
    o, sT = _run(x, g, g, dirs, 64, gla.SCHED_SINGLE_PASS, s0=s0)
    ref, refT = oracle.gla_forward(*x, g, g, dirs, s0=s0, return_state=True)
    e, eT = rel_err(o, ref), rel_err(sT, refT)
    say(f"  rel_err={e:.3e} state {eT:.3e}")
    assert e <= TOL and eT <= TOL


@pytest.mark.parametrize("B,H,g", [(8, 12, 64), (8, 16, 80), (4, 16, 96)])
def test_auto_single_pass_on_large_grids(B, H, g):
    # grids where gla_fwd takes the single pass with thousands of workgroups
    # in flight (chains of 64, 100 and 144 chunks): all four directions in one
    # launch, every (b, h) against the oracle
    assert gla.auto_schedule(B, H, g, g, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    x = W.make_inputs(B, g * g, H, 64, 64, np.float16, seed=900 + g)
    dirs = [b % 4 for b in range(B)]
    say(f"auto single pass B={B} H={H} grid {g}x{g}")
    tq, tk, tv, tg = to_dev(*x)
    o = gla.fwd(tq, tk, tv, tg, g, g, dirs, 64)
    torch.cuda.synchronize()
    err = rel_err(o.double().cpu().numpy(), oracle.gla_forward(*x, g, g, dirs))
    say(f"  rel_err={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("wi", [0, 1, 2])
def test_schedules_agree_on_workloads(wi):
    w = W.WORKLOADS[wi]
    for call in range(4 if wi else 1):
        x = W.workload_inputs(w, call)
        dirs = w.directions(call)
        say(f"workload {w.name} call {call}")
        o1, _ = _run(x, w.grid_h, w.grid_w, dirs, w.chunk, gla.SCHED_SINGLE_PASS)
        o3, _ = _run(x, w.grid_h, w.grid_w, dirs, w.chunk, gla.SCHED_THREE_PHASE)
        ref = oracle.gla_forward(*x, w.grid_h, w.grid_w, dirs)
        e1, e3 = rel_err(o1, ref), rel_err(o3, ref)
        say(f"  single {e1:.2e}  three {e3:.2e}  between {rel_err(o1, o3):.2e}")
        assert e1 <= TOL and e3 <= TOL


@pytest.mark.parametrize("gh,gw,chunk", [(4, 4, 16), (8, 8, 16), (40, 40, 64), (33, 31, 16),
                                         (80, 80, 64), (128, 128, 16)])
def test_single_pass_chains_and_carried_state(gh, gw, chunk):
    """N = 1, 4, 25, 64, 100 and 1024 chunks: one segment, several, the
    largest segment count; with a carried state in and out."""
    B, H, dk, dv = 1, 2, 64, 64
    x = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=410 + gh + chunk)
    s0 = (np.random.default_rng(5).standard_normal((B, H, dk, dv)) * 2).astype(np.float32)
    say(f"single pass grid={gh}x{gw} chunk={chunk} N={-(-gh * gw // chunk)}")
    o, sT = _run(x, gh, gw, [2], chunk, gla.SCHED_SINGLE_PASS, s0=s0)
    ro, rs = oracle.gla_forward(*x, gh, gw, [2], s0=s0, return_state=True)
    eo, es = rel_err(o, ro), rel_err(sT, rs)
    say(f"  o err {eo:.2e}  S_T err {es:.2e}")
    assert eo <= TOL and es <= TOL


def test_single_pass_strong_and_mixed_decay():
    w = W.WORKLOADS[4]
    gh, gw = 24, 24
    x = W.make_inputs(2, gh * gw, 3, 64, 64, np.float16, seed=420, gate="mixed")
    o, _ = _run(x, gh, gw, [1, 3], 64, gla.SCHED_SINGLE_PASS)
    assert rel_err(o, oracle.gla_forward(*x, gh, gw, [1, 3])) <= TOL
    assert w.gate == "mixed"


def test_control_words_stay_clean_across_sizes_and_calls():
    """One workspace, many single-pass calls of different sizes: the control
    words end every call at zero and the error word stays clear."""
    big = gla.alloc_workspace(2, 6, 80, 80, 64, 64, 16)
    for (B, H, gh, gw, C) in [(1, 6, 40, 40, 64), (2, 6, 80, 80, 16), (1, 1, 3, 3, 16),
                              (2, 3, 25, 26, 32), (1, 6, 40, 40, 64)]:
        x = W.make_inputs(B, gh * gw, H, 64, 64, np.float16, seed=430 + B + gh)
        dirs = [0] * B
        o, _ = _run(x, gh, gw, dirs, C, gla.SCHED_SINGLE_PASS, ws=big)
        assert rel_err(o, oracle.gla_forward(*x, gh, gw, dirs)) <= TOL
        ctrl = big[:gla.CTRL_BYTES].cpu().numpy()
        assert not ctrl.any(), np.flatnonzero(ctrl)[:8]
    assert gla.workspace_error(big) == 0


def test_batch_beyond_one_launch_single_pass():
    gh, gw, B, H = 4, 5, 1030, 1  # two launches: 1024 + 6 batch elements
    x = W.make_inputs(B, gh * gw, H, 32, 32, np.float16, seed=440)
    dirs = [b % 4 for b in range(B)]
    o, _ = _run(x, gh, gw, dirs, 16, gla.SCHED_SINGLE_PASS)
    assert rel_err(o, oracle.gla_forward(*x, gh, gw, dirs)) <= TOL


def test_single_pass_graph_replays_match_eager():
    """A captured single-pass call replayed several times, with eager work
    between replays: every replay equals the eager result exactly."""
    gh, gw, B, H = 40, 40, 1, 6
    x = W.make_inputs(B, gh * gw, H, 64, 64, np.float16, seed=450)
    tq, tk, tv, tg = to_dev(*x)
    ws = gla.alloc_workspace(B, H, gh, gw, 64, 64, 64)
    eager = gla.fwd(tq, tk, tv, tg, gh, gw, [1], workspace=ws, schedule=gla.SCHED_SINGLE_PASS)
    torch.cuda.synchronize()
    eager = eager.clone()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gla.fwd(tq, tk, tv, tg, gh, gw, [1], out=out, workspace=ws, stream=s,
                schedule=gla.SCHED_SINGLE_PASS)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            gla.fwd(tq, tk, tv, tg, gh, gw, [1], out=out, workspace=ws, stream=s,
                    schedule=gla.SCHED_SINGLE_PASS)
    torch.cuda.synchronize()
    for i in range(5):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        _ = (tq.float() * 2).sum().item()  # unrelated eager work between replays
    assert not ws[:gla.CTRL_BYTES].any().item()
    assert rel_err(eager.double().cpu().numpy(), oracle.gla_forward(*x, gh, gw, [1])) <= TOL


def test_single_pass_deterministic():
    gh, gw = 40, 40
    x = W.make_inputs(1, gh * gw, 6, 64, 64, np.float16, seed=460)
    a, _ = _run(x, gh, gw, [3], 64, gla.SCHED_SINGLE_PASS)
    b, _ = _run(x, gh, gw, [3], 64, gla.SCHED_SINGLE_PASS)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("sched", sorted(SCHEDS))
def test_longest_single_pass_chain(sched):
    """4,096 chunks in one chain (256 x 256 grid, chunk 16): the single pass's
    widest waits (64 segments of 64 chunks) and the scan's longest segments
    (256 chunks each, re-read past the register block), with a carried
    state."""
    gh, gw, chunk, B, H, dk, dv = 256, 256, 16, 1, 1, 32, 32
    x = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=470)
    s0 = np.random.default_rng(7).standard_normal((B, H, dk, dv)).astype(np.float32)
    say(f"{sched} grid={gh}x{gw} chunk={chunk} N={gh * gw // chunk}")
    o, sT = _run(x, gh, gw, [3], chunk, SCHEDS[sched], s0=s0)
    ro, rs = oracle.gla_forward(*x, gh, gw, [3], s0=s0, return_state=True)
    eo, es = rel_err(o, ro), rel_err(sT, rs)
    say(f"  o err {eo:.2e}  S_T err {es:.2e}")
    assert eo <= TOL and es <= TOL

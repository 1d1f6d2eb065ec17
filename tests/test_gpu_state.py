"""GPU parity of the carried-state forward (initial state in, final state
out) and of the boundary scan on long chunk chains, against the CPU oracle.

Bar: outputs and final states within 5e-3 of the float64 recurrence,
max|x - x_ref| / max|x_ref|.
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


def _state(rng, B, H, dk, dv, scale=1.0):
    return (rng.standard_normal((B, H, dk, dv)) * scale).astype(np.float32)


def _run_state(q, k, v, g, gh, gw, dirs, chunk, s0, in_place=False):
    tq, tk, tv, tg = to_dev(q, k, v, g)
    B, _, H, dk = q.shape
    dv = v.shape[-1]
    ts0 = None if s0 is None else to_dev(s0)[0]
    sf = ts0 if in_place else None
    o, sT = gla.fwd_state(tq, tk, tv, tg, gh, gw, list(dirs), chunk=chunk, s0=ts0, s_final=sf)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), sT.double().cpu().numpy()


@pytest.mark.parametrize("dk,dv,chunk", [(64, 64, 64), (32, 64, 64), (32, 32, 16), (64, 32, 32)])
def test_state_in_and_out_match_oracle(dk, dv, chunk):
    gh, gw, B, H = 20, 23, 2, 3  # 460 tokens, ragged tail for every chunk size
    q, k, v, g = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=300 + dk + dv + chunk)
    s0 = _state(np.random.default_rng(1), B, H, dk, dv, 4.0)
    dirs = [1, 2]
    say(f"state dk={dk} dv={dv} chunk={chunk}")
    o, sT = _run_state(q, k, v, g, gh, gw, dirs, chunk, s0)
    ro, rs = oracle.gla_forward(q, k, v, g, gh, gw, dirs, s0=s0, return_state=True)
    eo, es = rel_err(o, ro), rel_err(sT, rs)
    say(f"  o err {eo:.2e}  S_T err {es:.2e}")
    assert eo <= TOL and es <= TOL


def test_zero_state_and_null_state_agree_with_fwd():
    gh, gw, B, H = 16, 16, 1, 2
    q, k, v, g = W.make_inputs(B, gh * gw, H, 64, 64, np.float16, seed=310)
    o_null, sT = _run_state(q, k, v, g, gh, gw, [3], 64, None)
    o_zero, sT0 = _run_state(q, k, v, g, gh, gw, [3], 64, np.zeros((B, H, 64, 64), np.float32))
    tq, tk, tv, tg = to_dev(q, k, v, g)
    o_fwd = gla.fwd(tq, tk, tv, tg, gh, gw, [3], chunk=64).double().cpu().numpy()
    assert np.array_equal(o_null, o_fwd) and np.array_equal(o_zero, o_fwd)
    assert np.array_equal(sT, sT0)
    _, rs = oracle.gla_forward(q, k, v, g, gh, gw, [3], return_state=True)
    assert rel_err(sT, rs) <= TOL


def test_state_in_place_update():
    gh, gw, B, H = 12, 9, 2, 2
    q, k, v, g = W.make_inputs(B, gh * gw, H, 32, 64, np.float16, seed=311)
    s0 = _state(np.random.default_rng(2), B, H, 32, 64)
    o, sT = _run_state(q, k, v, g, gh, gw, [0, 2], 32, s0, in_place=True)
    ro, rs = oracle.gla_forward(q, k, v, g, gh, gw, [0, 2], s0=s0, return_state=True)
    assert rel_err(o, ro) <= TOL and rel_err(sT, rs) <= TOL


def test_two_frames_carry_equals_one_long_scan():
    """Frame 2 run from frame 1's final state equals the second half of one
    scan over both frames' token sequences."""
    gh, gw, B, H, dk, dv = 24, 24, 1, 4, 64, 64
    T = gh * gw
    x1 = W.make_inputs(B, T, H, dk, dv, np.float16, seed=320)
    x2 = W.make_inputs(B, T, H, dk, dv, np.float16, seed=321)
    dirs = [2]
    tq, tk, tv, tg = to_dev(*x1)
    _, s1 = gla.fwd_state(tq, tk, tv, tg, gh, gw, dirs, chunk=64)
    tq, tk, tv, tg = to_dev(*x2)
    o2, s2 = gla.fwd_state(tq, tk, tv, tg, gh, gw, dirs, chunk=64, s0=s1)
    torch.cuda.synchronize()
    scan = lambda x: oracle.to_scan(x, gh, gw, dirs)
    both = [np.concatenate([scan(a), scan(b)], axis=1) for a, b in zip(x1, x2)]
    ro, rs = oracle.recurrence_c(*both, return_state=True)
    ro2 = oracle.to_raster(ro[:, T:], gh, gw, dirs)
    e_o, e_s = rel_err(o2.double().cpu().numpy(), ro2), rel_err(s2.double().cpu().numpy(), rs)
    say(f"two frames: o err {e_o:.2e}  S err {e_s:.2e}")
    assert e_o <= TOL and e_s <= TOL


@pytest.mark.parametrize("gh,gw,chunk", [(16, 16, 16), (41, 40, 16), (128, 128, 16),
                                         (100, 99, 32), (128, 128, 64)])
def test_long_chunk_chains(gh, gw, chunk):
    """Chains of 16 up to 1024 chunks: one chunk per scan segment, several,
    and segments longer than the register block."""
    B, H, dk, dv = 1, 2, 32, 64
    q, k, v, g = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=330 + gh + chunk)
    s0 = _state(np.random.default_rng(3), B, H, dk, dv)
    say(f"chain grid={gh}x{gw} chunk={chunk} N={-(-gh * gw // chunk)}")
    o, sT = _run_state(q, k, v, g, gh, gw, [1], chunk, s0)
    ro, rs = oracle.gla_forward(q, k, v, g, gh, gw, [1], s0=s0, return_state=True)
    eo, es = rel_err(o, ro), rel_err(sT, rs)
    say(f"  o err {eo:.2e}  S_T err {es:.2e}")
    assert eo <= TOL and es <= TOL


def test_scan_phase_with_state_matches_chunked_model():
    gh, gw, B, H, dk, dv, C = 30, 31, 2, 2, 64, 64, 16  # 930 tokens: 59 chunks
    q, k, v, g = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=340)
    s0 = _state(np.random.default_rng(4), B, H, dk, dv, 2.0)
    dirs = [3, 0]
    tq, tk, tv, tg = to_dev(q, k, v, g)
    ts0 = to_dev(s0)[0]
    sf = torch.empty_like(ts0)
    ws = gla.chunk_summaries(tk, tv, tg, gh, gw, dirs, C)
    gla.state_scan(B, H, gh, gw, dk, dv, C, ws, s0=ts0, s_final=sf)
    torch.cuda.synchronize()
    _, _, S = gla.workspace_states(ws, B, H, gh, gw, dk, dv, C)
    s = lambda x: oracle.to_scan(x, gh, gw, dirs)
    _, _, _, S_ref, sT_ref = oracle.chunkwise(s(q), s(k), s(v), s(g), C, return_states=True, s0=s0)
    assert rel_err(S, S_ref) <= 2e-3
    assert rel_err(sf.double().cpu().numpy(), sT_ref) <= 2e-3


@pytest.mark.parametrize("B,H,gh,gw,dk,dv,chunk", [
    (8, 8, 16, 16, 64, 64, 16),    # 32,768 state groups, chains of 16 chunks (window 8)
    (8, 8, 32, 32, 64, 64, 16),    # chains of 64 chunks (window 16)
    (16, 16, 8, 8, 32, 32, 16),    # 32/32 heads, chains of 4 chunks (shorter than the window)
    (4, 8, 64, 64, 64, 64, 16),    # 16,384 groups with chains of 256 chunks
])
def test_serial_scan_with_carried_state(B, H, gh, gw, dk, dv, chunk):
    """Enough chains for the serial boundary scan: outputs and S_T against the
    oracle, and the scan's entering states against the chunked model."""
    q, k, v, g = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=350 + B + gh + dk)
    s0 = _state(np.random.default_rng(8), B, H, dk, dv)
    dirs = [b % 4 for b in range(B)]
    say(f"serial scan B={B} H={H} grid={gh}x{gw} dk={dk} dv={dv} chunk={chunk}")
    tq, tk, tv, tg = to_dev(q, k, v, g)
    ts0 = to_dev(s0)[0]
    o, sT = gla.fwd_state(tq, tk, tv, tg, gh, gw, dirs, chunk=chunk, s0=ts0,
                          schedule=gla.SCHED_THREE_PHASE)
    torch.cuda.synchronize()
    ro, rs = oracle.gla_forward(q, k, v, g, gh, gw, dirs, s0=s0, return_state=True)
    eo, es = rel_err(o.double().cpu().numpy(), ro), rel_err(sT.double().cpu().numpy(), rs)
    say(f"  o err {eo:.2e}  S_T err {es:.2e}")
    assert eo <= TOL and es <= TOL
    ws = gla.chunk_summaries(tk, tv, tg, gh, gw, dirs, chunk)
    gla.state_scan(B, H, gh, gw, dk, dv, chunk, ws, s0=ts0)
    torch.cuda.synchronize()
    _, _, S = gla.workspace_states(ws, B, H, gh, gw, dk, dv, chunk)
    s = lambda x: oracle.to_scan(x, gh, gw, dirs)
    _, _, _, S_ref, _ = oracle.chunkwise(s(q), s(k), s(v), s(g), chunk, return_states=True, s0=s0)
    assert rel_err(S, S_ref) <= 2e-3

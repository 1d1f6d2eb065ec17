"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: max|o - o_ref| / max|o_ref| <= 5e-3 with o_ref the float64 recurrence on
exactly the values the GPU receives; the scan-order permutation is bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, cosine, rel_err, run_fwd, say, to_dev
from recurrent_vision_token_gla_amd import gla
from recurrent_vision_token_gla_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gla.load()
    yield


# ---------------------------------------------------------------- scan order
# the large grids exercise the column walk's float-reciprocal division near its
# 2^22-token limit (prime heights, the largest quotients) and the integer
# division beyond it
@pytest.mark.parametrize("grid", [(1, 1), (1, 7), (7, 1), (5, 7), (8, 8), (13, 3), (40, 40),
                                  (80, 80), (128, 128), (3, 200), (1021, 4093), (3, 1398101),
                                  (2048, 2048), (2049, 2047)])
def test_scan_perm_bit_exact(grid):
    gh, gw = grid
    for d in range(4):
        say(f"scan_perm grid={grid} dir={d}")
        got = gla.scan_perm(gh, gw, d).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.scan_order(gh, gw, d))


# ---------------------------------------------------------------- workloads
def _check_workload_call(w, call):
    q, k, v, g = W.workload_inputs(w, call)
    dirs = w.directions(call)
    say(f"workload {w.index} {w.name} call {call} dirs={dirs[:4]}")
    o = run_fwd(q, k, v, g, w.grid_h, w.grid_w, dirs, w.chunk)
    assert np.all(np.isfinite(o))
    ref = oracle.gla_forward(q, k, v, g, w.grid_h, w.grid_w, dirs)
    err = rel_err(o, ref)
    say(f"  rel_err={err:.3e} cosine={cosine(o, ref):.7f}")
    assert err <= TOL, err
    return err


def test_workload0_tiny_fp32():
    _check_workload_call(W.WORKLOADS[0], 0)


@pytest.mark.parametrize("call", range(4))
def test_workload1_img640_each_direction(call):
    _check_workload_call(W.WORKLOADS[1], call)


@pytest.mark.parametrize("call", range(4))
def test_workload2_img1280_each_direction(call):
    _check_workload_call(W.WORKLOADS[2], call)


def test_workload3_batched_per_batch_directions():
    _check_workload_call(W.WORKLOADS[3], 0)


@pytest.mark.parametrize("call", range(12))
def test_workload4_stack_full(call):
    # every call of the 12-block stack (the directions cycle L2R, R2L, T2B,
    # B2T), every (b, h) against the oracle
    _check_workload_call(W.WORKLOADS[4], call)


# ---------------------------------------------------------------- phases
def test_phase_intermediates_match_chunked_model():
    """U, a and the boundary states S against the float64 chunked model."""
    gh, gw, B, H, dk, dv, C = 10, 13, 2, 3, 64, 32, 32  # 130 tokens: 5 chunks, ragged tail
    q, k, v, g = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=77)
    dirs = [2, 1]
    tq, tk, tv, tg = to_dev(q, k, v, g)
    ws = gla.chunk_summaries(tk, tv, tg, gh, gw, dirs, C)
    gla.state_scan(B, H, gh, gw, dk, dv, C, ws)
    torch.cuda.synchronize()
    U, a, S = gla.workspace_states(ws, B, H, gh, gw, dk, dv, C)
    s = lambda x: oracle.to_scan(x, gh, gw, dirs)
    _, U_ref, a_ref, S_ref, _ = oracle.chunkwise(s(q), s(k), s(v), s(g), C, return_states=True)
    say(f"U err {rel_err(U, U_ref):.2e}  a err {rel_err(a, a_ref):.2e}  "
        f"S err {rel_err(S, S_ref):.2e}")
    assert rel_err(U, U_ref) <= 2e-3
    assert rel_err(a, a_ref) <= 1e-5
    assert rel_err(S, S_ref) <= 2e-3
    o = gla.chunk_outputs(tq, tk, tv, tg, gh, gw, dirs, C, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.gla_forward(q, k, v, g, gh, gw, dirs)
    assert rel_err(o.double().cpu().numpy(), ref) <= TOL


# ---------------------------------------------------------------- shapes and edges
@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 64), (64, 32), (64, 64)])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_shapes_chunks_and_ragged_tail(dk, dv, chunk):
    gh, gw, B, H = 9, 17, 2, 2  # 153 tokens: several chunks and a ragged tail
    q, k, v, g = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=dk + dv + chunk)
    dirs = [0, 3]
    say(f"dk={dk} dv={dv} chunk={chunk}")
    o = run_fwd(q, k, v, g, gh, gw, dirs, chunk)
    ref = oracle.gla_forward(q, k, v, g, gh, gw, dirs)
    assert rel_err(o, ref) <= TOL


def test_chunk_size_invariance():
    gh, gw = 40, 40
    q, k, v, g = W.make_inputs(1, gh * gw, 6, 64, 64, np.float16, seed=9)
    ref = oracle.gla_forward(q, k, v, g, gh, gw, [2])
    outs = [run_fwd(q, k, v, g, gh, gw, [2], C) for C in (16, 32, 64)]
    for o in outs:
        assert rel_err(o, ref) <= TOL
    assert rel_err(outs[0], outs[2]) <= TOL


def test_fp32_inputs():
    gh, gw = 12, 12
    q, k, v, g = W.make_inputs(2, gh * gw, 3, 64, 64, np.float32, seed=10)
    o = run_fwd(q, k, v, g, gh, gw, [1, 2], 64)
    assert rel_err(o, oracle.gla_forward(q, k, v, g, gh, gw, [1, 2])) <= TOL


def test_no_decay_is_causal_linear_attention():
    gh, gw = 8, 12
    q, k, v, _ = W.make_inputs(1, gh * gw, 2, 64, 64, np.float16, seed=11)
    g = np.zeros_like(q)
    o = run_fwd(q, k, v, g, gh, gw, [0], 64)
    qd, kd, vd = (x.astype(np.float64) for x in (q, k, v))
    ref = np.stack([np.tril(qd[0, :, h] @ kd[0, :, h].T) @ vd[0, :, h] for h in range(2)], axis=1)[None]
    assert rel_err(o, ref) <= TOL


def test_overwhelming_decay_keeps_only_the_diagonal():
    gh, gw = 8, 8
    q, k, v, _ = W.make_inputs(1, gh * gw, 2, 64, 64, np.float16, seed=12)
    g = np.full(q.shape, -1e4, np.float16)
    o = run_fwd(q, k, v, g, gh, gw, [0], 64)
    assert np.all(np.isfinite(o))
    qd, kd, vd = (x.astype(np.float64) for x in (q, k, v))
    ref = np.sum(qd * kd, axis=-1, keepdims=True) * vd
    assert rel_err(o, ref) <= TOL


def test_strong_decay_mixed_channels_small():
    gh, gw = 16, 16
    q, k, v, g = W.make_inputs(2, gh * gw, 2, 64, 64, np.float16, seed=13, gate="mixed")
    o = run_fwd(q, k, v, g, gh, gw, [3, 0], 64)
    assert rel_err(o, oracle.gla_forward(q, k, v, g, gh, gw, [3, 0])) <= TOL


def test_single_token():
    q, k, v, g = W.make_inputs(3, 1, 2, 32, 64, np.float16, seed=14)
    o = run_fwd(q, k, v, g, 1, 1, [0, 1, 2], 16)
    qd, kd, vd = (x.astype(np.float64) for x in (q, k, v))
    assert rel_err(o, np.sum(qd * kd, -1, keepdims=True) * vd) <= TOL


def test_more_batches_than_one_launch_holds():
    B = 1030  # more than the per-launch direction pack: the batch is sliced
    q, k, v, g = W.make_inputs(B, 16, 1, 32, 32, np.float16, seed=15)
    dirs = [b % 4 for b in range(B)]
    o = run_fwd(q, k, v, g, 4, 4, dirs, 16)
    assert rel_err(o, oracle.gla_forward(q, k, v, g, 4, 4, dirs)) <= TOL


def test_empty_batch():
    q = torch.empty((0, 16, 2, 64), dtype=torch.float16, device="cuda")
    v = torch.empty((0, 16, 2, 64), dtype=torch.float16, device="cuda")
    o = gla.fwd(q, q.clone(), v, q.clone(), 4, 4, [], 64)
    assert o.shape == (0, 16, 2, 64)


# ---------------------------------------------------------------- behaviour
def test_deterministic():
    w = W.WORKLOADS[3]
    q, k, v, g = W.workload_inputs(w, 0)
    tq, tk, tv, tg = to_dev(q, k, v, g)
    o1 = gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, w.directions(0), 64)
    o2 = gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, w.directions(0), 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_writes_nothing_outside_the_output():
    gh, gw, B, H, dk, dv = 7, 9, 2, 3, 64, 64
    q, k, v, g = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=16)
    tq, tk, tv, tg = to_dev(q, k, v, g)
    n = B * gh * gw * H * dv
    pad = 4096
    big = torch.full((n + 2 * pad,), 1234.0, dtype=torch.float16, device="cuda")
    out = big[pad:pad + n].view(B, gh * gw, H, dv)
    wsn = gla.workspace_bytes(B, H, gh, gw, dk, dv, 64)
    wsbig = torch.full((wsn + 2 * 4096,), 77, dtype=torch.uint8, device="cuda")
    ws = wsbig[4096:4096 + wsn]
    gla.fwd(tq, tk, tv, tg, gh, gw, [1, 2], 64, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(big[:pad] == 1234.0) and torch.all(big[pad + n:] == 1234.0)
    assert torch.all(wsbig[:4096] == 77) and torch.all(wsbig[4096 + wsn:] == 77)
    ref = oracle.gla_forward(q, k, v, g, gh, gw, [1, 2])
    assert rel_err(out.double().cpu().numpy(), ref) <= TOL


def test_inputs_untouched():
    w = W.WORKLOADS[1]
    q, k, v, g = W.workload_inputs(w, 2)
    tq, tk, tv, tg = to_dev(q, k, v, g)
    copies = [t.clone() for t in (tq, tk, tv, tg)]
    gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, [2], 64)
    torch.cuda.synchronize()
    for a, b in zip((tq, tk, tv, tg), copies):
        assert torch.equal(a, b)


def test_graph_capture_replays_match_eager():
    w = W.WORKLOADS[1]
    q, k, v, g = W.workload_inputs(w, 1)
    tq, tk, tv, tg = to_dev(q, k, v, g)
    ws = gla.alloc_workspace(w.B, w.H, w.grid_h, w.grid_w, w.dk, w.dv, w.chunk)
    out = torch.empty_like(tv)
    eager = gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, [1], 64, out=torch.empty_like(tv),
                    workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            gla.fwd(tq, tk, tv, tg, w.grid_h, w.grid_w, [1], 64, out=out, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.fill_(0)
        ws.fill_(0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep

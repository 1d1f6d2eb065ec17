"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each check takes the implementation under test as arguments, so that the same
checks run on the oracle (they must pass) and on copies with planted mistakes
(at least one must fail; see test_oracle_mutations.py).

  scan   -- callable (grid_h, grid_w, direction) -> permutation array
  rec    -- callable (q, k, v, g) -> o, scan-ordered [B, T, H, D] float64
  rec_state -- callable (q, k, v, g, s0) -> (o, S_T): the carried-state
            form, s0 and S_T [B, H, dk, dv]
  chunked-- callable (q, k, v, g, chunk) -> o, same convention

What pins what:
  * hand-derived fixtures under tests/golden/ (scan orders, three recurrence
    cases, two whole-forward cases with every direction);
  * an O(T^2) brute-force closed form of the unrolled recurrence;
  * special cases that reduce to textbook formulas: no decay is causal linear
    attention (the pages cite "Transformers are RNNs"), a constant scalar
    decay is retention (the pages cite RetNet), a per-key-dimension constant
    decay has an integer-power closed form, overwhelming decay leaves only
    the diagonal term, one token gives (q . k) v;
  * invariants: linear in v, value columns independent, (batch, head) slices
    independent, reversed direction equals reversing the token sequence,
    top->bottom equals left->right on the transposed grid;
  * the scan-order permutation against its arithmetic closed form;
  * carried state: hand-derived fixtures, the brute-force closed form with
    the decayed initial state, no decay (S_0 + K^T V), a zero S_0 equals the
    stateless forward, and splitting a sequence anywhere and carrying the
    state across the cut changes nothing.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAMES = {"L2R": 0, "R2L": 1, "T2B": 2, "B2T": 3}


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_inputs(rng, B, T, H, dk, dv, gate_scale=0.3):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = -np.abs(rng.standard_normal((B, T, H, dk))) * gate_scale
    return q, k, v, g


def compose(scan, rec, q, k, v, g, grid_h, grid_w, dirs):
    """Raster in, raster out, using the given scan order and recurrence."""
    out = np.empty(v.shape, np.float64)
    for b, d in enumerate(dirs):
        p = np.asarray(scan(grid_h, grid_w, d))
        o = rec(q[b:b + 1, p], k[b:b + 1, p], v[b:b + 1, p], g[b:b + 1, p])
        out[b, p] = o[0]
    return out


def brute_force(q, k, v, g):
    """o_t = sum_{s<=t} sum_d q_t[d] k_s[d] exp(G_t[d] - G_s[d]) v_s,
    G_t = sum_{r<=t} g_r: the recurrence unrolled, evaluated pair by pair."""
    B, T, H, dk = q.shape
    G = np.cumsum(g, axis=1)
    o = np.zeros(v.shape)
    for t in range(T):
        for s in range(t + 1):
            w = np.sum(q[:, t] * k[:, s] * np.exp(G[:, t] - G[:, s]), axis=-1)
            o[:, t] += w[..., None] * v[:, s]
    return o


# ---------------------------------------------------------------- checks

def check_golden_scan(scan):
    for case in load_golden("scan_orders.json")["cases"]:
        for name, code in NAMES.items():
            got = np.asarray(scan(case["grid_h"], case["grid_w"], code))
            assert got.tolist() == case[name], (case["comment"], name, got)


def check_golden_recurrence(rec):
    for case in load_golden("recurrence_cases.json")["cases"]:
        arr = lambda key: np.asarray(case[key], np.float64)[None, :, None, :]
        o = rec(arr("q"), arr("k"), arr("v"), arr("g"))[0, :, 0, :]
        np.testing.assert_allclose(o, np.asarray(case["o"]), rtol=1e-12, atol=1e-12,
                                   err_msg=case["name"])


def check_golden_forward(scan, rec):
    for case in load_golden("forward_directions.json")["cases"]:
        gh, gw = case["grid_h"], case["grid_w"]
        T = gh * gw
        ones = np.ones((4, T, 1, 1))
        v = np.broadcast_to(np.asarray(case["v_raster"], np.float64)[None, :, None, None],
                            (4, T, 1, 1)).copy()
        g = np.full((4, T, 1, 1), case["g"])
        o = compose(scan, rec, ones, ones, v, g, gh, gw, [0, 1, 2, 3])
        for name, code in NAMES.items():
            np.testing.assert_allclose(o[code, :, 0, 0], case["o_raster"][name],
                                       rtol=1e-12, err_msg=f"{case['name']} {name}")


def check_brute_force(rec, seed=0):
    rng = np.random.default_rng(seed)
    for (B, T, H, dk, dv) in [(1, 1, 1, 1, 1), (2, 7, 3, 4, 5), (1, 13, 2, 8, 3)]:
        q, k, v, g = rand_inputs(rng, B, T, H, dk, dv)
        ref = brute_force(q, k, v, g)
        o = rec(q, k, v, g)
        err = np.max(np.abs(o - ref)) / max(1e-300, np.max(np.abs(ref)))
        assert err <= 1e-10, (B, T, H, dk, dv, err)


def check_no_decay_is_linear_attention(rec, seed=1):
    rng = np.random.default_rng(seed)
    q, k, v, _ = rand_inputs(rng, 2, 9, 2, 4, 3)
    o = rec(q, k, v, np.zeros_like(q))
    for b in range(2):
        for h in range(2):
            ref = np.tril(q[b, :, h] @ k[b, :, h].T) @ v[b, :, h]
            np.testing.assert_allclose(o[b, :, h], ref, rtol=1e-11, atol=1e-11)


def check_constant_decay_is_retention(rec, seed=2):
    rng = np.random.default_rng(seed)
    q, k, v, _ = rand_inputs(rng, 1, 10, 1, 3, 2)
    gamma = 0.8
    o = rec(q, k, v, np.full(q.shape, np.log(gamma)))
    t = np.arange(10)
    Gam = np.where(t[:, None] >= t[None, :], gamma ** (t[:, None] - t[None, :]).clip(0), 0.0)
    ref = (np.tril(q[0, :, 0] @ k[0, :, 0].T) * Gam) @ v[0, :, 0]
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-11, atol=1e-11)


def check_per_key_dim_constant_decay(rec, seed=3):
    """Key dim d decays by gamma_d each step: o_t = sum_s sum_d q_t[d] k_s[d]
    gamma_d^(t-s) v_s; the value side never decays."""
    rng = np.random.default_rng(seed)
    q, k, v, _ = rand_inputs(rng, 1, 8, 1, 3, 4)
    gam = np.array([0.9, 0.5, 0.25])
    o = rec(q, k, v, np.broadcast_to(np.log(gam), q.shape).copy())
    ref = np.zeros((8, 4))
    for t in range(8):
        for s in range(t + 1):
            w = np.sum(q[0, t, 0] * k[0, s, 0] * gam ** (t - s))
            ref[t] += w * v[0, s, 0]
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-11, atol=1e-11)


def check_overwhelming_decay(rec, seed=4):
    rng = np.random.default_rng(seed)
    q, k, v, _ = rand_inputs(rng, 1, 6, 2, 4, 3)
    o = rec(q, k, v, np.full(q.shape, -1e4))
    ref = np.sum(q * k, axis=-1, keepdims=True) * v
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert np.all(np.isfinite(o))


def check_single_token(rec, seed=5):
    rng = np.random.default_rng(seed)
    q, k, v, g = rand_inputs(rng, 3, 1, 2, 5, 4)
    o = rec(q, k, v, g)
    np.testing.assert_allclose(o, np.sum(q * k, axis=-1, keepdims=True) * v, rtol=1e-12)


def check_structure(rec, seed=6):
    rng = np.random.default_rng(seed)
    q, k, v, g = rand_inputs(rng, 2, 11, 3, 4, 5)
    o = rec(q, k, v, g)
    # linear in v
    v2 = rng.standard_normal(v.shape)
    np.testing.assert_allclose(rec(q, k, 2.0 * v - 3.0 * v2, g), 2.0 * o - 3.0 * rec(q, k, v2, g),
                               rtol=1e-10, atol=1e-10)
    # value column e of o depends on value column e of v only
    vp = v.copy()
    vp[..., 2] += 1.0
    op = rec(q, k, vp, g)
    keep = [0, 1, 3, 4]
    np.testing.assert_allclose(op[..., keep], o[..., keep], rtol=0, atol=1e-14)
    assert np.max(np.abs(op[..., 2] - o[..., 2])) > 1e-6
    # (batch, head) slices are independent
    qp = q.copy()
    qp[1, :, 2] += 1.0
    op = rec(qp, k, v, g)
    mask = np.ones((2, 3), bool)
    mask[1, 2] = False
    sel = np.broadcast_to(mask[:, None, :, None], o.shape)
    np.testing.assert_allclose(op[sel], o[sel], rtol=0, atol=1e-14)
    # causality: token t never sees a later token
    vq = v.copy()
    vq[:, 7:] += 5.0
    np.testing.assert_allclose(rec(q, k, vq, g)[:, :7], o[:, :7], rtol=0, atol=1e-14)
    # zero q or zero v gives zero output
    assert np.all(rec(np.zeros_like(q), k, v, g) == 0)
    assert np.all(rec(q, k, np.zeros_like(v), g) == 0)


def check_scan_closed_form(scan, grids):
    """pi_L2R(t)=t; pi_R2L(t)=T-1-t; pi_T2B(t)=(t mod gh)*gw + t div gh;
    pi_B2T(t)=pi_T2B(T-1-t); every order is a permutation."""
    for gh, gw in grids:
        T = gh * gw
        t = np.arange(T)
        t2b = (t % gh) * gw + t // gh
        expect = {0: t, 1: T - 1 - t, 2: t2b, 3: t2b[::-1]}
        for d in range(4):
            p = np.asarray(scan(gh, gw, d))
            assert p.tolist() == expect[d].tolist(), (gh, gw, d)
            assert sorted(p.tolist()) == list(range(T))


def check_direction_invariants(scan, rec, seed=7):
    rng = np.random.default_rng(seed)
    for gh, gw in [(3, 5), (4, 4), (1, 6), (6, 1)]:
        T = gh * gw
        q, k, v, g = rand_inputs(rng, 1, T, 2, 3, 2)
        fwd = lambda d, x=(q, k, v, g), a=gh, b=gw: compose(scan, rec, *x, a, b, [d])
        flip = lambda x: x[:, ::-1].copy()
        # reversing the direction equals reversing the token sequence
        o_r2l = fwd(1)
        o_ref = compose(scan, rec, flip(q), flip(k), flip(v), flip(g), gh, gw, [0])
        np.testing.assert_allclose(o_r2l, flip(o_ref), rtol=1e-12, atol=1e-12)
        o_b2t = fwd(3)
        o_ref = compose(scan, rec, flip(q), flip(k), flip(v), flip(g), gh, gw, [2])
        np.testing.assert_allclose(o_b2t, flip(o_ref), rtol=1e-12, atol=1e-12)

        # top->bottom on (gh, gw) equals left->right on the transposed grid
        def tr(x, a, b):
            return x.reshape(x.shape[0], a, b, *x.shape[2:]).swapaxes(1, 2).reshape(x.shape)
        o_t2b = fwd(2)
        o_ref = compose(scan, rec, tr(q, gh, gw), tr(k, gh, gw), tr(v, gh, gw),
                        tr(g, gh, gw), gw, gh, [0])
        np.testing.assert_allclose(o_t2b, tr(o_ref, gw, gh), rtol=1e-12, atol=1e-12)


def check_chunk_independence(rec, chunked, seed=8):
    """The chunked schedule reproduces the recurrence for any chunk size."""
    rng = np.random.default_rng(seed)
    for T in (1, 5, 64, 70):
        q, k, v, g = rand_inputs(rng, 2, T, 2, 4, 3)
        ref = rec(q, k, v, g)
        for C in sorted({1, 2, 4, 16, 64, T}):
            o = chunked(q, k, v, g, C)
            err = np.max(np.abs(o - ref)) / np.max(np.abs(ref))
            assert err <= 1e-12, (T, C, err)


def brute_force_state(q, k, v, g, s0):
    """The recurrence unrolled from S_0:
    o_t = q_t diag(exp(G_t)) S_0 + sum_{s<=t} (q_t . k_s exp(G_t - G_s)) v_s,
    S_T = diag(exp(G_{T-1})) S_0 + sum_s diag(exp(G_{T-1} - G_s)) k_s^T v_s."""
    o = brute_force(q, k, v, g)
    G = np.cumsum(g, axis=1)
    B, T, H, dk = q.shape
    for t in range(T):
        o[:, t] += np.einsum("bhd,bhde->bhe", q[:, t] * np.exp(G[:, t]), s0)
    w = np.exp(G[:, -1:] - G)                               # [B, T, H, dk]
    sT = np.exp(G[:, -1])[..., None] * s0 + np.einsum("bthd,bthe->bhde", k * w, v)
    return o, sT


def check_golden_state(rec_state):
    for case in load_golden("state_cases.json")["cases"]:
        arr = lambda key: np.asarray(case[key], np.float64)[None, :, None, :]
        s0 = np.asarray(case["s0"], np.float64)[None, None]
        o, sT = rec_state(arr("q"), arr("k"), arr("v"), arr("g"), s0)
        np.testing.assert_allclose(o[0, :, 0, :], case["o"], rtol=1e-12, atol=1e-12,
                                   err_msg=case["name"])
        np.testing.assert_allclose(sT[0, 0], case["s_final"], rtol=1e-12, atol=1e-12,
                                   err_msg=case["name"])


def check_state_brute_force(rec_state, seed=20):
    rng = np.random.default_rng(seed)
    for (B, T, H, dk, dv) in [(1, 1, 1, 1, 1), (2, 6, 2, 3, 3), (1, 9, 2, 4, 2)]:
        q, k, v, g = rand_inputs(rng, B, T, H, dk, dv)
        s0 = rng.standard_normal((B, H, dk, dv))
        ro, rs = brute_force_state(q, k, v, g, s0)
        o, sT = rec_state(q, k, v, g, s0)
        assert np.max(np.abs(o - ro)) <= 1e-10 * np.max(np.abs(ro)), (B, T, H, dk, dv)
        assert np.max(np.abs(sT - rs)) <= 1e-10 * np.max(np.abs(rs)), (B, T, H, dk, dv)


def check_state_no_decay(rec_state, seed=21):
    rng = np.random.default_rng(seed)
    q, k, v, _ = rand_inputs(rng, 1, 7, 1, 3, 3)
    s0 = rng.standard_normal((1, 1, 3, 3))
    o, sT = rec_state(q, k, v, np.zeros_like(q), s0)
    Q, K, V = q[0, :, 0], k[0, :, 0], v[0, :, 0]
    np.testing.assert_allclose(o[0, :, 0], Q @ s0[0, 0] + np.tril(Q @ K.T) @ V,
                               rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(sT[0, 0], s0[0, 0] + K.T @ V, rtol=1e-11, atol=1e-11)


def check_state_split(rec_state, seed=22):
    """Running [x1; x2] from S_0 equals running x1 from S_0, then x2 from the
    state x1 hands back: same outputs, same final state."""
    rng = np.random.default_rng(seed)
    T = 11
    q, k, v, g = rand_inputs(rng, 2, T, 2, 3, 4)
    s0 = rng.standard_normal((2, 2, 3, 4))
    o, sT = rec_state(q, k, v, g, s0)
    for cut in (1, 4, 10):
        o1, s1 = rec_state(q[:, :cut], k[:, :cut], v[:, :cut], g[:, :cut], s0)
        o2, s2 = rec_state(q[:, cut:], k[:, cut:], v[:, cut:], g[:, cut:], s1)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(s2, sT, rtol=1e-11, atol=1e-11)


def check_state_zero_is_stateless(rec_state, rec, seed=23):
    rng = np.random.default_rng(seed)
    q, k, v, g = rand_inputs(rng, 2, 8, 2, 4, 3)
    o, _ = rec_state(q, k, v, g, np.zeros((2, 2, 4, 3)))
    np.testing.assert_allclose(o, rec(q, k, v, g), rtol=1e-12, atol=1e-12)


ALL_STATE_CHECKS = [check_golden_state, check_state_brute_force, check_state_no_decay,
                    check_state_split]


ALL_REC_CHECKS = [check_golden_recurrence, check_brute_force,
                  check_no_decay_is_linear_attention, check_constant_decay_is_retention,
                  check_per_key_dim_constant_decay, check_overwhelming_decay,
                  check_single_token, check_structure]

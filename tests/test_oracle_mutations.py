"""Planted mistakes in copies of the oracle must be caught by the pins.

Each mutant below is the oracle's arithmetic with one plausible slip (a
dropped term, a wrong sign or index, a swapped operand, a wrong axis). The
test passes only if at least one pin in tests/pins.py fails on the mutant,
which shows that the pins are strong enough to catch that class of mistake.
Everything here runs on the CPU.
"""
import numpy as np
import pytest

import oracle
import pins


def _rec_generic(q, k, v, g, decay_then_add=True, inclusive=True, swap_qk=False,
                 gate_shift=0, gate_sign=1.0, scalar_gate=False, no_gate=False,
                 out_with_k=False):
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    if swap_qk:
        q, k = k, q
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        tg = t - gate_shift
        gt = g[:, tg] if 0 <= tg < T else np.zeros_like(g[:, 0])
        if scalar_gate:
            gt = np.broadcast_to(gt.mean(-1, keepdims=True), gt.shape)
        a = np.exp(gate_sign * gt)[..., None]
        if no_gate:
            a = 1.0
        kv = k[:, t][..., None] * v[:, t][:, :, None, :]
        if not inclusive:
            o[:, t] = np.einsum("bhd,bhde->bhe", (k if out_with_k else q)[:, t], S)
        S = a * S + kv if decay_then_add else a * (S + kv)
        if inclusive:
            o[:, t] = np.einsum("bhd,bhde->bhe", (k if out_with_k else q)[:, t], S)
    return o


REC_MUTANTS = {
    "decay_after_add": dict(decay_then_add=False),
    "exclusive_output": dict(inclusive=False),
    "q_k_swapped": dict(swap_qk=True),
    "gate_index_late": dict(gate_shift=1),
    "gate_index_early": dict(gate_shift=-1),
    "gate_sign_flipped": dict(gate_sign=-1.0),
    "gate_shared_over_key_dims": dict(scalar_gate=True),
    "gate_dropped": dict(no_gate=True),
    "output_reads_k": dict(out_with_k=True),
}


def _failures(checks):
    failed = []
    for name, fn in checks:
        try:
            with np.errstate(all="ignore"):
                fn()
        except (AssertionError, ValueError, FloatingPointError, IndexError) as e:
            failed.append(name)
    return failed


def test_unmutated_generic_copy_passes():
    rec = lambda q, k, v, g: _rec_generic(q, k, v, g)
    checks = [(c.__name__, lambda c=c: c(rec)) for c in pins.ALL_REC_CHECKS]
    assert _failures(checks) == []


@pytest.mark.parametrize("name", sorted(REC_MUTANTS))
def test_recurrence_mutant_is_caught(name):
    rec = lambda q, k, v, g: _rec_generic(q, k, v, g, **REC_MUTANTS[name])
    checks = [(c.__name__, lambda c=c: c(rec)) for c in pins.ALL_REC_CHECKS]
    checks.append(("golden_forward", lambda: pins.check_golden_forward(oracle.scan_order, rec)))
    assert _failures(checks), f"no pin caught mutant {name}"


def _scan_generic(gh, gw, d, mistake):
    raster = np.arange(gh * gw).reshape(gh, gw)
    if d == 0:
        return raster.ravel()
    if d == 1:
        return raster[:, ::-1].ravel() if mistake == "r2l_per_row" else raster.ravel()[::-1]
    t2b = (np.arange(gh * gw).reshape(gw, gh).T.ravel() if mistake == "t2b_wrong_reshape"
           else raster.T.ravel())
    if d == 2:
        return t2b
    if mistake == "b2t_reverses_l2r":
        return raster.ravel()[::-1]
    if mistake == "b2t_per_column":
        return raster.T[:, ::-1].ravel()
    return t2b[::-1]


SCAN_MUTANTS = ["r2l_per_row", "t2b_wrong_reshape", "b2t_reverses_l2r", "b2t_per_column"]


@pytest.mark.parametrize("mistake", SCAN_MUTANTS)
def test_scan_mutant_is_caught(mistake):
    scan = lambda gh, gw, d: _scan_generic(gh, gw, d, mistake)
    checks = [
        ("golden_scan", lambda: pins.check_golden_scan(scan)),
        ("closed_form", lambda: pins.check_scan_closed_form(scan, [(2, 3), (3, 2), (4, 5)])),
        ("golden_forward", lambda: pins.check_golden_forward(scan, oracle.recurrence_numpy)),
        ("direction_invariants", lambda: pins.check_direction_invariants(scan, oracle.recurrence_numpy)),
    ]
    assert _failures(checks), f"no pin caught scan mutant {mistake}"


def test_unmutated_scan_copy_passes():
    scan = lambda gh, gw, d: _scan_generic(gh, gw, d, None)
    pins.check_golden_scan(scan)
    pins.check_scan_closed_form(scan, [(2, 3), (3, 2), (4, 5)])


def _chunked_generic(q, k, v, g, C, mistake=None):
    """The chunked schedule with one planted mistake."""
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    for n in range(-(-T // C)):
        sl = slice(n * C, min(T, (n + 1) * C))
        L = sl.stop - sl.start
        qn, kn, vn, gn = (np.transpose(x[:, sl], (0, 2, 1, 3)) for x in (q, k, v, g))
        b = np.cumsum(gn, axis=2)
        if mistake == "exclusive_cumsum":
            b = b - gn
        Bt = b[:, :, -1]
        wk = np.exp(Bt[:, :, None, :] - b)
        if mistake == "summary_without_decay":
            wk = np.ones_like(wk)
        U = np.einsum("bhjd,bhje->bhde", kn * wk, vn)
        causal = np.tril(np.ones((L, L), bool))[None, None, :, :, None]
        diff = np.where(causal, b[:, :, :, None, :] - b[:, :, None, :, :], 0.0)
        dec = np.where(causal, np.exp(diff), 0.0)
        if mistake == "strict_causal_mask":
            dec = dec * (1 - np.eye(L))[None, None, :, :, None]
        A = np.einsum("bhid,bhjd,bhijd->bhij", qn, kn, dec)
        qd = qn * np.exp(b)
        if mistake == "readout_without_decay":
            qd = qn
        out = np.einsum("bhij,bhje->bhie", A, vn)
        if mistake != "readout_dropped":
            out = out + np.einsum("bhid,bhde->bhie", qd, S)
        o[:, sl] = np.transpose(out, (0, 2, 1, 3))
        a = np.exp(Bt)[..., None]
        if mistake == "scan_without_decay":
            a = 1.0
        S = a * S + U
    return o


CHUNK_MUTANTS = ["exclusive_cumsum", "summary_without_decay", "strict_causal_mask",
                 "readout_without_decay", "readout_dropped", "scan_without_decay"]


@pytest.mark.parametrize("mistake", CHUNK_MUTANTS)
def test_chunked_mutant_is_caught(mistake):
    chunked = lambda q, k, v, g, C: _chunked_generic(q, k, v, g, C, mistake)
    checks = [("chunk_independence",
               lambda: pins.check_chunk_independence(oracle.recurrence_c, chunked))]
    assert _failures(checks), f"no pin caught chunked mutant {mistake}"


def test_unmutated_chunked_copy_passes():
    chunked = lambda q, k, v, g, C: _chunked_generic(q, k, v, g, C, None)
    pins.check_chunk_independence(oracle.recurrence_c, chunked)


def _rec_state_generic(q, k, v, g, s0, mistake=None):
    """The carried-state recurrence with one planted mistake."""
    q, k, v, g, s0 = (np.asarray(x, np.float64) for x in (q, k, v, g, s0))
    B, T, H, dk = q.shape
    S = np.zeros_like(s0) if mistake == "s0_ignored" else s0.copy()
    if mistake == "s0_transposed":
        S = np.swapaxes(s0, -1, -2).copy()
    o = np.zeros(v.shape)
    prev = S
    for t in range(T):
        a = np.exp(g[:, t])[..., None]
        if mistake == "s0_not_decayed" and t == 0:
            a = 1.0
        prev = S
        S = a * S + k[:, t][..., None] * v[:, t][:, :, None, :]
        o[:, t] = np.einsum("bhd,bhde->bhe", q[:, t], S)
    if mistake == "final_before_last_token":
        return o, prev
    if mistake == "final_decayed_twice":
        return o, np.exp(g[:, -1])[..., None] * S
    return o, S


STATE_MUTANTS = ["s0_ignored", "s0_transposed", "s0_not_decayed", "final_before_last_token",
                 "final_decayed_twice"]


@pytest.mark.parametrize("mistake", STATE_MUTANTS)
def test_state_mutant_is_caught(mistake):
    rec_state = lambda q, k, v, g, s0: _rec_state_generic(q, k, v, g, s0, mistake)
    checks = [(c.__name__, lambda c=c: c(rec_state)) for c in pins.ALL_STATE_CHECKS]
    assert _failures(checks), f"no pin caught state mutant {mistake}"


def test_unmutated_state_copy_passes():
    rec_state = lambda q, k, v, g, s0: _rec_state_generic(q, k, v, g, s0, None)
    checks = [(c.__name__, lambda c=c: c(rec_state)) for c in pins.ALL_STATE_CHECKS]
    assert _failures(checks) == []

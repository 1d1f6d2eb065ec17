"""The epilogue oracles against their pins, and planted mistakes that the pins
must catch (no GPU)."""
import numpy as np
import pytest

import oracle
import pins_epilogue as P

GATE_CHECKS = [P.check_golden_gate, P.check_gate_against_torch, P.check_gate_properties]
SSW_CHECKS = [P.check_golden_ssw, P.check_ssw_against_torch, P.check_ssw_properties]


@pytest.mark.parametrize("check", GATE_CHECKS, ids=lambda f: f.__name__)
def test_gate_pins(check):
    check(oracle.rmsnorm_gate)


@pytest.mark.parametrize("check", SSW_CHECKS, ids=lambda f: f.__name__)
def test_spatial_swiglu_pins(check):
    check(oracle.spatial_swiglu)


def _gate_mutant(o, z, w, eps, mistake):
    o, z, w = (np.asarray(x, np.float64) for x in (o, z, w))
    if mistake == "mean_over_rows":
        ms = np.mean(o * o, axis=0, keepdims=True)
    elif mistake == "sum_not_mean":
        ms = np.sum(o * o, axis=-1, keepdims=True)
    else:
        ms = np.mean(o * o, axis=-1, keepdims=True)
    rms = np.sqrt(ms) + eps if mistake == "eps_outside_sqrt" else np.sqrt(ms + eps)
    g = 1 / (1 + np.exp(-z)) if mistake == "sigmoid_not_silu" else z / (1 + np.exp(-z))
    if mistake == "silu_of_output":
        g = o / (1 + np.exp(-o))
    ww = 1.0 if mistake == "weight_dropped" else w
    return o / rms * ww * g


GATE_MUTANTS = ["mean_over_rows", "sum_not_mean", "eps_outside_sqrt", "sigmoid_not_silu",
                "silu_of_output", "weight_dropped"]


def _caught(checks, fn):
    for c in checks:
        try:
            with np.errstate(all="ignore"):
                c(fn)
        except (AssertionError, ValueError, IndexError):
            return True
    return False


@pytest.mark.parametrize("mistake", GATE_MUTANTS)
def test_gate_mutant_is_caught(mistake):
    assert _caught(GATE_CHECKS, lambda o, z, w, eps: _gate_mutant(o, z, w, eps, mistake))


def _ssw_mutant(a, u, weight, bias, gh, gw, mistake):
    a, u, w = (np.asarray(x, np.float64) for x in (a, u, weight))
    B, T, Fc = u.shape
    if mistake == "grid_transposed":
        gh, gw = gw, gh
    g = u.reshape(B, gh, gw, Fc)
    if mistake == "wraparound_padding":
        pad = np.pad(g, ((0, 0), (1, 1), (1, 1), (0, 0)), mode="wrap")
    else:
        pad = np.pad(g, ((0, 0), (1, 1), (1, 1), (0, 0)))
    if mistake == "kernel_flipped":
        w = w[:, ::-1, ::-1]
    if mistake == "channels_reversed":
        w = w[::-1]
    conv = np.zeros((B, gh, gw, Fc))
    if bias is not None and mistake != "bias_dropped":
        conv += np.asarray(bias, np.float64)
    for i in range(3):
        for j in range(3):
            conv += w[:, i, j] * pad[:, i:i + gh, j:j + gw]
    conv = conv.reshape(B, T, Fc)
    if mistake == "silu_on_value":
        return a * conv / (1 + np.exp(-conv))
    return a / (1 + np.exp(-a)) * conv


SSW_MUTANTS = ["grid_transposed", "wraparound_padding", "kernel_flipped", "channels_reversed",
               "bias_dropped", "silu_on_value"]


@pytest.mark.parametrize("mistake", SSW_MUTANTS)
def test_spatial_swiglu_mutant_is_caught(mistake):
    assert _caught(SSW_CHECKS, lambda *x: _ssw_mutant(*x, mistake))


def test_unmutated_copies_pass():
    for c in GATE_CHECKS:
        c(lambda o, z, w, eps: _gate_mutant(o, z, w, eps, None))
    for c in SSW_CHECKS:
        c(lambda *x: _ssw_mutant(*x, None))

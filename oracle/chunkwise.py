"""Chunked fp64 model of the forward: the pages' execution schedule, plainly.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages describe the inference operator as the same state update run on a
different schedule (GTR project page, "A Kernel That Makes Recurrence Fast";
ai.info summary of GTR, "Methodology in Plain English"): the token sequence is
cut into chunks of C tokens; a summary of every chunk is computed in parallel
over the chunk x head grid; only the chunk-boundary states are carried
sequentially; then every chunk's outputs are computed independently from a
within-chunk score-value product plus a readout of the boundary state.

This module writes those steps out in float64 with no blocking inside a
chunk, so that tests can check (a) that the schedule reproduces the
token-by-token recurrence for any C, and (b) the GPU path's intermediate
chunk summaries and boundary states, not only its outputs.

Per chunk n of one (batch, head), with local token index i = 0..L-1:
    b_i   = sum_{r <= i} g_r                 cumulative log-decay (dk-vector)
    B_n   = b_{L-1},  a_n = exp(B_n)          total decay of the chunk
    U_n   = sum_j diag(exp(B_n - b_j)) k_j^T v_j           chunk summary
    S_0   = 0 (or a carried state),  S_{n+1} = diag(a_n) S_n + U_n   scan
    A_ij  = sum_d q_i[d] k_j[d] exp(b_i[d] - b_j[d]),  j <= i, else 0
    o_i   = sum_j A_ij v_j + (q_i * exp(b_i)) S_n          output
A last chunk shorter than C is simply shorter (L < C).
"""
from __future__ import annotations

import numpy as np


def chunkwise(q, k, v, g, chunk: int, return_states: bool = False, s0=None):
    """Scan-ordered [B, T, H, D] inputs -> scan-ordered o (float64).

    s0 [B, H, dk, dv] is the state before the first token (None for zero).
    With return_states, also returns U [B, H, N, dk, dv], a [B, H, N, dk],
    the states entering every chunk S [B, H, N, dk, dv] and the state after
    the last chunk [B, H, dk, dv].
    """
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    N = -(-T // chunk)
    o = np.zeros((B, T, H, dv))
    U = np.zeros((B, H, N, dk, dv))
    a = np.zeros((B, H, N, dk))
    S_in = np.zeros((B, H, N, dk, dv))
    # [B, T, H, D] -> [B, H, T, D]
    qh, kh, vh, gh = (np.transpose(x, (0, 2, 1, 3)) for x in (q, k, v, g))

    # summaries, independent over chunks
    for n in range(N):
        sl = slice(n * chunk, min(T, (n + 1) * chunk))
        bcum = np.cumsum(gh[:, :, sl], axis=2)          # [B, H, L, dk]
        Btot = bcum[:, :, -1]                           # [B, H, dk]
        a[:, :, n] = np.exp(Btot)
        kdec = kh[:, :, sl] * np.exp(Btot[:, :, None, :] - bcum)
        U[:, :, n] = np.einsum("bhjd,bhje->bhde", kdec, vh[:, :, sl])

    # boundary-state scan, sequential over chunks
    S = np.zeros((B, H, dk, dv)) if s0 is None else np.array(s0, np.float64)
    for n in range(N):
        S_in[:, :, n] = S
        S = a[:, :, n][..., None] * S + U[:, :, n]

    # outputs, independent over chunks
    for n in range(N):
        sl = slice(n * chunk, min(T, (n + 1) * chunk))
        L = sl.stop - sl.start
        bcum = np.cumsum(gh[:, :, sl], axis=2)          # [B, H, L, dk]
        diff = bcum[:, :, :, None, :] - bcum[:, :, None, :, :]  # [B,H,i,j,dk]
        causal = np.tril(np.ones((L, L), bool))
        decay = np.where(causal[None, None, :, :, None], np.exp(np.where(
            causal[None, None, :, :, None], diff, 0.0)), 0.0)
        A = np.einsum("bhid,bhjd,bhijd->bhij", qh[:, :, sl], kh[:, :, sl], decay)
        intra = np.einsum("bhij,bhje->bhie", A, vh[:, :, sl])
        readout = np.einsum("bhid,bhde->bhie", qh[:, :, sl] * np.exp(bcum),
                            S_in[:, :, n])
        o[:, sl] = np.transpose(intra + readout, (0, 2, 1, 3))
    if return_states:
        return o, U, a, S_in, S
    return o

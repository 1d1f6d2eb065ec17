"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
device copies of seeded inputs and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from recurrent_vision_token_gla_amd import gla

TOL = 5e-3  # max|o - o_ref| / max|o_ref|, fp16 operands with fp32 accumulation


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


def run_fwd(q, k, v, g, gh, gw, dirs, chunk):
    tq, tk, tv, tg = to_dev(q, k, v, g)
    o = gla.fwd(tq, tk, tv, tg, gh, gw, list(dirs), chunk=chunk)
    torch.cuda.synchronize()
    return o.double().cpu().numpy()


def rel_err(o, ref):
    return float(np.max(np.abs(o - ref)) / max(1e-30, np.max(np.abs(ref))))


def cosine(o, ref):
    a, b = o.ravel(), ref.ravel()
    return float(a @ b / max(1e-300, np.linalg.norm(a) * np.linalg.norm(b)))

"""The allocation-free forward (gla_fwd_noalloc, workspace in the library's
static scratch) against gla_fwd with a caller workspace: two calls in a row on
one GPU, the second smaller, each within the parity bar of the other and of the
float64 oracle; and the size limit of the scratch."""
import ctypes

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


def _pair(B, H, gh, gw, dk, dv, chunk, dirs, seed):
    x = W.make_inputs(B, gh * gw, H, dk, dv, np.float16, seed=seed)
    tq, tk, tv, tg = to_dev(*x)
    say(f"noalloc B={B} H={H} grid={gh}x{gw} dk={dk} dv={dv} chunk={chunk} dirs={dirs}")
    o_na = gla.fwd_noalloc(tq, tk, tv, tg, gh, gw, dirs, chunk)
    torch.cuda.synchronize()
    o_na = o_na.double().cpu().numpy()
    o_ws = gla.fwd(tq, tk, tv, tg, gh, gw, dirs, chunk)
    torch.cuda.synchronize()
    o_ws = o_ws.double().cpu().numpy()
    ref = oracle.gla_forward(*x, gh, gw, dirs)
    e_pair, e_ref = rel_err(o_na, o_ws), rel_err(o_na, ref)
    say(f"  vs gla_fwd {e_pair:.2e}  vs oracle {e_ref:.2e}  identical {np.array_equal(o_na, o_ws)}")
    assert e_pair <= TOL and e_ref <= TOL


def test_two_calls_in_a_row_second_smaller():
    _pair(1, 6, 40, 40, 64, 64, 64, [1], seed=8101)        # 1,600 tokens, 25-chunk chains
    _pair(2, 3, 12, 10, 64, 32, 32, [0, 3], seed=8102)     # 120 tokens, ragged tail


def test_scratch_size_limit_is_an_error():
    lib = gla.load()
    arr = (ctypes.c_int32 * 4)(0, 1, 2, 3)
    fake = 0x10000
    # 4 x 16 x 80x80 chunk 64: far more than 64 MiB of workspace; refused
    # before anything is launched or dereferenced
    assert gla.workspace_bytes(4, 16, 80, 80, 64, 64, 64) > (64 << 20)
    st = lib.gla_fwd_noalloc(fake, fake + 0x1000, fake + 0x2000, fake + 0x3000, fake + 0x4000,
                             4, 16, 80, 80, 64, 64, arr, 64, 0, None)
    assert st == gla.E_WORKSPACE
    assert b"64" in lib.gla_last_error_detail() or b"67108864" in lib.gla_last_error_detail()

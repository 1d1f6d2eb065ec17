"""The Python binding rejects tensors the kernels would misuse, before any
launch: an output of the wrong shape, dtype or layout, a non-contiguous
workspace, tensors on another device or in the wrong dtype; and it sizes a
workspace of any dtype in bytes."""
import numpy as np
import pytest
import torch

from gpu_util import to_dev
from recurrent_vision_token_gla_amd import gla
from recurrent_vision_token_gla_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def inputs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gla.load()
    x = W.make_inputs(2, 9 * 17, 2, 32, 64, np.float16, seed=490)
    return to_dev(*x)


def test_bad_outputs_are_rejected(inputs):
    q, k, v, g = inputs
    for out in (torch.empty(2, 9 * 17, 2, 32, dtype=torch.float16, device="cuda"),   # dk, not dv
                torch.empty_like(v, dtype=torch.float32),                              # dtype
                torch.empty(2, 2, 9 * 17, 64, dtype=torch.float16, device="cuda").transpose(1, 2),  # layout
                torch.empty_like(v, device="cpu")):                                    # device
        with pytest.raises(ValueError):
            gla.fwd(q, k, v, g, 9, 17, [0, 1], 16, out=out)
        with pytest.raises(ValueError):
            gla.fwd_state(q, k, v, g, 9, 17, [0, 1], 16, out=out)


def test_bad_workspaces_and_states_are_rejected(inputs):
    q, k, v, g = inputs
    ws = gla.alloc_workspace(2, 2, 9, 17, 32, 64, 16)
    wide = torch.zeros(2 * ws.numel(), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        gla.fwd(q, k, v, g, 9, 17, [0, 1], 16, workspace=wide[::2])  # not contiguous
    with pytest.raises(ValueError):
        gla.fwd(q, k, v, g, 9, 17, [0, 1], 16, workspace=ws.cpu())
    with pytest.raises(ValueError):
        gla.fwd_state(q, k, v, g, 9, 17, [0, 1], 16, s0=torch.zeros(2, 2, 64, 32, device="cuda"))
    with pytest.raises(ValueError):
        gla.fwd_state(q, k, v, g, 9, 17, [0, 1], 16, s0=torch.zeros(2, 2, 32, 64, device="cpu"))
    with pytest.raises(ValueError):
        gla.fwd(q, k.cpu(), v, g, 9, 17, [0, 1], 16)
    with pytest.raises(ValueError):
        gla.chunk_outputs(q, k, v, g, 9, 17, [0, 1], 16)  # no workspace to read S from


def test_workspace_of_any_dtype_is_sized_in_bytes(inputs):
    q, k, v, g = inputs
    ref = gla.fwd(q, k, v, g, 9, 17, [0, 1], 16)
    n = gla.workspace_bytes(2, 2, 9, 17, 32, 64, 16)
    ws32 = torch.zeros((n + 3) // 4, dtype=torch.float32, device="cuda")
    gla.workspace_init(ws32)  # prepared like the binding's own: same schedule, same bits
    o = gla.fwd(q, k, v, g, 9, 17, [0, 1], 16, workspace=ws32)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    gla.workspace_release(ws32)

"""Thin ctypes binding over libgla_mi355x.so (C ABI in include/gla.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the forward runs in the library's HIP kernels. There is
no fallback: if the library is not built, or a call fails, this module raises.
"""
from __future__ import annotations

import ctypes
import os
import weakref
from typing import Optional, Sequence, Union

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgla_mi355x.so")

L2R, R2L, T2B, B2T = 0, 1, 2, 3
F16, F32 = 0, 1
SCHED_AUTO, SCHED_SINGLE_PASS, SCHED_THREE_PHASE, SCHED_RUNS = 0, 1, 2, 3
CTRL_BYTES = 65536  # control words at the start of every workspace
OK, E_ARG, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_UNPREPARED = 0, -1, -2, -3, -4, -5
ERR_SPIN = 1  # sticky error bit: a single-pass wait ran out of its poll budget
ABI_VERSION = 5

# every symbol declared in include/gla.h
EXPORTS = ["gla_abi_version", "gla_fwd_workspace_bytes", "gla_workspace_layout", "gla_fwd",
           "gla_fwd_state", "gla_fwd_gated", "gla_fwd_schedule", "gla_auto_schedule", "gla_workspace_init",
           "gla_workspace_release", "gla_workspace_is_prepared", "gla_workspace_status",
           "gla_chunk_summaries", "gla_spatial_swiglu", "gla_state_scan", "gla_chunk_outputs", "gla_scan_perm",
           "gla_status_string", "gla_last_error_detail", "gla_fwd_noalloc"]

# With check_errors(True), every forward call made through this module waits
# for its stream and raises if the workspace's sticky error word is set
# (skipped while the stream is being captured into a graph). Off by default:
# the check synchronises.
_check_errors = False


def check_errors(on: bool) -> None:
    global _check_errors
    _check_errors = bool(on)

_lib = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_i32p = ctypes.POINTER(ctypes.c_int32)


class GLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.gla_status_string(status).decode()
        detail = lib.gla_last_error_detail().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail and status == E_HIP else ""))
        self.status = status


def load():
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing; run "
                           "__graft_entry__.build() or recurrent_vision_token_gla_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    lib.gla_abi_version.restype = _i32
    lib.gla_fwd_workspace_bytes.restype = _sz
    lib.gla_fwd_workspace_bytes.argtypes = [_i32] * 7
    lib.gla_workspace_layout.restype = _i32
    lib.gla_workspace_layout.argtypes = [_i32] * 7 + [ctypes.POINTER(_sz)] * 5
    lib.gla_fwd.restype = _i32
    lib.gla_fwd.argtypes = [_vp] * 5 + [_i32] * 6 + [_i32p, _i32, _i32, _vp, _sz, _vp]
    lib.gla_fwd_noalloc.restype = _i32
    lib.gla_fwd_noalloc.argtypes = [_vp] * 5 + [_i32] * 6 + [_i32p, _i32, _i32, _vp]
    lib.gla_fwd_state.restype = _i32
    lib.gla_fwd_state.argtypes = ([_vp] * 5 + [_i32] * 6 + [_i32p, _i32, _i32, _vp, _vp, _vp, _sz,
                                                            _vp])
    lib.gla_fwd_gated.restype = _i32
    lib.gla_fwd_gated.argtypes = ([_vp] * 6 + [ctypes.c_float, _vp] + [_i32] * 6 +
                                  [_i32p, _i32, _i32, _vp, _vp, _vp, _sz, _vp])
    lib.gla_fwd_schedule.restype = _i32
    lib.gla_fwd_schedule.argtypes = ([_vp] * 5 + [_i32] * 6 + [_i32p, _i32, _i32, _vp, _vp, _i32,
                                                               _vp, _sz, _vp])
    lib.gla_auto_schedule.restype = _i32
    lib.gla_auto_schedule.argtypes = [_i32] * 7
    lib.gla_workspace_init.restype = _i32
    lib.gla_workspace_init.argtypes = [_vp, _sz, _vp]
    lib.gla_workspace_release.restype = _i32
    lib.gla_workspace_release.argtypes = [_vp]
    lib.gla_workspace_is_prepared.restype = _i32
    lib.gla_workspace_is_prepared.argtypes = [_vp]
    lib.gla_workspace_status.restype = _i32
    lib.gla_workspace_status.argtypes = [_vp, _sz, ctypes.POINTER(ctypes.c_uint32), _i32, _vp]
    lib.gla_chunk_summaries.restype = _i32
    lib.gla_chunk_summaries.argtypes = [_vp] * 3 + [_i32] * 6 + [_i32p, _i32, _i32, _vp, _sz, _vp]
    lib.gla_state_scan.restype = _i32
    lib.gla_state_scan.argtypes = [_i32] * 7 + [_vp, _vp, _vp, _sz, _vp]
    lib.gla_chunk_outputs.restype = _i32
    lib.gla_chunk_outputs.argtypes = [_vp] * 5 + [_i32] * 6 + [_i32p, _i32, _i32, _vp, _sz, _vp]
    lib.gla_scan_perm.restype = _i32
    lib.gla_scan_perm.argtypes = [_vp, _i32, _i32, _i32, _vp]
    lib.gla_spatial_swiglu.restype = _i32
    lib.gla_spatial_swiglu.argtypes = [_vp] * 5 + [_i32] * 5 + [_vp]
    lib.gla_status_string.restype = ctypes.c_char_p
    lib.gla_status_string.argtypes = [_i32]
    lib.gla_last_error_detail.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != OK:
        raise GLAError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; use float16 or float32")


def _dirs(direction: Union[int, Sequence[int]], B: int):
    if isinstance(direction, int):
        vals = [direction] * B
    else:
        vals = [int(d) for d in direction]
        if len(vals) != B:
            raise ValueError(f"need one direction per batch element ({B}), got {len(vals)}")
    arr = (ctypes.c_int32 * max(1, B))(*vals)
    return arr


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def workspace_bytes(B, H, grid_h, grid_w, dk, dv, chunk=64) -> int:
    return int(load().gla_fwd_workspace_bytes(B, H, grid_h, grid_w, dk, dv, chunk))


def workspace_layout(B, H, grid_h, grid_w, dk, dv, chunk=64):
    """(off_U, off_a, off_S, off_scales, total) byte offsets inside the workspace."""
    vals = [_sz() for _ in range(5)]
    _check(load().gla_workspace_layout(B, H, grid_h, grid_w, dk, dv, chunk,
                                       *[ctypes.byref(x) for x in vals]), "gla_workspace_layout")
    return tuple(int(x.value) for x in vals)


def alloc_workspace(B, H, grid_h, grid_w, dk, dv, chunk=64, device=None,
                    prepare: bool = True) -> torch.Tensor:
    """A workspace for this problem. With prepare (the default) it is prepared
    for the single pass by gla_workspace_init, and released from the
    library's record of prepared workspaces when the tensor is collected."""
    n = workspace_bytes(B, H, grid_h, grid_w, dk, dv, chunk)
    ws = torch.empty(max(n, CTRL_BYTES), dtype=torch.uint8, device=device or "cuda")
    if prepare:
        workspace_init(ws)
        weakref.finalize(ws, load().gla_workspace_release, ws.data_ptr())
    return ws


def auto_schedule(B, H, grid_h, grid_w, dk, dv, chunk=64) -> int:
    """The schedule gla_fwd takes for this shape (SCHED_SINGLE_PASS or
    SCHED_THREE_PHASE)."""
    st = load().gla_auto_schedule(B, H, grid_h, grid_w, dk, dv, chunk)
    if st < 0:
        raise GLAError(st, "gla_auto_schedule")
    return st


def workspace_init(workspace: torch.Tensor, stream=None) -> None:
    """Prepare a workspace for the single pass: zero its control words (and
    the sticky error word) with a kernel and record it as prepared."""
    ws, nws = _ws(workspace, workspace.device)
    with _on_device(workspace.device):
        st = load().gla_workspace_init(ws, nws, _stream_ptr(stream))
    _check(st, "gla_workspace_init")


def workspace_release(workspace: torch.Tensor) -> None:
    """Drop a workspace from the library's record of prepared workspaces."""
    _check(load().gla_workspace_release(workspace.data_ptr()), "gla_workspace_release")


def is_prepared(workspace: torch.Tensor) -> bool:
    return bool(load().gla_workspace_is_prepared(workspace.data_ptr()))


def workspace_error(workspace: torch.Tensor, clear: bool = False, stream=None) -> int:
    """The sticky error word (bit 0: a single-pass wait ran out), read after
    the work queued on the stream; optionally cleared. Synchronises."""
    ws, nws = _ws(workspace, workspace.device)
    bits = ctypes.c_uint32(0)
    with _on_device(workspace.device):
        st = load().gla_workspace_status(ws, nws, ctypes.byref(bits), int(clear),
                                         _stream_ptr(stream))
    _check(st, "gla_workspace_status")
    return int(bits.value)


def _after_call(workspace: torch.Tensor, stream) -> None:
    """With check_errors on: raise if the call left the sticky error word set
    (only a prepared workspace runs the single pass and has one)."""
    if not _check_errors or torch.cuda.is_current_stream_capturing() or not is_prepared(workspace):
        return
    bits = workspace_error(workspace, clear=True, stream=stream)
    if bits:
        raise GLAError(E_HIP, f"single-pass wait ran out (error bits {bits:#x})")


def _ws(workspace: torch.Tensor, device):
    """(pointer, size in bytes) of a workspace: a contiguous device tensor on
    the inputs' device, of any dtype."""
    if not workspace.is_cuda or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _out(out: Optional[torch.Tensor], shape, dtype, device) -> torch.Tensor:
    """The caller's output tensor, checked (the kernels write all of it), or
    a new one."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype or out.device != device or \
            not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")
    return out


def _on_device(device):
    """Calls run on the inputs' device (its current stream unless one is given)."""
    return torch.cuda.device(device)


def _shapes(q, k, v, gk, grid_h, grid_w):
    for name, t in (("q", q), ("k", k), ("v", v), ("gk", gk)):
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a device tensor on q's device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, T, H, D]")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, T, H, D]")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, gk must share one dtype")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if T != grid_h * grid_w:
        raise ValueError(f"T={T} but grid is {grid_h}x{grid_w}")
    if k.shape != q.shape or gk.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("shape mismatch between q, k, gk [B,T,H,dk] and v [B,T,H,dv]")
    return B, T, H, dk, dv


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gk: torch.Tensor,
        grid_h: int, grid_w: int, direction: Union[int, Sequence[int]] = L2R,
        chunk: int = 64, out: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None, schedule: int = SCHED_AUTO) -> torch.Tensor:
    """o = key-only GLA forward along `direction` (int, or one per batch element)."""
    B, T, H, dk, dv = _shapes(q, k, v, gk, grid_h, grid_w)
    out = _out(out, (B, T, H, dv), q.dtype, q.device)
    if workspace is None:
        workspace = alloc_workspace(B, H, grid_h, grid_w, dk, dv, chunk, q.device)
    if schedule == SCHED_AUTO:
        ws, nws = _ws(workspace, q.device)
        with _on_device(q.device):
            st = load().gla_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(),
                                out.data_ptr(), B, H, grid_h, grid_w, dk, dv, _dirs(direction, B),
                                chunk, _dtype_code(q), ws, nws, _stream_ptr(stream))
        _check(st, "gla_fwd")
        _after_call(workspace, stream)
        return out
    return fwd_state(q, k, v, gk, grid_h, grid_w, direction, chunk, return_state=False, out=out,
                     workspace=workspace, stream=stream, schedule=schedule)


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gk: torch.Tensor,
                grid_h: int, grid_w: int, direction: Union[int, Sequence[int]] = L2R,
                chunk: int = 64, out: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The forward on the library's static scratch (gla_fwd_noalloc): no
    workspace is allocated; calls on one GPU must not overlap in time."""
    B, T, H, dk, dv = _shapes(q, k, v, gk, grid_h, grid_w)
    out = _out(out, (B, T, H, dv), q.dtype, q.device)
    with _on_device(q.device):
        st = load().gla_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(),
                                    out.data_ptr(), B, H, grid_h, grid_w, dk, dv,
                                    _dirs(direction, B), chunk, _dtype_code(q), _stream_ptr(stream))
    _check(st, "gla_fwd_noalloc")
    return out


def _state_ptr(t: Optional[torch.Tensor], B, H, dk, dv, name, device=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or \
            (device is not None and t.device != device):
        raise ValueError(f"{name} must be a contiguous float32 tensor on the inputs' device")
    if tuple(t.shape) != (B, H, dk, dv):
        raise ValueError(f"{name} must be [B, H, dk, dv] = {(B, H, dk, dv)}, got {tuple(t.shape)}")
    return t.data_ptr()


def fwd_state(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gk: torch.Tensor,
              grid_h: int, grid_w: int, direction: Union[int, Sequence[int]] = L2R,
              chunk: int = 64, s0: Optional[torch.Tensor] = None,
              s_final: Optional[torch.Tensor] = None, return_state: bool = True,
              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None, schedule: int = SCHED_AUTO):
    """Forward from the carried state s0 ([B, H, dk, dv] float32, None for
    zero); returns (o, S_T) with S_T written into s_final (allocated if None)
    when return_state, else o. schedule picks the kernel schedule."""
    B, T, H, dk, dv = _shapes(q, k, v, gk, grid_h, grid_w)
    out = _out(out, (B, T, H, dv), q.dtype, q.device)
    if return_state and s_final is None:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, H, grid_h, grid_w, dk, dv, chunk, q.device)
    ws, nws = _ws(workspace, q.device)
    p0 = _state_ptr(s0, B, H, dk, dv, "s0", q.device)
    pf = _state_ptr(s_final, B, H, dk, dv, "s_final", q.device)
    with _on_device(q.device):
        st = load().gla_fwd_schedule(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(),
                                     out.data_ptr(), B, H, grid_h, grid_w, dk, dv,
                                     _dirs(direction, B), chunk, _dtype_code(q), p0, pf, schedule,
                                     ws, nws, _stream_ptr(stream))
    _check(st, "gla_fwd_schedule")
    _after_call(workspace, stream)
    return (out, s_final) if return_state else out


def fwd_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gk: torch.Tensor,
              gate: torch.Tensor, norm_weight: torch.Tensor, eps: float, grid_h: int,
              grid_w: int, direction: Union[int, Sequence[int]] = L2R, chunk: int = 64,
              s0: Optional[torch.Tensor] = None, s_final: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """y = RMSNorm(o) * norm_weight * silu(gate) with o the forward (from s0,
    None for zero; S_T into s_final if given); gate [B, T, H, dv] in q's
    dtype, norm_weight [dv] float32."""
    B, T, H, dk, dv = _shapes(q, k, v, gk, grid_h, grid_w)
    if gate.shape != v.shape or gate.dtype != q.dtype or not gate.is_contiguous() or \
            gate.device != q.device:
        raise ValueError("gate must be a contiguous tensor shaped like v, in q's dtype and on its device")
    if norm_weight.dtype != torch.float32 or tuple(norm_weight.shape) != (dv,) or \
            norm_weight.device != q.device or not norm_weight.is_contiguous():
        raise ValueError("norm_weight must be a contiguous float32 [dv] tensor on q's device")
    out = _out(out, (B, T, H, dv), q.dtype, q.device)
    if workspace is None:
        workspace = alloc_workspace(B, H, grid_h, grid_w, dk, dv, chunk, q.device)
    ws, nws = _ws(workspace, q.device)
    p0 = _state_ptr(s0, B, H, dk, dv, "s0", q.device)
    pf = _state_ptr(s_final, B, H, dk, dv, "s_final", q.device)
    with _on_device(q.device):
        st = load().gla_fwd_gated(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(),
                                  gate.data_ptr(), norm_weight.data_ptr(), float(eps),
                                  out.data_ptr(), B, H, grid_h, grid_w, dk, dv,
                                  _dirs(direction, B), chunk, _dtype_code(q), p0, pf, ws, nws,
                                  _stream_ptr(stream))
    _check(st, "gla_fwd_gated")
    _after_call(workspace, stream)
    return out


def chunk_summaries(k, v, gk, grid_h, grid_w, direction=L2R, chunk=64, workspace=None,
                    stream=None) -> torch.Tensor:
    """Phase 1 only; returns the workspace holding U and a."""
    B, T, H, dk, dv = _shapes(k, k, v, gk, grid_h, grid_w)
    if workspace is None:
        workspace = alloc_workspace(B, H, grid_h, grid_w, dk, dv, chunk, k.device)
    ws, nws = _ws(workspace, k.device)
    with _on_device(k.device):
        st = load().gla_chunk_summaries(k.data_ptr(), v.data_ptr(), gk.data_ptr(), B, H, grid_h,
                                        grid_w, dk, dv, _dirs(direction, B), chunk, _dtype_code(k),
                                        ws, nws, _stream_ptr(stream))
    _check(st, "gla_chunk_summaries")
    return workspace


def state_scan(B, H, grid_h, grid_w, dk, dv, chunk, workspace, s0=None, s_final=None,
               stream=None) -> torch.Tensor:
    ws, nws = _ws(workspace, workspace.device)
    p0 = _state_ptr(s0, B, H, dk, dv, "s0", workspace.device)
    pf = _state_ptr(s_final, B, H, dk, dv, "s_final", workspace.device)
    with _on_device(workspace.device):
        st = load().gla_state_scan(B, H, grid_h, grid_w, dk, dv, chunk, p0, pf, ws, nws,
                                   _stream_ptr(stream))
    _check(st, "gla_state_scan")
    return workspace


def chunk_outputs(q, k, v, gk, grid_h, grid_w, direction=L2R, chunk=64, workspace=None,
                  out=None, stream=None) -> torch.Tensor:
    B, T, H, dk, dv = _shapes(q, k, v, gk, grid_h, grid_w)
    out = _out(out, (B, T, H, dv), q.dtype, q.device)
    if workspace is None:
        raise ValueError("chunk_outputs needs the workspace that holds the entering states")
    ws, nws = _ws(workspace, q.device)
    with _on_device(q.device):
        st = load().gla_chunk_outputs(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(),
                                      out.data_ptr(), B, H, grid_h, grid_w, dk, dv,
                                      _dirs(direction, B), chunk, _dtype_code(q), ws, nws,
                                      _stream_ptr(stream))
    _check(st, "gla_chunk_outputs")
    return out


def workspace_views(workspace: torch.Tensor, B, H, grid_h, grid_w, dk, dv, chunk=64):
    """Views of the stored arrays of the three phases: U [B,H,N,dk,dv] f16,
    a [B,H,N,dk] f32, S [B,H,N,dk,dv] f16, m [B,H,N,dk] f32 (the largest
    |U| of each row; a and m are the two halves of the stored (a, m) pairs)
    and the row scales sigS [B,H,N,dk] f32. The value of U row d is
    U[..., d, :] * row_scale(m[..., d]), that of S row d is
    S[..., d, :] * sigS[..., d]."""
    off_U, off_a, off_S, off_ss, _ = workspace_layout(B, H, grid_h, grid_w, dk, dv, chunk)
    N = -(-(grid_h * grid_w) // chunk)
    n_us = B * H * N * dk * dv
    n_a = B * H * N * dk
    U = workspace[off_U:off_U + 2 * n_us].view(torch.float16).view(B, H, N, dk, dv)
    pairs = workspace[off_a:off_a + 8 * n_a].view(torch.float32).view(B, H, N, dk, 2)
    S = workspace[off_S:off_S + 2 * n_us].view(torch.float16).view(B, H, N, dk, dv)
    sig_s = workspace[off_ss:off_ss + 4 * n_a].view(torch.float32).view(B, H, N, dk)
    return U, pairs[..., 0], S, pairs[..., 1], sig_s


def workspace_states(workspace: torch.Tensor, B, H, grid_h, grid_w, dk, dv, chunk=64):
    """(U, a, S) as float64 host arrays with the row scales applied."""
    U, a, S, m, ss = (x.double().cpu().numpy()
                      for x in workspace_views(workspace, B, H, grid_h, grid_w, dk, dv, chunk))
    return U * row_scale(m)[..., None], a, S * ss[..., None]


def row_scale(m):
    """The power-of-two scale a state row with largest magnitude m is stored
    divided by (the library's rule): 1 while m < 2^14, else the power of two
    that brings m into [2^13, 2^14)."""
    import numpy as np
    m = np.asarray(m, np.float32)
    e = ((m.view(np.uint32) >> 23) & 0xFF).astype(np.int64) - 140
    out = np.ldexp(np.float32(1), np.maximum(e, 0)).astype(np.float64)
    return np.where((e <= 0) | (e == 115), 1.0, out)


def scan_perm(grid_h: int, grid_w: int, direction: int, device="cuda", stream=None) -> torch.Tensor:
    """Device-computed scan order (raster index per scan position), int32."""
    perm = torch.empty(max(1, grid_h * grid_w), dtype=torch.int32, device=device)
    with _on_device(perm.device):
        st = load().gla_scan_perm(perm.data_ptr(), grid_h, grid_w, direction, _stream_ptr(stream))
    _check(st, "gla_scan_perm")
    return perm[:grid_h * grid_w]


def spatial_swiglu(a: torch.Tensor, u: torch.Tensor, weight: torch.Tensor,
                   bias: Optional[torch.Tensor], grid_h: int, grid_w: int,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """h = silu(a) * (3x3 depthwise conv of u on the grid + bias); a, u [B, T, F]
    (float16 or float32, contiguous), weight [F, 3, 3] and bias [F] float32."""
    for name, t in (("a", a), ("u", u)):
        if not t.is_cuda or t.device != u.device or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous [B, T, F] device tensor on u's device")
    if a.shape != u.shape or a.dtype != u.dtype:
        raise ValueError("a and u must share shape and dtype")
    B, T, Fc = u.shape
    if T != grid_h * grid_w:
        raise ValueError(f"T={T} but grid is {grid_h}x{grid_w}")
    if weight.dtype != torch.float32 or tuple(weight.shape) != (Fc, 3, 3) or \
            not weight.is_contiguous() or weight.device != u.device:
        raise ValueError("weight must be a contiguous float32 [F, 3, 3] tensor on u's device")
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (Fc,)
                             or bias.device != u.device or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [F] tensor on u's device")
    out = _out(out, tuple(u.shape), u.dtype, u.device)
    with _on_device(u.device):
        st = load().gla_spatial_swiglu(a.data_ptr(), u.data_ptr(), weight.data_ptr(),
                                       None if bias is None else bias.data_ptr(), out.data_ptr(),
                                       B, grid_h, grid_w, Fc, _dtype_code(u), _stream_ptr(stream))
    _check(st, "gla_spatial_swiglu")
    return out

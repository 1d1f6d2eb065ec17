"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/gla.h declares, and rejects bad arguments on the host before any HIP
call. No call here launches a kernel."""
import ctypes
import os
import re

import pytest

from recurrent_vision_token_gla_amd import gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(gla_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gla.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return gla.load()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(gla.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.gla_abi_version() == gla.ABI_VERSION == 5
    for st in (0, -1, -2, -3, -4, 7):
        s = lib.gla_status_string(st)
        assert s and isinstance(s, bytes)
    assert lib.gla_status_string(-3).startswith(b"GLA_E_WORKSPACE")
    assert lib.gla_last_error_detail() == b""


def test_workspace_bytes(lib):
    # control words (64 KiB) + U (f16) + (a, U row scale) pairs (2 x f32; twice
    # as many for dv = 64, whose single pass may split the value columns in
    # two) + S (f16) + single-pass segment pairs (2 x f32) + S row scales
    # (f32), each padded to 256 bytes
    B, H, gh, gw, dk, dv, C = 1, 6, 40, 40, 64, 64, 64
    N = 25
    units = B * H * N
    expect = (65536 + units * dk * dv * 2 + 2 * units * dk * 8 + units * dk * dv * 2
              + units * dk * 8 + units * dk * 4)
    assert gla.workspace_bytes(B, H, gh, gw, dk, dv, C) == expect
    units32 = 1 * 1 * 4  # 8x8 grid, chunk 16, dv = 32: one set of pairs
    assert gla.workspace_bytes(1, 1, 8, 8, 32, 32, 16) == (
        65536 + units32 * 32 * 32 * 2 + units32 * 32 * 8 + units32 * 32 * 32 * 2
        + units32 * 32 * 8 + units32 * 32 * 4)
    assert gla.workspace_bytes(0, H, gh, gw, dk, dv, C) == 0
    assert gla.workspace_bytes(1, 1, 5, 7, 32, 32, 16) > 0
    assert gla.workspace_bytes(1, 1, 8, 8, 48, 32, 16) == 0  # unsupported dk
    off_U, off_a, off_S, off_sc, total = gla.workspace_layout(B, H, gh, gw, dk, dv, C)
    assert off_U == 65536 and off_a % 256 == 0 and off_S % 256 == 0 and total == expect
    assert off_sc % 256 == 0 and off_sc + units * dk * 4 == total


FAKE = 0x10000  # 256-aligned, never dereferenced: every call below fails validation first


def _fwd(lib, q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, g=FAKE + 0x3000, o=FAKE + 0x4000,
         B=1, H=1, gh=4, gw=4, dk=32, dv=32, dirs=(0,), chunk=16, dtype=0, ws=FAKE + 0x5000,
         ws_bytes=0):
    arr = (ctypes.c_int32 * max(1, len(dirs)))(*dirs) if dirs is not None else None
    return lib.gla_fwd(q, k, v, g, o, B, H, gh, gw, dk, dv, arr, chunk, dtype, ws, ws_bytes, None)


def test_argument_errors_before_any_launch(lib):
    E_ARG, E_UNS, E_WS = gla.E_ARG, gla.E_UNSUPPORTED, gla.E_WORKSPACE
    assert _fwd(lib, q=None) == E_ARG
    assert _fwd(lib, o=None) == E_ARG
    assert _fwd(lib, q=FAKE + 2) == E_ARG            # misaligned
    assert _fwd(lib, B=-1) == E_ARG
    assert _fwd(lib, gh=-3) == E_ARG
    assert _fwd(lib, dtype=5) == E_ARG
    assert _fwd(lib, dk=48) == E_UNS
    assert _fwd(lib, dv=128) == E_UNS
    assert _fwd(lib, chunk=48) == E_UNS
    assert _fwd(lib, dirs=(4,)) == E_ARG
    assert _fwd(lib, dirs=(-1,)) == E_ARG
    assert _fwd(lib, dirs=None) == E_ARG
    assert _fwd(lib, o=FAKE) == E_ARG                 # o aliases q
    assert _fwd(lib, ws=None) == E_ARG
    assert _fwd(lib, ws=FAKE + 0x5010) == E_ARG       # workspace not 256-aligned
    need = gla.workspace_bytes(1, 1, 4, 4, 32, 32, 16)
    assert _fwd(lib, ws_bytes=need - 1) == E_WS
    assert _fwd(lib, B=2, dirs=(0, 9), ws_bytes=10 ** 9) == E_ARG
    assert lib.gla_last_error_detail() == b""


def _fwd_state(lib, s0=None, sf=None, q=FAKE, o=FAKE + 0x4000, ws=FAKE + 0x5000, ws_bytes=10 ** 6):
    arr = (ctypes.c_int32 * 1)(0)
    return lib.gla_fwd_state(q, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, o, 1, 1, 4, 4, 32, 32,
                             arr, 16, 0, s0, sf, ws, ws_bytes, None)


def test_carried_state_argument_errors(lib):
    assert _fwd_state(lib, s0=FAKE + 0x6002) == gla.E_ARG      # misaligned s0
    assert _fwd_state(lib, sf=FAKE + 0x6004) == gla.E_ARG      # misaligned s_final
    assert _fwd_state(lib, sf=FAKE) == gla.E_ARG               # s_final aliases q
    assert _fwd_state(lib, sf=FAKE + 0x4000) == gla.E_ARG      # s_final aliases o
    assert _fwd_state(lib, sf=FAKE + 0x5000) == gla.E_ARG      # s_final aliases the workspace
    assert _fwd_state(lib, q=None, s0=FAKE + 0x6000) == gla.E_ARG
    assert _fwd_state(lib, s0=FAKE + 0x6000, ws_bytes=1) == gla.E_WORKSPACE
    # empty problem: nothing examined
    arr = (ctypes.c_int32 * 1)(0)
    assert lib.gla_fwd_state(None, None, None, None, None, 0, 1, 4, 4, 32, 32, arr, 16, 0, None,
                             None, None, 0, None) == gla.OK


def test_empty_problems_are_noops(lib):
    # nothing to compute: returns OK and does not look at the pointers
    assert _fwd(lib, q=None, k=None, v=None, g=None, o=None, ws=None, B=0, dirs=None) == gla.OK
    assert _fwd(lib, q=None, k=None, v=None, g=None, o=None, ws=None, H=0) == gla.OK
    assert _fwd(lib, q=None, k=None, v=None, g=None, o=None, ws=None, gh=0) == gla.OK
    assert lib.gla_scan_perm(None, 0, 5, 0, None) == gla.OK


def test_phase_entry_points_validate(lib):
    arr = (ctypes.c_int32 * 1)(0)
    assert lib.gla_chunk_summaries(None, FAKE, FAKE, 1, 1, 4, 4, 32, 32, arr, 16, 0, FAKE, 10 ** 6,
                                   None) == gla.E_ARG
    assert lib.gla_state_scan(1, 1, 4, 4, 32, 32, 16, None, None, FAKE, 1, None) == gla.E_WORKSPACE
    assert lib.gla_state_scan(1, 1, 4, 4, 32, 32, 24, None, None, FAKE, 10 ** 6,
                              None) == gla.E_UNSUPPORTED
    assert lib.gla_state_scan(1, 1, 4, 4, 32, 32, 16, FAKE + 4, None, FAKE, 10 ** 6,
                              None) == gla.E_ARG          # misaligned s0
    assert lib.gla_state_scan(1, 1, 4, 4, 32, 32, 16, None, FAKE + 8, FAKE, 10 ** 6,
                              None) == gla.E_ARG          # misaligned s_final
    assert lib.gla_chunk_outputs(FAKE, FAKE + 0x100, FAKE + 0x200, FAKE + 0x300, FAKE + 0x100, 1, 1,
                                 4, 4, 32, 32, arr, 16, 0, FAKE, 10 ** 6, None) == gla.E_ARG
    assert lib.gla_scan_perm(FAKE, 4, 4, 7, None) == gla.E_ARG
    assert lib.gla_scan_perm(None, 4, 4, 0, None) == gla.E_ARG
    assert lib.gla_scan_perm(FAKE + 1, 4, 4, 0, None) == gla.E_ARG


def test_schedule_and_workspace_init_validate(lib):
    arr = (ctypes.c_int32 * 1)(0)
    big = 10 ** 12  # never allocated: every call below fails before any launch

    def sched(schedule, gh=4, gw=4, chunk=16, ws_bytes=big):
        return lib.gla_fwd_schedule(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000,
                                    FAKE + 0x4000, 1, 1, gh, gw, 32, 32, arr, chunk, 0, None, None,
                                    schedule, FAKE + 0x5000, ws_bytes, None)
    assert sched(4) == gla.E_ARG
    assert sched(-1) == gla.E_ARG
    # runs of chunks: 64-token chunks only
    assert sched(gla.SCHED_RUNS, chunk=16) == gla.E_UNSUPPORTED
    assert sched(gla.SCHED_RUNS, gh=8, gw=8, chunk=64) == gla.E_UNPREPARED
    # 4097 chunks in one chain: more than the single pass waits on
    assert sched(gla.SCHED_SINGLE_PASS, gh=4097, gw=16, chunk=16) == gla.E_UNSUPPORTED
    assert sched(gla.SCHED_SINGLE_PASS, ws_bytes=100) == gla.E_WORKSPACE
    # a workspace that gla_workspace_init has not prepared: no single pass
    assert sched(gla.SCHED_SINGLE_PASS) == gla.E_UNPREPARED
    assert b"gla_workspace_init" in lib.gla_last_error_detail()
    assert lib.gla_workspace_init(None, 1 << 20, None) == gla.E_ARG
    assert lib.gla_workspace_init(FAKE + 0x10, 1 << 20, None) == gla.E_ARG
    assert lib.gla_workspace_init(FAKE, 65535, None) == gla.E_WORKSPACE


def test_workspace_record_and_status_validate(lib):
    assert lib.gla_workspace_is_prepared(FAKE) == 0
    assert lib.gla_workspace_is_prepared(None) == 0
    assert lib.gla_workspace_release(None) == gla.E_ARG
    assert lib.gla_workspace_release(FAKE) == gla.OK  # not recorded: nothing to drop
    bits = ctypes.c_uint32(7)
    assert lib.gla_workspace_status(None, 1 << 20, ctypes.byref(bits), 0, None) == gla.E_ARG
    assert lib.gla_workspace_status(FAKE + 0x10, 1 << 20, ctypes.byref(bits), 0, None) == gla.E_ARG
    assert lib.gla_workspace_status(FAKE, 1 << 20, None, 0, None) == gla.E_ARG
    assert lib.gla_workspace_status(FAKE, 100, ctypes.byref(bits), 0, None) == gla.E_WORKSPACE
    assert bits.value == 7  # untouched by failed calls
    assert lib.gla_status_string(gla.E_UNPREPARED).startswith(b"GLA_E_UNPREPARED")


def test_state_overlap_validates(lib):
    arr = (ctypes.c_int32 * 1)(0)
    st = FAKE + 0x10000  # state [1][1][32][32] float = 4 KiB

    def state(s0, sf):
        return lib.gla_fwd_state(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000,
                                 FAKE + 0x4000, 1, 1, 4, 4, 32, 32, arr, 16, 0, s0, sf,
                                 FAKE + 0x5000, 100, None)
    # s_final overlapping s0 without being s0 is rejected before the workspace
    # check; s_final == s0 passes it (and fails on the tiny workspace)
    assert state(st, st + 16) == gla.E_ARG
    assert state(st, st) == gla.E_WORKSPACE
    assert state(st, st + 4096) == gla.E_WORKSPACE


def test_auto_schedule(lib):
    # chains of up to 64 chunks: single pass at any grid; 100 and 144: on
    # large grids only (chunk-heads x N from 1.2e6); longer: three phases
    assert gla.auto_schedule(1, 6, 40, 40, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(4, 6, 40, 40, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(8, 12, 40, 40, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(1, 6, 56, 56, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(4, 12, 56, 56, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(1, 6, 64, 64, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(8, 12, 64, 64, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(1, 6, 80, 80, 64, 64, 64) == gla.SCHED_THREE_PHASE
    assert gla.auto_schedule(4, 16, 80, 80, 64, 64, 64) == gla.SCHED_THREE_PHASE
    assert gla.auto_schedule(8, 16, 80, 80, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(1, 6, 96, 96, 64, 64, 64) == gla.SCHED_THREE_PHASE
    assert gla.auto_schedule(4, 16, 96, 96, 64, 64, 64) == gla.SCHED_SINGLE_PASS
    assert gla.auto_schedule(4, 16, 128, 128, 64, 64, 64) == gla.SCHED_THREE_PHASE
    assert gla.auto_schedule(1, 1, 4097, 16, 32, 32, 16) == gla.SCHED_THREE_PHASE
    # more chains than the control words hold in one launch: three phases
    assert gla.auto_schedule(1024, 64, 8, 8, 32, 32, 16) == gla.SCHED_THREE_PHASE
    assert lib.gla_auto_schedule(1, 1, 4, 4, 48, 32, 16) == gla.E_UNSUPPORTED
    assert lib.gla_auto_schedule(-1, 1, 4, 4, 32, 32, 16) == gla.E_ARG


def test_gated_forward_validates(lib):
    arr = (ctypes.c_int32 * 1)(0)

    def gated(gate=FAKE + 0x6000, w=FAKE + 0x7000, eps=1e-6, y=FAKE + 0x4000):
        return lib.gla_fwd_gated(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, gate, w,
                                 ctypes.c_float(eps), y, 1, 1, 4, 4, 32, 32, arr, 16, 0, None,
                                 None, FAKE + 0x5000, 10 ** 6, None)
    assert gated(gate=None) == gla.E_ARG
    assert gated(gate=FAKE + 0x6008) == gla.E_ARG     # misaligned gate
    assert gated(w=None) == gla.E_ARG
    assert gated(w=FAKE + 0x7004) == gla.E_ARG        # misaligned weight
    assert gated(eps=-1.0) == gla.E_ARG
    assert gated(y=FAKE + 0x6000) == gla.E_ARG        # output is the gate buffer
    assert gated(y=FAKE) == gla.E_ARG                 # output is q

"""CPU oracle for GTR's key-only gated linear attention forward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
anything in this package: only the tests, the smoke check and the CPU
baseline leg of the benchmark do. It shares no code with the HIP path; the
two meet only at the seeded input generators, which hold none of the
forward's arithmetic.

Contents:
  scan_order  -- the four scan orders from plain numpy grid operations
  recurrence  -- the token-by-token float64 recurrence (C with OpenMP, and a
                 numpy twin), plus the raster <-> scan gather/scatter
  chunkwise   -- a float64 model of the chunked schedule (summaries, boundary
                 scan, outputs), checked against the recurrence
  epilogue    -- the block's RMS-normalised, SiLU-gated output and the
                 Spatial SwiGLU mixer (3x3 depthwise convolution on the
                 value branch times SiLU of the gate branch)

Every function here is pinned by the CPU tests (tests/test_oracle_*.py)
against hand-derived fixtures, a brute-force closed form, textbook special
cases and invariants.
"""
from .scan_order import B2T, L2R, R2L, T2B, scan_order, to_raster, to_scan
from .recurrence import gla_forward, oracle_threads, recurrence_c, recurrence_numpy
from .chunkwise import chunkwise
from .epilogue import rmsnorm_gate, silu, spatial_swiglu

__all__ = ["L2R", "R2L", "T2B", "B2T", "scan_order", "to_scan", "to_raster",
           "gla_forward", "recurrence_c", "recurrence_numpy", "oracle_threads",
           "chunkwise", "rmsnorm_gate", "silu", "spatial_swiglu"]

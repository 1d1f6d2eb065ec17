"""The bench's roofline accounting (CPU only): algorithmic bytes and flops per
token-head and per kernel launch, and the fields of the summary it prints."""
import importlib.util
import json
import os

import pytest

from recurrent_vision_token_gla_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_whole_forward_bytes_and_flops_per_token_head(bench):
    w = W.WORKLOADS[1]  # 64/64, chunk 64, fp16
    # read q, k, gk (dk each) and v (dv), write o (dv): 5 rows of 64 halves
    assert bench.per_unit_bytes(w) == 640
    th = w.B * w.T * w.H
    # 2 dk dv (summary) + 2 dk dv (readout) + C (dk + dv) (causal halves)
    assert bench.phase_flops(w)["single_pass"] == th * 24576
    assert bench.phase_bytes(w)["single_pass"] == th * 640


def test_three_phase_bytes_per_launch(bench):
    w = W.WORKLOADS[2]
    th, ch = w.B * w.T * w.H, w.B * w.H * (w.T // w.chunk)
    pb = bench.phase_bytes(w)
    # k, gk, v in; U and the (a, row max) pairs out
    assert pb["summaries"] == th * 3 * 128 + ch * (8192 + 512)
    # U and the pairs in; S and its row scales out
    assert pb["scan"] == ch * (8192 + 512 + 8192 + 256)
    # q, k, gk, v in, o out; S and its row scales in
    assert pb["outputs"] == th * 5 * 128 + ch * (8192 + 256)
    assert pb["runs"] == pb["single_pass"]
    fl = bench.phase_flops(w)
    assert fl["summaries"] + fl["outputs"] == fl["single_pass"] and fl["scan"] == 0


def test_fp32_rows_count_four_bytes(bench):
    w = W.WORKLOADS[0]  # 32/32 fp32
    assert bench.per_unit_bytes(w) == (3 * 32 + 2 * 32) * 4


def test_summary_line_fields(bench):
    w = W.WORKLOADS[1]
    res = dict(ms_per_step=0.0572, warm_ms_per_step=0.0537, lat_us=[60.0, 61.0],
               phase_us={"single_pass": 12.7, "summaries": 4.3, "scan": 2.9, "outputs": 6.4},
               phase_warm_us={"single_pass": 12.2, "summaries": 4.0, "scan": 2.9, "outputs": 5.9},
               used=["single_pass"], schedule="single_pass", sets=22, set_bytes=24576000)
    s = bench.summarize(w, res)
    json.dumps(s)
    assert s["value"] == pytest.approx(4 * 1600 / 57.2e-6)
    r = s["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(6144000 / 12.7e-6 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    m = s["mfma_roofline"]
    assert m["unit"] == "TFLOP/s" and m["achieved"] == pytest.approx(9600 * 24576 / 12.7e-6 / 1e12)
    assert s["warm"]["call_us"] == pytest.approx(53.7 / 4)

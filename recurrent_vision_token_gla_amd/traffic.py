"""HBM traffic per launch from rocprofv3 counter runs, merged into
profiles/traffic.json (which bench.py reads for its `traffic` fields).

Two counter passes over one bench run each (FETCH_SIZE, then WRITE_SIZE; the
counters read KiB per dispatch), with a plain device copy of known size run
first (bench.py --calibrate-copy-mib M): each counter is scaled by what it
reads for that copy, so bytes = FETCH * (copy bytes / copy FETCH) +
WRITE * (copy bytes / copy WRITE). Per kernel class the dispatches are
averaged; a dispatch's value is the sum of its rows (rocprofv3 may report a
counter per hardware instance).

  python -m recurrent_vision_token_gla_amd.traffic --workload 4 \
      --fetch gpurun_out/tr_FETCH_SIZE --write gpurun_out/tr_WRITE_SIZE \
      --copy-mib 256 [--json profiles/traffic.json]
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import importlib.util
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kernel_class(name: str) -> str | None:
    """The bench's name for a kernel of this library, None for others."""
    if "copyBuffer" in name:
        return "copy"
    if "chunk_kernel" in name:
        # template arguments <DK, DV, C, InT, kFused, kGate, GR>: the flags
        # mangle as Lb<0|1>ELb<0|1>E and GR (chunks per workgroup) as Li<GR>E;
        # demangled, "true, false, 4>"
        m = (re.search(r"Lb([01])ELb([01])ELi(\d+)E", name)
             or re.search(r"(true|false), (true|false), (\d+)>", name))
        if m and int(m.group(3)) > 1:
            return "runs"
        return "single_pass" if m and m.group(1) in ("1", "true") else "outputs"
    if "summary_kernel" in name:
        return "summaries"
    if "scan_serial_kernel" in name or "scan_kernel" in name:
        return "scan"
    if "runs_kernel" in name:
        return "runs"
    return None


def per_dispatch(d: str, counter: str) -> dict[str, list[float]]:
    """Counter value (summed over its rows) of every dispatch, by kernel class."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    tot: dict[tuple[str, str], float] = collections.defaultdict(float)
    cls: dict[tuple[str, str], str] = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                c = kernel_class(r["Kernel_Name"])
                if c is None:
                    continue
                key = (f, r["Dispatch_Id"])
                tot[key] += float(r["Counter_Value"])
                cls[key] = c
    out: dict[str, list[float]] = collections.defaultdict(list)
    for key, v in tot.items():
        out[cls[key]].append(v)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--workload", type=int, required=True)
    ap.add_argument("--fetch", required=True, help="rocprofv3 output dir of the FETCH_SIZE pass")
    ap.add_argument("--write", required=True, help="rocprofv3 output dir of the WRITE_SIZE pass")
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    args = ap.parse_args()

    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    from recurrent_vision_token_gla_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    fetch = per_dispatch(args.fetch, "FETCH_SIZE")
    write = per_dispatch(args.write, "WRITE_SIZE")
    copy_kib = args.copy_mib * 1024.0
    if not fetch.get("copy") or not write.get("copy"):
        raise SystemExit("the calibration copy is missing from the counter runs")
    # the copy is the largest dispatch of its class in each run
    ff = copy_kib / max(fetch["copy"])
    wf = copy_kib / max(write["copy"])
    pb = bench.phase_bytes(w)
    sha = bench.source_sha()
    entries = []
    for k in ("single_pass", "runs", "summaries", "scan", "outputs"):
        if not fetch.get(k) or not write.get(k):
            continue
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write[k]) / len(write[k])
        hbm = int(round((fk * ff + wk * wf) * 1024))
        entries.append({"kernel": k, "workload": w.name, "source_sha": sha,
                        "dispatches": len(fetch[k]),
                        "fetch_kib_per_dispatch": round(fk, 1),
                        "write_kib_per_dispatch": round(wk, 1),
                        "hbm_bytes_per_launch": hbm,
                        "algorithmic_bytes_per_launch": pb[k],
                        "ratio": round(hbm / pb[k], 3)})
    try:
        with open(args.json) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    rec["about"] = ("HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (one "
                    "pass each, KiB per dispatch), each scaled by what the same counter reads for "
                    "a plain device copy of known size in the same run; written by "
                    "recurrent_vision_token_gla_amd/traffic.py")
    rec.setdefault("calibration", {})[w.name] = {"copy_bytes": args.copy_mib << 20,
                                                  "fetch_factor": round(ff, 4),
                                                  "write_factor": round(wf, 4)}
    keep = [e for e in rec.get("entries", []) if e.get("workload") != w.name]
    rec["entries"] = keep + entries
    with open(args.json, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    for e in entries:
        print(f"{w.name} {e['kernel']:12s} fetch {e['fetch_kib_per_dispatch']:12.1f} KiB  write "
              f"{e['write_kib_per_dispatch']:12.1f} KiB  -> {e['hbm_bytes_per_launch']:13d} B "
              f"({e['ratio']:.2f}x of {e['algorithmic_bytes_per_launch']})")
    print(f"factors: fetch {ff:.4f} write {wf:.4f}")


if __name__ == "__main__":
    main()

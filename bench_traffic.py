#!/usr/bin/env python3
"""HBM traffic of the dominant GEMM kernel from rocprofv3 counter runs.

Reads four ``rocprofv3 --pmc`` output folders (CSV):
  --gemm-fetch / --gemm-write : ``bench.py --steps 1 --warmup 0 --layers 1``
                                under FETCH_SIZE, then under WRITE_SIZE;
  --copy-fetch / --copy-write : ``bench.py --calibrate-copy`` under the same
                                counters (a plain 1 GiB device copy).
FETCH_SIZE / WRITE_SIZE are KiB per dispatch.  Each is scaled by what the same
counter reads for the copy of known size, so a GEMM launch's HBM bytes =
fetch / (copy fetch per byte) + write / (copy write per byte).  Prints the
markdown summary that bench.py reads (``- `key`: `value``` lines), including
the hash of the GEMM sources the counters were taken on.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (source hash and file locations)
import synth  # noqa: E402  (the dense shapes)

KERNEL = "k_gemm_pp<0, false>"  # the dense block-scaled GEMM of the M=8192 linears


def per_dispatch(folder: str, counter: str, name_filter) -> list[float]:
    paths = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    vals = collections.defaultdict(float)
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and name_filter(r["Kernel_Name"]):
                    vals[(p, r["Dispatch_Id"])] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for the kernel in {folder}")
    return list(vals.values())


def main():
    ap = argparse.ArgumentParser()
    for k in ("gemm-fetch", "gemm-write", "copy-fetch", "copy-write"):
        ap.add_argument(f"--{k}", required=True)
    ap.add_argument("--command", action="append", default=[],
                    help="command lines that produced the folders (for the summary)")
    a = ap.parse_args()

    def is_gemm(n):
        return KERNEL in n

    def is_copy(n):
        return "copy" in n.lower()

    gf = per_dispatch(a.gemm_fetch, "FETCH_SIZE", is_gemm)
    gw = per_dispatch(a.gemm_write, "WRITE_SIZE", is_gemm)
    cf = per_dispatch(a.copy_fetch, "FETCH_SIZE", is_copy)
    cw = per_dispatch(a.copy_write, "WRITE_SIZE", is_copy)
    copy_bytes = float(1 << 30)
    f_fetch = (sum(cf) / len(cf)) * 1024.0 / copy_bytes
    f_write = (sum(cw) / len(cw)) * 1024.0 / copy_bytes
    fetch_kib = sum(gf) / len(gf)
    write_kib = sum(gw) / len(gw)
    traffic = fetch_kib * 1024.0 / f_fetch + write_kib * 1024.0 / f_write

    alg = 0.0
    for N, K in synth.DENSE_SHAPES.values():
        M = 8192
        alg += M * K + N * K + 4 * (M * (K // 128) + (N // 128) * (K // 128)) + 2 * M * N
    alg /= len(synth.DENSE_SHAPES)

    print("# HBM traffic: block-scaled GEMM `k_gemm_pp<0, false>`, the M=8192 dense linears\n")
    print("Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each in its own "
          "rocprofv3 run, over bench.py's one timed and one instrumented step of the four "
          "M=8192 linears (qkv, o, gate_up, down; two launches each), scaled by the same "
          "counters over a plain 1 GiB device copy.\n")
    print("Commands (from the repository root `R` on one MI355X, after "
          "`cd /tmp && export TMPDIR=/tmp`):\n")
    print("```")
    for c in a.command:
        print(c)
    print("```\n")
    print(f"- `gemm_dispatches`: `{len(gf)}`")
    print(f"- `fetch_kib_per_launch`: `{fetch_kib:.1f}`")
    print(f"- `write_kib_per_launch`: `{write_kib:.1f}`")
    print(f"- `copy_fetch_factor`: `{f_fetch:.4f}`")
    print(f"- `copy_write_factor`: `{f_write:.4f}`")
    print(f"- `traffic_bytes_per_launch`: `{traffic:.0f}`")
    print(f"- `algorithmic_bytes_per_launch`: `{alg:.0f}`")
    print(f"- `traffic_over_algorithmic`: `{traffic / alg:.3f}`")
    print(f"- `source_sha256`: `{bench.gemm_source_hash()}`")
    print("\nPer-launch values are means over the dispatches of the kernel (two per "
          "linear shape, so the mean matches the per-launch mean over a 36-layer step). "
          "The factors are counter bytes per true byte of the copy; traffic divides the "
          "GEMM's counter bytes by them.")


if __name__ == "__main__":
    main()

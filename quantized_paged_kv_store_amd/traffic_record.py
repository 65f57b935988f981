"""Write a profiles/*_traffic.json record from two rocprofv3 counter runs.

The HBM traffic a kernel causes per launch is measured with two
`rocprofv3 --pmc` runs of the same program, one for FETCH_SIZE and one for
WRITE_SIZE (KiB per dispatch), and scaled by what the same counters read for a
plain device copy of known size (`bench.py --copy-ref`: 1 GiB read, 1 GiB
written by `__amd_rocclr_copyBuffer`). The record also holds the SHA-256 of
the kernel's source files; `bench.py` reports the traffic only while those
sources still hash to it, so a record never outlives the code it measured.

    python -m quantized_paged_kv_store_amd.traffic_record --out profiles/NAME_traffic.json \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --kernel SUBSTRING \\
        --sources FILE[,FILE...] --kernel-desc TEXT --workload-desc TEXT

DIR is a rocprofv3 output directory holding run_counter_collection.csv.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def _rows(d: str, counter: str):
    with open(os.path.join(d, "run_counter_collection.csv")) as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def kernel_median(d: str, counter: str, substring: str) -> tuple[float, int]:
    """Median counter value over the dispatches whose kernel name holds
    `substring`, and their number."""
    v = [float(r["Counter_Value"]) for r in _rows(d, counter) if substring in r["Kernel_Name"]]
    if not v:
        raise SystemExit(f"{d}: no {counter} rows for kernels matching {substring!r}")
    return statistics.median(v), len(v)


def copy_median(d: str, counter: str) -> float:
    """Median over the reference copies: the copy-kernel dispatches with the
    largest grid (the 1 GiB copies, not the program's small ones)."""
    rows = [r for r in _rows(d, counter) if COPY_KERNEL in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"{d}: no {counter} rows for {COPY_KERNEL}")
    g = max(int(r["Grid_Size"]) for r in rows)
    return statistics.median(float(r["Counter_Value"]) for r in rows if int(r["Grid_Size"]) == g)


def sources_sha256(sources: list[str]) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    for a in ("--out", "--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--sources",
              "--kernel-desc", "--workload-desc"):
        ap.add_argument(a, required=True)
    ap.add_argument("--note", default="")
    args = ap.parse_args()
    fetch, nf = kernel_median(args.fetch, "FETCH_SIZE", args.kernel)
    write, nw = kernel_median(args.write, "WRITE_SIZE", args.kernel)
    cf, cw = copy_median(args.copy_fetch, "FETCH_SIZE"), copy_median(args.copy_write, "WRITE_SIZE")
    kib = COPY_BYTES / 1024
    rec = {
        "kernel": args.kernel_desc,
        "workload": args.workload_desc,
        "sources_sha256": sources_sha256(args.sources.split(",")),
        "sources": args.sources.split(","),
        "fetch_size_kib_per_dispatch": fetch,
        "write_size_kib_per_dispatch": write,
        "dispatches": {"fetch": nf, "write": nw},
        "copy_reference": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "fetch_size_kib": cf,
                           "write_size_kib": cw},
        "fetch_scale": round(kib / cf, 4),
        "write_scale": round(kib / cw, 4),
        "note": ("kernel counters are medians over the matching dispatches, scaled by known bytes / counter "
                 "reading of a plain 1 GiB device copy" + (f"; {args.note}" if args.note else "")),
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    mb = 1024 * (fetch * rec["fetch_scale"] + write * rec["write_scale"]) / 1e6
    print(f"{args.out}: {fetch:.1f} KiB fetched, {write:.1f} KiB written per dispatch "
          f"(x{rec['fetch_scale']}, x{rec['write_scale']}) = {mb:.1f} MB per launch")


if __name__ == "__main__":
    main()

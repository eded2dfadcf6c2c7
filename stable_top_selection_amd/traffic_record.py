"""Write the HBM-traffic record of the select kernel that bench.py reports as
``roofline.traffic``, from two rocprofv3 counter runs of ``bench.py --pmc``:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o fetch -- python3 bench.py --pmc
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o write -- python3 bench.py --pmc
    python -m stable_top_selection_amd.traffic_record gpurun_out/pmc_fetch/fetch_counter_collection.csv \\
        gpurun_out/pmc_write/write_counter_collection.csv

``bench.py --pmc`` runs three 512 MiB device copies and then 64 HBM-cold
select launches on the large workload.  The counters report KiB per dispatch
in the units of their hardware blocks; each is scaled by the factor that makes
the copy's median read (or write) equal to its 512 MiB, and the select's
median over its dispatches, so scaled, is the record's bytes per launch.  The
record holds the sha256 of the select source it was measured on; bench.py
reports it only while the source is unchanged.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORD = os.path.join(ROOT, "profiles", "select_large_rows256_traffic.json")
SOURCE = os.path.join(ROOT, "stable_top_selection_amd", "csrc", "select.hip")
KERNEL = "stable_topk_kernel<512, 2, 16, true"  # the large workload's kernel (8-byte pairs, 16 items per lane)
COPY_KIB = 512 * 1024
ALGORITHMIC = 256 * 8192 * 8 + 256 * 2048 * 8  # candidates read + output written per launch


def medians(path: str, counter: str) -> tuple[float, float, str]:
    """(select median, copy median, select kernel name) of one counter."""
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    sel = [r for r in rows if KERNEL in r["Kernel_Name"]]
    cp = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
    if not sel or not cp:
        raise SystemExit(f"{path}: no {counter} rows for the select kernel and the copy")
    return statistics.median(float(r["Counter_Value"]) for r in sel), statistics.median(cp), sel[0]["Kernel_Name"]


def main(fetch_csv: str, write_csv: str) -> dict:
    fs, fc, name = medians(fetch_csv, "FETCH_SIZE")
    ws, wc, _ = medians(write_csv, "WRITE_SIZE")
    fscale, wscale = COPY_KIB / fc, COPY_KIB / wc
    fb, wb = round(fs * 1024 * fscale), round(ws * 1024 * wscale)
    with open(SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    rec = {
        "kernel": name,
        "workload": "large: 256 rows x 8192 candidates, K 2048, HBM-cold pool",
        "select_source_sha256": sha,
        "fetch_size_kib_per_dispatch": fs,
        "write_size_kib_per_dispatch": ws,
        "copy_512MiB_fetch_size_kib": fc,
        "copy_512MiB_write_size_kib": wc,
        "fetch_scale": fscale,
        "write_scale": wscale,
        "fetch_bytes_per_launch": fb,
        "write_bytes_per_launch": wb,
        "bytes_per_launch": fb + wb,
        "algorithmic_bytes_per_launch": ALGORITHMIC,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o fetch -- python3 bench.py --pmc",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o write -- python3 bench.py --pmc",
        ],
    }
    with open(RECORD, "w") as f:
        json.dump(rec, f, indent=2)
        f.write("\n")
    return rec


if __name__ == "__main__":
    if len(sys.argv) != 3:
        raise SystemExit(__doc__)
    r = main(sys.argv[1], sys.argv[2])
    print(f"{r['bytes_per_launch']} bytes per launch, {r['bytes_per_launch'] / ALGORITHMIC:.4f} x the algorithmic bytes")

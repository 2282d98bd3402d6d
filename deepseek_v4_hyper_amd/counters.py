"""HBM traffic per launch from rocprofv3 counter passes, for bench.py's
``roofline.traffic``.

Two passes over the same benchmark command, each in a run of its own:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o fetch -- \
        python3 bench.py --workload W --path P --steps 3 --warmup 1 --sets 1 \
        --no-cpu-baseline --copy-calibration
    rocprofv3 --pmc WRITE_SIZE ... (same) ...

``--copy-calibration`` makes the last dispatch of the process a plain
elementwise copy of 1 GiB (read 1 GiB, write 1 GiB). FETCH_SIZE and
WRITE_SIZE are in KiB per dispatch; each is scaled by
``known bytes / counter reading`` of that copy, so the figure is in the same
units as the algorithmic bytes. Then

    python -m deepseek_v4_hyper_amd.counters --fetch <dir_f> --write <dir_w> \
        --kernel hc_tile_kernel --workload prefill --out profiles/<file>.json \
        --command-fetch "..." --command-write "..."

writes the record bench.py reads. It stores a hash of the kernel sources, and
bench.py reports ``traffic`` only while the sources still match it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_SOURCES = ["deepseek_v4_hyper_amd/csrc/hc_kernels.hip",
                  "deepseek_v4_hyper_amd/csrc/hc_device.hpp",
                  "deepseek_v4_hyper_amd/csrc/hc_launch.hpp"]
CALIBRATION_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_dispatches(outdir: str, counter: str):
    """[(dispatch id, kernel name, value)] for one counter, in dispatch order."""
    rows = []
    files = glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {outdir}")
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    # a counter that sums over instances appears once per dispatch after aggregation;
    # merge any per-instance rows of one dispatch
    merged = {}
    for did, name, v in rows:
        n0, v0 = merged.get(did, (name, 0.0))
        merged[did] = (n0, v0 + v)
    return [(did, merged[did][0], merged[did][1]) for did in sorted(merged)]


def per_launch(outdir: str, counter: str, kernel: str):
    ds = read_dispatches(outdir, counter)
    mine = [v for _, name, v in ds if kernel in name]
    if not mine:
        raise ValueError(f"no dispatch of {kernel} in {outdir}")
    calib_name, calib = ds[-1][1], ds[-1][2]
    if kernel in calib_name:
        raise ValueError("the last dispatch is not the calibration copy; run with --copy-calibration")
    return sum(mine) / len(mine), len(mine), calib, calib_name


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True, help="rocprofv3 output directory of the FETCH_SIZE pass")
    ap.add_argument("--write", required=True, help="rocprofv3 output directory of the WRITE_SIZE pass")
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--algorithmic-bytes", type=int, default=None)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command-fetch", default="")
    ap.add_argument("--command-write", default="")
    a = ap.parse_args()
    f_kib, nf, f_cal, cal_name = per_launch(a.fetch, "FETCH_SIZE", a.kernel)
    w_kib, nw, w_cal, _ = per_launch(a.write, "WRITE_SIZE", a.kernel)
    f_scale = CALIBRATION_BYTES / f_cal
    w_scale = CALIBRATION_BYTES / w_cal
    rec = {
        "kernel": a.kernel,
        "workload": a.workload,
        "source_sha256": kernel_source_hash(),
        "fetch_size_kib_per_dispatch": f_kib,
        "write_size_kib_per_dispatch": w_kib,
        "dispatches": {"fetch": nf, "write": nw},
        "calibration": {"kernel": cal_name[:120], "bytes_read": CALIBRATION_BYTES,
                        "bytes_written": CALIBRATION_BYTES, "fetch_size_kib": f_cal,
                        "write_size_kib": w_cal},
        "fetch_bytes_per_counter_unit": f_scale,
        "write_bytes_per_counter_unit": w_scale,
        "traffic_read_bytes_per_launch": f_kib * f_scale,
        "traffic_write_bytes_per_launch": w_kib * w_scale,
        "traffic_bytes_per_launch": f_kib * f_scale + w_kib * w_scale,
        "commands": {"fetch": a.command_fetch, "write": a.command_write},
    }
    if a.algorithmic_bytes:
        rec["algorithmic_bytes_per_launch"] = a.algorithmic_bytes
        rec["traffic_over_algorithmic"] = rec["traffic_bytes_per_launch"] / a.algorithmic_bytes
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps({k: rec[k] for k in ("kernel", "traffic_bytes_per_launch",
                                          "fetch_bytes_per_counter_unit",
                                          "write_bytes_per_counter_unit")}))


if __name__ == "__main__":
    main()

"""HBM traffic per launch from rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE).

The counters are read in their own profiler runs, one counter per run, as CSV
(``rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o run -- ...``).  A plain
device-to-device copy of a known size (512 MiB, ``torch`` ``copy_`` between two device
buffers, run inline with ``python3 -c``) profiled the same way gives the factor between each
counter's units and bytes.  The result is written as JSON next to
the summaries under ``profiles/``, tagged with a hash of the kernel sources and build
flags; ``bench.py`` reports it as ``roofline.traffic`` only while that hash matches.

    python -m decoding_step_amd.traffic --workload mixed_b16_l32 --kernel gemm_r512_kernel \\
        --fetch prof/pmc_FETCH --write prof/pmc_WRITE \\
        --copy-fetch prof/pmc_copy_FETCH --copy-write prof/pmc_copy_WRITE
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ("decoding_step_amd/csrc/dlm_device.hpp", "decoding_step_amd/csrc/dlm.hip", "decoding_step_amd/build.py")
COPY_KERNEL = "copyBuffer"


def kernel_source_hash() -> str:
    """SHA-256 over the kernel sources and the build script (its flags shape the code)."""
    h = hashlib.sha256()
    for f in SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_values(run_dir: str, counter: str, kernel: str) -> list:
    """Per-dispatch values of `counter` for kernels whose name contains `kernel`."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    out = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
                out.append(float(r["Counter_Value"]))
    if not out:
        raise ValueError(f"no {counter} rows for a kernel matching {kernel!r} in {files[0]}")
    return out


def mean(xs):
    return sum(xs) / len(xs)


def summarize(workload, kernel, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, skip=0):
    cf = mean(counter_values(copy_fetch_dir, "FETCH_SIZE", COPY_KERNEL))
    cw = mean(counter_values(copy_write_dir, "WRITE_SIZE", COPY_KERNEL))
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    kf = counter_values(fetch_dir, "FETCH_SIZE", kernel)[skip:]
    kw = counter_values(write_dir, "WRITE_SIZE", kernel)[skip:]
    if not kf or not kw:
        raise ValueError(f"no dispatches of {kernel!r} left after skipping {skip}")
    rd = mean(kf) * 1024.0 * fetch_scale
    wr = mean(kw) * 1024.0 * write_scale
    return {
        "kernel": kernel,
        "workload": workload,
        "kernel_source_sha256": kernel_source_hash(),
        "dispatches": {"fetch": len(kf), "write": len(kw), "skipped": skip},
        "fetch_size_kib_per_dispatch": round(mean(kf), 1),
        "write_size_kib_per_dispatch": round(mean(kw), 1),
        "copy_calibration": {"bytes_per_copy": copy_bytes, "fetch_size_kib": round(cf, 1),
                             "write_size_kib": round(cw, 1), "fetch_scale": fetch_scale,
                             "write_scale": write_scale},
        "hbm_read_bytes_per_launch": int(round(rd)),
        "hbm_write_bytes_per_launch": int(round(wr)),
        "hbm_bytes_per_launch": int(round(rd + wr)),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kernel", required=True, help="substring of the kernel name")
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-mib", type=int, default=512)
    ap.add_argument("--skip", type=int, default=0,
                    help="leave out the first N matching dispatches (e.g. the whole-vocabulary launches "
                         "that record the trajectory before a shard run)")
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    d = summarize(a.workload, a.kernel, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib << 20, a.skip)
    out = a.out or os.path.join(ROOT, "profiles", f"{a.workload}_counters.json")
    with open(out, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(d, indent=1))


if __name__ == "__main__":
    main()

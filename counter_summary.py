"""Counter summary behind bench.py's ``roofline.traffic``.

Reads the rocprofv3 counter CSVs of two runs of the same bench command, one
with ``--pmc FETCH_SIZE`` and one with ``--pmc WRITE_SIZE``, both given
``--copy-calibration-mib M`` (three plain device copies of M MiB), and writes
``profiles/pmc_traffic.json``:

* per configuration: the mean FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of
  the partition kernel and of the merge kernel;
* the scale of each counter: the copy's true bytes (M MiB read, M MiB
  written) over what the counter reported for it. The copies are the
  ``__amd_rocclr_copyBuffer`` dispatches whose WRITE_SIZE is M MiB; the FETCH
  run issues the same dispatch sequence, so the same dispatch ids select them
  there;
* the digest of the device source the counters were taken on (bench.py
  reports the traffic only while the source matches).

Usage (repository root):

    python counter_summary.py --copy-mib 1024 --out profiles/pmc_traffic.json \\
        KEY:FETCH_DIR:WRITE_DIR [KEY:FETCH_DIR:WRITE_DIR ...]

KEY is the configuration key bench.py builds for the run
(``workload:P<page>:part<tokens>:<fused|separate>:<prefix|noprefix>[:k8]``);
each DIR holds the run's ``*counter_collection.csv``.
"""

import argparse
import csv
import glob
import json
import os
import sys

import bench

PARTITION = "decode_partition_kernel"
MERGE = "lse_reduce"
COPY = "__amd_rocclr_copyBuffer"


def load(directory, counter):
    paths = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if len(paths) != 1:
        sys.exit("%s: expected one counter_collection.csv, found %d" % (directory, len(paths)))
    rows = []
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def mean_of(rows, name):
    vals = [v for _, k, v in rows if name in k]
    return (sum(vals) / len(vals) if vals else 0.0), len(vals)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--out", default=os.path.join("profiles", "pmc_traffic.json"))
    ap.add_argument("runs", nargs="+", help="KEY:FETCH_DIR:WRITE_DIR")
    args = ap.parse_args()
    copy_kib = args.copy_mib * 1024.0

    configs = {}
    fetch_scales, write_scales = [], []
    for spec in args.runs:
        key, fdir, wdir = spec.rsplit(":", 2)
        fetch = load(fdir, "FETCH_SIZE")
        write = load(wdir, "WRITE_SIZE")
        copies = {d for d, k, v in write if COPY in k and abs(v - copy_kib) <= 0.01 * copy_kib}
        if len(copies) != 3:
            sys.exit("%s: found %d calibration copies, expected 3" % (wdir, len(copies)))
        fc = [v for d, k, v in fetch if d in copies]
        if len(fc) != 3:
            sys.exit("%s: the calibration dispatches are not all in the FETCH run" % fdir)
        fetch_scales.append(copy_kib / (sum(fc) / 3))
        write_scales.append(1.0)                    # selected as exactly the copy's bytes
        pf, n_pf = mean_of(fetch, PARTITION)
        pw, n_pw = mean_of(write, PARTITION)
        mf, n_mf = mean_of(fetch, MERGE)
        mw, _ = mean_of(write, MERGE)
        if n_pf == 0 or n_pf != n_pw:
            sys.exit("%s: partition-kernel dispatches differ between the runs (%d, %d)" % (key, n_pf, n_pw))
        configs[key] = {
            "workload": key.split(":")[0],
            "fetch_kib_per_call": round(pf + mf, 1),
            "write_kib_per_call": round(pw + mw, 1),
            "partition_kernel": {"fetch_kib": round(pf, 1), "write_kib": round(pw, 1), "n": n_pf},
            "reduce_kernel": {"fetch_kib": round(mf, 1), "write_kib": round(mw, 1), "n": n_mf},
        }
    fetch_scale = sum(fetch_scales) / len(fetch_scales)
    rec = {
        "configs": configs,
        "kernel_code_sha256": bench.kernel_source_digest(),
        "fetch_scale": round(fetch_scale, 4),
        "write_scale": 1.0,
        "calibration": "%d MiB device-to-device copy: FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB"
                       % (args.copy_mib, copy_kib / fetch_scale, copy_kib),
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()

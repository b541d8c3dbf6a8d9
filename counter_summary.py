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
  reports the traffic only while the source matches);
* with ``--rdreq KEY:DIR``, a check of the FETCH_SIZE scale from a third run
  of the same command with ``--pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum
  TCC_EA0_RDREQ_128B_sum TCC_BUBBLE_sum``: read bytes rebuilt from the request
  counts by size (128 B, 32 B, the rest 64 B) for the three calibration
  copies and for the partition kernel. FETCH_SIZE's own expression takes
  TCC_BUBBLE as the 128-byte request count; where that counter reads zero
  while TCC_EA0_RDREQ_128B does not, FETCH_SIZE prices 128-byte requests at
  64 bytes and its scale is 2.

Usage (repository root):

    python counter_summary.py --copy-mib 1024 --out profiles/pmc_traffic.json \\
        [--rdreq KEY:RDREQ_DIR] KEY:FETCH_DIR:WRITE_DIR [KEY:FETCH_DIR:WRITE_DIR ...]

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


RDREQ = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_128B_sum", "TCC_BUBBLE_sum")


def rdreq_check(directory, copy_kib):
    """Read bytes per dispatch from the request counts by size, for the three
    calibration copies (the copy dispatches that read the copy's size) and
    the partition kernel."""
    per = {}
    for c in RDREQ:
        for d, k, v in load(directory, c):
            per.setdefault(d, {"kernel": k})[c] = v

    def kib(c):
        n, n32, n128 = c["TCC_EA0_RDREQ_sum"], c["TCC_EA0_RDREQ_32B_sum"], c["TCC_EA0_RDREQ_128B_sum"]
        return (128 * n128 + 32 * n32 + 64 * (n - n128 - n32)) / 1024

    copies = [c for c in per.values() if COPY in c["kernel"] and abs(kib(c) - copy_kib) <= 0.02 * copy_kib]
    parts = [c for c in per.values() if PARTITION in c["kernel"]]
    if len(copies) != 3 or not parts:
        sys.exit("%s: found %d calibration copies and %d partition dispatches" % (directory, len(copies), len(parts)))
    mean = lambda xs: sum(xs) / len(xs)
    return {
        "copy_read_kib_from_requests": round(mean([kib(c) for c in copies]), 1),
        "copy_kib": copy_kib,
        "partition_read_kib_from_requests": round(mean([kib(c) for c in parts]), 1),
        "partition_requests": {c: round(mean([p[c] for p in parts]), 1) for c in RDREQ},
        "n": len(parts),
    }


def mean_of(rows, name):
    vals = [v for _, k, v in rows if name in k]
    return (sum(vals) / len(vals) if vals else 0.0), len(vals)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--out", default=os.path.join("profiles", "pmc_traffic.json"))
    ap.add_argument("--rdreq", default=None, help="KEY:DIR of the request-count run")
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
    if args.rdreq:
        key, rdir = args.rdreq.rsplit(":", 1)
        chk = rdreq_check(rdir, copy_kib)
        chk["config"] = key
        if key in configs:
            chk["partition_fetch_kib_scaled"] = round(configs[key]["partition_kernel"]["fetch_kib"] * fetch_scale, 1)
        rec["fetch_scale_check"] = chk
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()

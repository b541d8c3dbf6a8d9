"""counter_summary.py: the counter record behind bench.py's roofline.traffic,
built from synthetic rocprofv3 counter CSVs (CPU only)."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
PART = "void (anonymous namespace)::decode_partition_kernel<128, 4, true, true, false, false>(DecodeParams)"
MERGE = "void (anonymous namespace)::lse_reduce_kernel<128>(DecodeParams)"
COPY = "__amd_rocclr_copyBuffer"


def write_run(directory, counter, dispatches):
    """dispatches: (dispatch id, kernel name, value) rows of one counter run."""
    os.makedirs(directory)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, v in dispatches:
            row = {k: 0 for k in FIELDS}
            row.update(Dispatch_Id=d, Kernel_Name=name, Counter_Name=counter, Counter_Value=v)
            w.writerow(row)


def make_pair(base, copy_kib, fetch_ratio):
    """A FETCH and a WRITE run of one command: small uploads, three calibration
    copies, then three partition + merge calls."""
    fetch, write = [], []
    d = 1
    for v in (100.0, 2000.0):                              # uploads through the copy kernel
        fetch.append((d, COPY, v))
        write.append((d, COPY, v * 3))
        d += 1
    for _ in range(3):                                     # calibration copies
        fetch.append((d, COPY, copy_kib / fetch_ratio))
        write.append((d, COPY, copy_kib))
        d += 1
    for i in range(3):
        fetch.append((d, PART, 1000.0 + 10 * i))
        write.append((d, PART, 50.0 + i))
        d += 1
        fetch.append((d, MERGE, 20.0))
        write.append((d, MERGE, 4.0))
        d += 1
    write_run(os.path.join(base, "FETCH_SIZE"), "FETCH_SIZE", fetch)
    write_run(os.path.join(base, "WRITE_SIZE"), "WRITE_SIZE", write)
    return os.path.join(base, "FETCH_SIZE"), os.path.join(base, "WRITE_SIZE")


def run(args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "counter_summary.py")] + args, cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def test_summary_scales_and_means(tmp_path):
    f, w = make_pair(str(tmp_path / "a"), 1024 * 1024.0, 2.0)
    out = tmp_path / "pmc.json"
    key = "llama3-8b-gqa-prefix:P16:part1024:fused:prefix"
    r = run(["--copy-mib", "1024", "--out", str(out), "%s:%s:%s" % (key, f, w)])
    assert r.returncode == 0, r.stderr
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == 1.0
    assert rec["kernel_code_sha256"] == bench.kernel_source_digest()
    c = rec["configs"][key]
    assert c["workload"] == "llama3-8b-gqa-prefix"
    assert c["partition_kernel"] == {"fetch_kib": 1010.0, "write_kib": 51.0, "n": 3}
    assert c["reduce_kernel"] == {"fetch_kib": 20.0, "write_kib": 4.0, "n": 3}
    assert c["fetch_kib_per_call"] == pytest.approx(1030.0)
    assert c["write_kib_per_call"] == pytest.approx(55.0)


def test_bench_reads_the_summary_it_matches(tmp_path, monkeypatch):
    # bench.measured_traffic reads profiles/pmc_traffic.json under ROOT: point ROOT at a copy
    f, w = make_pair(str(tmp_path / "a"), 1024 * 1024.0, 2.0)
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "paged_kv_cache_279_amd" / "csrc"
    src.mkdir(parents=True)
    with open(os.path.join(ROOT, "paged_kv_cache_279_amd", "csrc", "pkv_device.hip")) as fh:
        (src / "pkv_device.hip").write_text(fh.read())
    key = "w:P16:part0:fused:noprefix"
    r = run(["--copy-mib", "1024", "--out", str(tmp_path / "profiles" / "pmc_traffic.json"), "%s:%s:%s" % (key, f, w)])
    assert r.returncode == 0, r.stderr
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", key) == pytest.approx((1010.0 * 2.0 + 51.0) * 1024)
    assert bench.measured_traffic("other", key) is None
    # an edit of the kernel code orphans the record
    (src / "pkv_device.hip").write_text((src / "pkv_device.hip").read_text() + "\nint x;\n")
    assert bench.measured_traffic("w", key) is None


def test_summary_rejects_runs_without_calibration(tmp_path):
    f, w = make_pair(str(tmp_path / "a"), 1024 * 1024.0, 2.0)
    r = run(["--copy-mib", "512", "--out", str(tmp_path / "x.json"), "k:%s:%s" % (f, w)])
    assert r.returncode != 0
    assert "calibration copies" in r.stderr

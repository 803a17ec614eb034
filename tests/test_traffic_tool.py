"""The counter-to-bytes tool on synthetic counter files (no GPU): every
request counted at its size, totals over the matching kernel's dispatches
(several per call) divided by the calls the bench made, other kernels'
rows ignored, and the entry keyed to the fingerprint of the kernel in the
built library."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY = "void (anonymous namespace)::copy_kernel<false>((anonymous namespace)::CopyArgs)"
OTHER = "void at::native::some_elementwise_kernel<4>(int)"


def _csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for d, k, c, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c,
                        "Counter_Value": f"{v:.6f}"})


def test_bytes_per_call_from_request_counts(tmp_path):
    # three calls of two launches each: per launch 1000 128-byte, 10 64-byte,
    # 4 32-byte reads; 500 64-byte and 6 32-byte writes
    rd, wr = [], []
    for d in range(6):
        rd += [(d, COPY, "TCC_EA0_RDREQ_sum", 1014), (d, COPY, "TCC_EA0_RDREQ_32B_sum", 4),
               (d, COPY, "TCC_EA0_RDREQ_64B_sum", 10), (d, COPY, "TCC_EA0_RDREQ_128B_sum", 1000)]
        wr += [(d, COPY, "TCC_EA0_WRREQ_sum", 506), (d, COPY, "TCC_EA0_WRREQ_64B_sum", 500)]
    rd += [(99, OTHER, "TCC_EA0_RDREQ_128B_sum", 10 ** 9)]          # not the measured kernel
    wr += [(99, OTHER, "TCC_EA0_WRREQ_64B_sum", 10 ** 9)]
    _csv(tmp_path / "r.csv", rd)
    _csv(tmp_path / "w.csv", wr)
    for name in ("r.json", "w.json"):
        (tmp_path / name).write_text("noise\n" + json.dumps({"calls_made": {"copy": 3}}) + "\n")
    out = tmp_path / "traffic.json"
    subprocess.run([sys.executable, "-m", "zero_partition_aware_amd.traffic",
                    "--read", str(tmp_path / "r.csv"), "--write", str(tmp_path / "w.csv"),
                    "--match", "copy_kernel<false>",
                    "--bench-json", str(tmp_path / "r.json"), str(tmp_path / "w.json"),
                    "--label", "copy", "--algorithmic-bytes", "270000", "--key", "t:copy",
                    "--out", str(out)], check=True, cwd=ROOT, capture_output=True)
    e = json.loads(out.read_text())["t:copy"]
    read_per_launch = 128 * 1000 + 64 * 10 + 32 * 4
    write_per_launch = 64 * 500 + 32 * 6
    assert e["read_bytes_per_call"] == 2 * read_per_launch
    assert e["write_bytes_per_call"] == 2 * write_per_launch
    assert e["hbm_bytes_per_call"] == 2 * (read_per_launch + write_per_launch)
    assert e["calls"] == [3, 3] and e["dispatches"] == [6, 6]
    assert e["read_requests_by_size_sum_to_total"] is True
    assert abs(e["traffic_over_algorithmic"] - 2 * (read_per_launch + write_per_launch) / 270000) < 1e-12
    assert list(e["kernel_sha"]) == [COPY]

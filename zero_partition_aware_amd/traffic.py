"""Turn two rocprofv3 counter runs into HBM bytes per call of one kernel.

Counters (gfx950, TCC = the L2, EA = its interface to memory; each summed over
the 16 channels of every XCD):

* read pass:  ``TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum
  TCC_EA0_RDREQ_128B_sum`` -- read requests to memory, in total and by size;
* write pass: ``TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum`` -- write requests in
  total (32- or 64-byte) and the 64-byte ones.

read bytes  = 128 * RDREQ_128B + 64 * RDREQ_64B + 32 * RDREQ_32B
write bytes = 64 * WRREQ_64B + 32 * (WRREQ - WRREQ_64B)

No calibration factor: every request is counted at its size.  (The derived
FETCH_SIZE metric counts a 128-byte read as 64 bytes on this part, which is
why it reads half the true bytes.)  A call of the library can be cut into
several equal launches, so the bytes are summed over every dispatch of the
matching kernels and divided by the number of calls the bench made
(``calls_made`` in its JSON line, counter runs taken with ``--no-parity``).

    python -m zero_partition_aware_amd.traffic \\
        --read R.csv --write W.csv --match 'reduce_kernel<float, 8,' \\
        --bench-json B.json --label fused --algorithmic-bytes 58219394048 \\
        --key llama3-8b:fused --out profiles/traffic.json
"""

import argparse
import csv
import json
import os
import shlex
import sys

from .build import kernel_hashes

READ = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
        "TCC_EA0_RDREQ_128B_sum")
WRITE = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")


def counter_totals(path, match, names):
    """{counter: total over matching dispatches}, dispatch count, kernel names."""
    tot = {n: 0.0 for n in names}
    dispatches, kernels = set(), set()
    for r in csv.DictReader(open(path)):
        if match not in r["Kernel_Name"] or r["Counter_Name"] not in tot:
            continue
        tot[r["Counter_Name"]] += float(r["Counter_Value"])
        dispatches.add(r["Dispatch_Id"])
        kernels.add(r["Kernel_Name"])
    if not dispatches:
        raise SystemExit(f"no dispatch of a kernel matching {match!r} in {path}")
    return tot, len(dispatches), kernels


def read_bytes(t):
    return 128 * t["TCC_EA0_RDREQ_128B_sum"] + 64 * t["TCC_EA0_RDREQ_64B_sum"] + \
        32 * t["TCC_EA0_RDREQ_32B_sum"]


def write_bytes(t):
    return 64 * t["TCC_EA0_WRREQ_64B_sum"] + \
        32 * (t["TCC_EA0_WRREQ_sum"] - t["TCC_EA0_WRREQ_64B_sum"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--read", required=True, help="counter_collection.csv of the read pass")
    ap.add_argument("--write", required=True, help="counter_collection.csv of the write pass")
    ap.add_argument("--match", required=True, help="substring of the kernel name")
    ap.add_argument("--bench-json", nargs=2, required=True, metavar=("READ_RUN", "WRITE_RUN"),
                    help="bench.py's JSON line of each counter run")
    ap.add_argument("--label", required=True, help="the bench's label of the measured call")
    ap.add_argument("--algorithmic-bytes", type=int, default=None, help="per call")
    ap.add_argument("--key", required=True)
    ap.add_argument("--out", required=True)
    args = ap.parse_args()

    rt, nr, r_names = counter_totals(args.read, args.match, READ)
    wt, nw, w_names = counter_totals(args.write, args.match, WRITE)
    calls = []
    for path in args.bench_json:
        line = [ln for ln in open(path) if ln.startswith("{")][-1]
        calls.append(json.loads(line)["calls_made"][args.label])
    rsum = rt["TCC_EA0_RDREQ_32B_sum"] + rt["TCC_EA0_RDREQ_64B_sum"] + rt["TCC_EA0_RDREQ_128B_sum"]
    read_b = read_bytes(rt) / calls[0]
    write_b = write_bytes(wt) / calls[1]
    hashes = kernel_hashes()
    measured = sorted(r_names | w_names)
    missing = [n for n in measured if n not in hashes]
    if missing:
        raise SystemExit(f"no fingerprint in the built library for {missing}")
    entry = {"kernel_sha": {n: hashes[n] for n in measured},
             "hbm_bytes_per_call": round(read_b + write_b),
             "read_bytes_per_call": round(read_b),
             "write_bytes_per_call": round(write_b),
             "calls": calls, "dispatches": [nr, nw],
             "raw_counts": {"read_pass": {k: round(v) for k, v in rt.items()},
                            "write_pass": {k: round(v) for k, v in wt.items()}},
             "read_requests_by_size_sum_to_total": round(rsum) == round(rt["TCC_EA0_RDREQ_sum"]),
             "bytes": "128*RDREQ_128B + 64*RDREQ_64B + 32*RDREQ_32B read; "
                      "64*WRREQ_64B + 32*(WRREQ - WRREQ_64B) written; totals over the "
                      "matching dispatches divided by the calls made",
             "command": "python -m zero_partition_aware_amd.traffic " +
                        " ".join(shlex.quote(a) for a in sys.argv[1:]),
             "counter_runs": "rocprofv3 --pmc " + " ".join(READ) + " (then --pmc " +
                             " ".join(WRITE) + ") --output-format csv -- python3 bench.py "
                             "--no-cpu-baseline --no-parity ..."}
    if args.algorithmic_bytes:
        entry["algorithmic_bytes_per_call"] = args.algorithmic_bytes
        entry["traffic_over_algorithmic"] = (read_b + write_b) / args.algorithmic_bytes
    data = {}
    if os.path.exists(args.out):
        data = json.load(open(args.out))
    data[args.key] = entry
    with open(args.out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps({args.key: entry}, indent=1))


if __name__ == "__main__":
    main()

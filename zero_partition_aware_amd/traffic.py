"""Turn rocprofv3 ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs into HBM
bytes per launch, calibrated against a plain copy of known size.

The TCC counters FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch; on
gfx950 FETCH_SIZE reads a fixed fraction of the true read bytes.  Each counter
is scaled by (known bytes of the copy kernel) / (counter on the copy kernel).

    python -m zero_partition_aware_amd.traffic \\
        --fetch F.csv --write W.csv --match reduce_kernel \\
        --copy-fetch CF.csv --copy-write CW.csv --copy-match elementwise \\
        --copy-bytes 4294967296 --key gpt2-small:fused --out profiles/traffic.json
"""

import argparse
import csv
import json
import os
import shlex
import sys

from .build import kernel_hashes


def _avg_kib(path, match):
    rows = [r for r in csv.DictReader(open(path)) if match in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no dispatch of a kernel matching {match!r} in {path}")
    vals = [float(r["Counter_Value"]) for r in rows]
    return sum(vals) / len(vals), len(vals), {r["Kernel_Name"] for r in rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--match", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-match", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True,
                    help="bytes the copy kernel reads (= bytes it writes)")
    ap.add_argument("--algorithmic-bytes", type=int, default=None)
    ap.add_argument("--key", required=True)
    ap.add_argument("--out", required=True)
    args = ap.parse_args()

    f_kib, nf, f_names = _avg_kib(args.fetch, args.match)
    w_kib, nw, w_names = _avg_kib(args.write, args.match)
    cf_kib, _, _ = _avg_kib(args.copy_fetch, args.copy_match)
    cw_kib, _, _ = _avg_kib(args.copy_write, args.copy_match)
    f_scale = args.copy_bytes / (cf_kib * 1024)
    w_scale = args.copy_bytes / (cw_kib * 1024)
    read_b = f_kib * 1024 * f_scale
    write_b = w_kib * 1024 * w_scale
    # The entry is keyed to the fingerprints of the kernels it measured.
    hashes = kernel_hashes()
    measured = sorted(f_names | w_names)
    missing = [n for n in measured if n not in hashes]
    if missing:
        raise SystemExit(f"no fingerprint in the built library for {missing}")
    entry = {"kernel_sha": {n: hashes[n] for n in measured},
             "hbm_bytes_per_launch": round(read_b + write_b),
             "read_bytes_per_launch": round(read_b),
             "write_bytes_per_launch": round(write_b),
             "fetch_size_kib": f_kib, "write_size_kib": w_kib,
             "dispatches": [nf, nw],
             "fetch_scale": f_scale, "write_scale": w_scale,
             "calibration": f"copy kernel matching {args.copy_match!r}, "
                            f"{args.copy_bytes} B read and written",
             "command": "python -m zero_partition_aware_amd.traffic " +
                        " ".join(shlex.quote(a) for a in sys.argv[1:]),
             "counter_runs": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv "
                             "-- python3 bench.py ... for the kernel and for --workload copy"}
    if args.algorithmic_bytes:
        entry["algorithmic_bytes_per_launch"] = args.algorithmic_bytes
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

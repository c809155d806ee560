"""HBM traffic per launch from rocprofv3 counter runs, calibrated by a plain copy.

Four counter runs feed this (each a separate `rocprofv3 --pmc <counter>
--output-format csv` run, because one pass cannot hold both counters):

  FETCH_SIZE and WRITE_SIZE of   python3 bench.py --mode launch --config C --steps S
  FETCH_SIZE and WRITE_SIZE of   python3 bench.py --mode copy --copy-mib M --steps S

The copy moves exactly M MiB in and M MiB out per launch, so
    factor_fetch = M MiB / (copy FETCH_SIZE KiB * 1024),
and likewise for writes.  The attention kernel's bytes per launch are its mean
counter value times 1024 times that factor.  The result is written to
profiles/traffic.json under the workload name, together with the hash of the
kernel sources it was taken on (bench.py reports it only while that hash still
matches), and a readable summary is printed.

Run:  python -m exact_attention_forward_tiled_amd.traffic --config 2 --copy-mib 1024 \
          --attn-fetch DIR --attn-write DIR --copy-fetch DIR --copy-write DIR
"""

import argparse
import csv
import glob
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def counter_values(run_dir, counter, name_filter):
    """Per-dispatch values of `counter` for kernels whose name contains name_filter."""
    paths = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for p in paths:
        with open(p) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter or name_filter not in r["Kernel_Name"]:
                    continue
                key = (p, r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {name_filter!r} in {run_dir}")
    return list(per.values())


def main():
    sys.path.insert(0, ROOT)
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--attn-fetch", required=True)
    ap.add_argument("--attn-write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--kernel-filter", default=None,
                    help="kernel-name substring (default: the workload's forward kernel)")
    ap.add_argument("--copy-filter", default="copy")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    args = ap.parse_args()

    import bench
    import synth
    w = synth.workload(args.config)
    kfilter = args.kernel_filter or f"fwd_{w.fmt}_kernel"

    copy_bytes = args.copy_mib * (1 << 20)
    cf = statistics.median(counter_values(args.copy_fetch, "FETCH_SIZE", args.copy_filter))
    cw = statistics.median(counter_values(args.copy_write, "WRITE_SIZE", args.copy_filter))
    f_fetch = copy_bytes / (cf * 1024.0)
    f_write = copy_bytes / (cw * 1024.0)
    af = statistics.mean(counter_values(args.attn_fetch, "FETCH_SIZE", kfilter))
    aw = statistics.mean(counter_values(args.attn_write, "WRITE_SIZE", kfilter))
    fetch_b = af * 1024.0 * f_fetch
    write_b = aw * 1024.0 * f_write

    # algorithmic bytes: one read of the operands and one write of O, LSE (fp32).
    # bf16: Q, K, V at 2 B per element.  mxfp4 / mxfp8: E2M1 codes (0.5 B) or E4M3 codes
    # (1 B) plus one E8M0 scale byte per 32 elements, for Q, K and the transposed V.
    elems = w.B * w.Hq * w.N * w.d + 2 * w.B * w.Hkv * w.N * w.d
    alg_in = {"bf16": 2 * elems, "mxfp4": elems // 2 + elems // 32,
              "mxfp8": elems + elems // 32}[w.fmt]
    alg_out = 4 * (w.B * w.Hq * w.N * w.d + w.B * w.Hq * w.N)

    rec = {"kernel_hash": bench.kernel_hash(w.fmt), "kernel_filter": kfilter,
           "hbm_bytes_per_launch": round(fetch_b + write_b),
           "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
           "algorithmic_bytes_per_launch": alg_in + alg_out,
           "calibration": {"copy_mib": args.copy_mib, "fetch_factor": f_fetch,
                           "write_factor": f_write,
                           "copy_fetch_kib": cf, "copy_write_kib": cw},
           "raw_kib": {"fetch": af, "write": aw}}
    try:
        with open(args.out) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    table[w.name] = rec
    with open(args.out, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")

    print(f"workload {w.name}")
    print(f"copy calibration: {args.copy_mib} MiB copy read {cf:.0f} KiB / wrote {cw:.0f} KiB "
          f"per launch -> factors fetch {f_fetch:.4f}, write {f_write:.4f}")
    print(f"attention kernel: FETCH_SIZE {af:.0f} KiB, WRITE_SIZE {aw:.0f} KiB per launch")
    print(f"HBM bytes per launch: fetch {fetch_b/2**20:.1f} MiB + write {write_b/2**20:.1f} MiB "
          f"= {(fetch_b + write_b)/2**20:.1f} MiB")
    print(f"algorithmic bytes per launch: in {alg_in/2**20:.1f} MiB + out {alg_out/2**20:.1f} MiB "
          f"= {(alg_in + alg_out)/2**20:.1f} MiB")
    print(f"wrote {args.out}")


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Attention-forward benchmark on one MI355X: prints ONE JSON line.

A step is one fused attention forward (QK^T, mask, online softmax with
thresholded rescale, PV, LSE) over one batch of synthetic inputs already
resident in HBM.  The headline workload is causal B=4, H=16, N=2048, d=128
bf16 (workload 2); `--config` picks another.  The spec workloads with
N >= 8192 (3 and 4) and the exp-mode comparison are reported under "extra".

Timing: W untimed warm-up launches, then K launches bracketed by a device
synchronise on both sides; each launch is also bracketed by HIP events on the
stream it runs on, which gives the average kernel duration used for the
roofline.  FLOPs follow the metric: 4*B*H*N^2*d, halved for causal.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (4·B·H·N²·d, causal halved) and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2516.6      # dense bf16 MFMA, 256 CUs x 2.4 GHz x 4096 flop/clk
PEAK_FP4_TFLOPS = 10066.3      # dense MXFP4 MFMA
KERNEL_SOURCES = ["exact_attention_forward_tiled_amd/csrc/attn_fwd_bf16.hip",
                  "exact_attention_forward_tiled_amd/csrc/attn_mxfp4.hip",
                  "exact_attention_forward_tiled_amd/csrc/common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[workload_name]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def make_inputs(w):
    import torch
    from synth import workload  # noqa: F401  (inputs come from the seeded generator only)
    import numpy as np
    qb, kb, vb = w.make()
    dev = [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
           for x in (qb, kb, vb)]
    return dev, (qb, kb, vb)


def time_launches(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    total_ms = ev[0][0].elapsed_time(ev[-1][1])
    return {"ms_per_step": total_ms / steps, "kernel_ms_avg": sum(per) / len(per),
            "kernel_ms_min": min(per), "kernel_ms_max": max(per), "wall_s": wall}


def bench_bf16(w, steps, warmup, exp_mode="hw", tau=8.0):
    import torch
    import exact_attention_forward_tiled_amd as fa
    (q, k, v), _ = make_inputs(w)
    o = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")

    def step():
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, tau=tau, exp_mode=exp_mode, out=(o, lse))
    t = time_launches(step, steps, warmup)
    t["tflops"] = w.flops / (t["ms_per_step"] * 1e-3) / 1e12
    t["kernel_tflops"] = w.flops / (t["kernel_ms_avg"] * 1e-3) / 1e12
    # skip ratio of the thresholded rescale (separate, untimed launch)
    stats = torch.zeros(2, dtype=torch.int64, device="cuda")
    fa.fwd(q, k, v, causal=w.causal, scale=w.scale, tau=tau, exp_mode=exp_mode, stats=stats,
           out=(o, lse))
    torch.cuda.synchronize()
    s, r = (int(x) for x in stats.cpu())
    t["skip_ratio"] = (1.0 - r / s) if s else None
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return t


def cpu_baseline(w, budget_s=12.0):
    """The float64 oracle, as it stands, on whole (batch, head) slices of the same workload."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    qb, kb, vb = w.make()
    q, k, v = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    done, t0 = 0, time.perf_counter()
    for b, h in heads:
        oracle.attention_head(q, k, v, w.causal, w.scale, b, h)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    flops = w.flops * done / len(heads)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} (batch, head) slices of {w.name}, float64 numpy, "
                      f"{el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--exp", default="hw", choices=["hw", "poly"])
    ap.add_argument("--tau", type=float, default=8.0)
    ap.add_argument("--extra", default="3,4", help="other workloads to time (comma list, or '')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this attention-forward build runs on exactly one GPU; "
              f"--gpus {args.gpus} (WORLD_SIZE {world}) is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = synth.workload(args.config)
    if w.fmt != "bf16":
        print("bench.py: the headline line times a bf16 workload", file=sys.stderr)
        sys.exit(2)

    log(f"timing {w.name}: warmup {args.warmup}, steps {args.steps}")
    t = bench_bf16(w, args.steps, args.warmup, args.exp, args.tau)
    kernel_tf = t["kernel_tflops"]
    traffic = load_traffic(w.name)

    extra = {"kernel_ms_avg": t["kernel_ms_avg"], "kernel_ms_min": t["kernel_ms_min"],
             "pct_of_bf16_peak": 100.0 * t["tflops"] / PEAK_BF16_TFLOPS,
             "skip_ratio": t["skip_ratio"], "exp_mode": args.exp, "tau": args.tau,
             "kernel_hash": kernel_hash(), "workloads": {}}
    other = "poly" if args.exp == "hw" else "hw"
    log(f"timing {w.name} with exp mode {other}")
    t2 = bench_bf16(w, args.steps, args.warmup, other, args.tau)
    extra["workloads"][f"{w.name}/exp={other}"] = {
        "tflops": round(t2["tflops"], 2), "ms": round(t2["ms_per_step"], 4)}
    for idx in [int(x) for x in args.extra.split(",") if x.strip()]:
        wx = synth.workload(idx)
        if wx.fmt != "bf16" or idx == args.config:
            continue
        log(f"timing {wx.name}")
        tx = bench_bf16(wx, max(5, args.steps // 2), args.warmup, args.exp, args.tau)
        extra["workloads"][wx.name] = {
            "tflops": round(tx["tflops"], 2), "ms": round(tx["ms_per_step"], 4),
            "pct_of_bf16_peak": round(100.0 * tx["tflops"] / PEAK_BF16_TFLOPS, 2),
            "skip_ratio": tx["skip_ratio"]}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host")
        cpu = cpu_baseline(w)

    line = {
        "metric": METRIC,
        "value": round(t["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(w.describe()),
        "roofline": {"bound": "mfma", "achieved": round(kernel_tf, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kernel_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

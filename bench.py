#!/usr/bin/env python3
"""Attention-forward benchmark on one MI355X: prints ONE JSON line.

A step is one fused attention forward (QK^T, mask, online softmax with
thresholded rescale, PV, LSE) over one batch of synthetic inputs already
resident in HBM.  The headline workload is the largest bf16 one that fits a
GPU: non-causal B=2, H=16, N=16384, d=128 with q, k ~ N(0, 3^2) (the running
max moves often, so the rescale skip ratio is exercised).  By default the
causal GQA workload B=1, Hq=32, Hkv=8, N=8192 and the MXFP4 Direct-P and
MXFP8 workloads (B=1, H=24, N=16384) are timed beside it, reported under
"extra" (the block-scaled ones with their accuracy on stored reference rows);
`--config` picks another headline and `--extra` another list of workloads
(never in the headline fields).

Timing: the GPU is first driven with untimed launches for `--warmup-seconds`
(clocks ramp up under load), then W untimed warm-up steps, then K timed steps
bracketed by a device synchronise on both sides and by two HIP events on the
stream the kernel runs on; the events' span / K is the step time and the mean
kernel duration used for the roofline (the launches run back to back).  A
separate pass with events around every launch gives min / median / max.
FLOPs follow the metric: 4*B*H*N^2*d, halved for causal.

Other modes (for rocprofv3 counter runs; they print nothing on stdout):
  --mode launch   run the workload's kernel --steps times, no timing, no oracle
                  (with --bwd: the three backward kernels instead)
  --mode copy     a plain device-to-device copy of --copy-mib MiB, --steps times
                  (calibrates the HBM byte counters against a known transfer)
and ones that print their own JSON line:
  --mode lds-patterns  LDS access patterns of the MXFP8 kernel and alternatives, one
                  dispatch each, for a run under the LDS bank-conflict counter
  --mode rates    issue-rate microbenchmarks from the test-only probe library:
                  v_exp_f32 vs the VALU cubic exp2 vs a plain FMA, back-to-back
                  v_mfma_f32_32x32x16_bf16, and LDS reads (ds_read_b128 and the
                  transposing ds_read_b64_tr_b16), each at 2 and 4 waves per SIMD
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (4·B·H·N²·d, causal halved) and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2516.6      # dense bf16 MFMA, 256 CUs x 2.4 GHz x 4096 flop/clk
PEAK_FP4_TFLOPS = 10066.3      # dense MXFP4 MFMA, 256 CUs x 2.4 GHz x 16384 flop/clk
PEAK_FP8_TFLOPS = 5033.2       # dense FP8 MFMA, 256 CUs x 2.4 GHz x 8192 flop/clk
PEAKS = {"bf16": PEAK_BF16_TFLOPS, "mxfp4": PEAK_FP4_TFLOPS, "mxfp8": PEAK_FP8_TFLOPS}
PEAK_CLOCK_GHZ = 2.4           # the clock the published peaks assume
KERNEL_SOURCES = {
    "bf16": ["exact_attention_forward_tiled_amd/csrc/attn_fwd_bf16.hip",
             "exact_attention_forward_tiled_amd/csrc/common.h",
             "exact_attention_forward_tiled_amd/csrc/exp2_poly.h"],
    "mxfp4": ["exact_attention_forward_tiled_amd/csrc/attn_mxfp4.hip",
              "exact_attention_forward_tiled_amd/csrc/common.h"],
    "mxfp8": ["exact_attention_forward_tiled_amd/csrc/attn_mxfp8.hip",
              "exact_attention_forward_tiled_amd/csrc/common.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(fmt="bf16"):
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[fmt]:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name, fmt="bf16"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)[workload_name]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash(fmt):
        return None
    return rec.get("hbm_bytes_per_launch")


def skip_ratio_model(workload_name):
    """The skip ratio the tau rule gives in float64 over 32-row groups and 64-key tiles on
    every head of the workload (stored by tests/golden/make_skip_ratio.py), or None."""
    path = os.path.join(ROOT, "tests", "golden", "skip_ratio.json")
    try:
        with open(path) as fh:
            return json.load(fh)[workload_name]["skip_ratio"]
    except (OSError, KeyError, ValueError):
        return None


def mx_accuracy(wl):
    """Accuracy of a block-scaled workload's last output on stored reference rows (written
    by tests/golden/make_mx_reference_rows.py from the oracle): the mean row cosine against
    exact attention on the unquantised inputs (the explainer page quotes about 0.944 for
    Direct-P and 0.990 for its FP8 path), and the largest per-row relative error against
    the emulation of the same quantisation; None when no rows are stored for it."""
    import numpy as np
    path = os.path.join(ROOT, "tests", "golden", "mx_reference_rows.npz")
    name = wl.w.name
    try:
        ref = np.load(path)
        heads, rows = ref[f"{name}/heads"], ref[f"{name}/rows"]
        exact, emul = ref[f"{name}/exact"], ref[f"{name}/emulated"]
    except (OSError, KeyError, ValueError):
        return None
    got = wl.o[0][heads][:, rows].cpu().numpy().astype(np.float64)
    cos = np.sum(got * exact, -1) / (np.linalg.norm(got, axis=-1) * np.linalg.norm(exact, axis=-1))
    row_err = np.linalg.norm(got - emul, axis=-1) / np.linalg.norm(emul, axis=-1)
    return {"rows": int(cos.size), "mean_row_cosine_vs_exact": round(float(cos.mean()), 5),
            "min_row_cosine_vs_exact": round(float(cos.min()), 5),
            "max_row_relerr_vs_emulation": float(row_err.max()),
            "rows_matching_emulation_within_1e-5": round(float(np.mean(row_err < 1e-5)), 4)}


def device_inputs(w):
    import numpy as np
    import torch
    qb, kb, vb = w.make()
    return [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
            for x in (qb, kb, vb)]


class Workload:
    """Device buffers and one launch closure for a bf16 workload."""

    def __init__(self, w, exp_mode, tau, poly_frac=None, window=0, doc_offsets=None,
                 alibi=False, softcap=0.0):
        import torch
        import exact_attention_forward_tiled_amd as fa
        self.w = w
        self.window = window
        self.docs = (None if doc_offsets is None else
                     torch.tensor(doc_offsets, dtype=torch.int32, device="cuda"))
        self.alibi = alibi_slopes(w.Hq) if alibi else None
        self.softcap = softcap
        self.q, self.k, self.v = device_inputs(w)
        self.o = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
        self.fa = fa
        self.exp_mode, self.tau, self.poly_frac = exp_mode, tau, poly_frac

    def launch(self, stats=None):
        self.fa.fwd(self.q, self.k, self.v, causal=self.w.causal, scale=self.w.scale, tau=self.tau,
                    exp_mode=self.exp_mode, stats=stats, out=(self.o, self.lse),
                    poly_frac=self.poly_frac, window=self.window, docs=self.docs,
                    alibi=self.alibi, softcap=self.softcap)


def alibi_slopes(H):
    """The usual geometric ALiBi slopes 2^(-8 h / H), h = 1 .. H (float32 on the device)."""
    import torch
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32,
                        device="cuda")


class Mxfp4Workload:
    """MXFP4 Direct-P workload: fp32 draws quantised on the GPU once (untimed), then the
    forward on the resident codes and scales."""

    def __init__(self, w, tau, window=0, doc_offsets=None):
        import numpy as np
        import torch
        import exact_attention_forward_tiled_amd as fa
        self.w = w
        self.window = window
        self.docs = (None if doc_offsets is None else
                     torch.tensor(doc_offsets, dtype=torch.int32, device="cuda"))
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in w.make())
        self.q4, self.qs = fa.quantize_mxfp4_rows(q)
        self.k4, self.ks = fa.quantize_mxfp4_rows(k)
        self.vt4, self.vts = fa.quantize_mxfp4_cols_t(v)
        torch.cuda.synchronize()
        del q, k, v
        self.o = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
        self.fa = fa
        self.tau = tau

    def launch(self, stats=None):
        self.fa.fwd_mxfp4(self.q4, self.qs, self.k4, self.ks, self.vt4, self.vts,
                          causal=self.w.causal, scale=self.w.scale, tau=self.tau, stats=stats,
                          out=(self.o, self.lse), window=self.window, docs=self.docs)


class Mxfp8Workload:
    """MXFP8 workload: fp32 draws quantised on the GPU once (untimed), then the forward on
    the resident codes and scales."""

    def __init__(self, w, tau, window=0, doc_offsets=None):
        import numpy as np
        import torch
        import exact_attention_forward_tiled_amd as fa
        self.w = w
        self.window = window
        self.docs = (None if doc_offsets is None else
                     torch.tensor(doc_offsets, dtype=torch.int32, device="cuda"))
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in w.make())
        self.q8, self.qs = fa.quantize_mxfp8_rows(q)
        self.k8, self.ks = fa.quantize_mxfp8_rows(k)
        self.vt8, self.vts = fa.quantize_mxfp8_cols_t(v)
        torch.cuda.synchronize()
        del q, k, v
        self.o = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
        self.fa = fa
        self.tau = tau

    def launch(self, stats=None):
        self.fa.fwd_mxfp8(self.q8, self.qs, self.k8, self.ks, self.vt8, self.vts,
                          causal=self.w.causal, scale=self.w.scale, tau=self.tau, stats=stats,
                          out=(self.o, self.lse), window=self.window, docs=self.docs)


class BwdWorkload:
    """bf16 backward on a bf16 workload: the forward's O and LSE computed once (untimed),
    a seeded dO, then the three backward kernels per step (with the forward's sliding window
    and / or documents when given)."""

    def __init__(self, w, window=0, doc_offsets=None, alibi=False, softcap=0.0):
        import torch
        import exact_attention_forward_tiled_amd as fa
        import synth
        self.w = w
        self.window = window
        self.docs = (None if doc_offsets is None else
                     torch.tensor(doc_offsets, dtype=torch.int32, device="cuda"))
        self.alibi = alibi_slopes(w.Hq) if alibi else None
        self.softcap = softcap
        self.q, self.k, self.v = device_inputs(w)
        self.o, self.lse = fa.fwd(self.q, self.k, self.v, causal=w.causal, scale=w.scale,
                                  window=window, docs=self.docs, alibi=self.alibi,
                                  softcap=softcap)
        gb = synth.normal_bf16((w.B, w.Hq, w.N, w.d), 1000 * w.index + 4, 1.0)
        self.do = device_inputs_bits(gb)
        self.dq = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device="cuda")
        self.dk = torch.empty((w.B, w.Hkv, w.N, w.d), dtype=torch.float32, device="cuda")
        self.dv = torch.empty_like(self.dk)
        self.delta = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        self.fa = fa

    def launch(self, stats=None):
        self.fa.bwd(self.q, self.k, self.v, self.o, self.lse, self.do, causal=self.w.causal,
                    scale=self.w.scale, out=(self.dq, self.dk, self.dv), delta=self.delta,
                    window=self.window, docs=self.docs, alibi=self.alibi, softcap=self.softcap)


def device_inputs_bits(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def visible_pairs(N, causal, window, doc_offsets=None):
    """(query, key) pairs a sliding window of width `window` and/or packed documents show
    (exact count)."""
    import numpy as np
    i = np.arange(N, dtype=np.int64)
    lo = np.maximum(0, i - window + 1) if window else np.zeros_like(i)
    hi = i if causal else (np.minimum(N - 1, i + window - 1) if window else np.full_like(i, N - 1))
    if doc_offsets is not None:
        off = np.asarray(doc_offsets, dtype=np.int64)
        d = np.searchsorted(off, i, side="right") - 1
        lo = np.maximum(lo, off[d])
        hi = np.minimum(hi, off[d + 1] - 1)
    return int((hi - lo + 1).sum())


def make_workload(w, exp_mode, tau, poly_frac=None):
    if w.fmt == "mxfp4":
        return Mxfp4Workload(w, tau)
    if w.fmt == "mxfp8":
        return Mxfp8Workload(w, tau)
    return Workload(w, exp_mode, tau, poly_frac)


def time_workload(wl, steps, warmup, warmup_seconds):
    """Ramp, warm up, then K back-to-back launches between two HIP events on the launch
    stream (their span / K is both ms_per_step and the mean kernel duration); a second,
    separate pass brackets each launch with its own events for min / median / max."""
    import torch
    stream = torch.cuda.current_stream()
    t_end = time.perf_counter() + warmup_seconds
    n_ramp = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            wl.launch()
        n_ramp += 8
        torch.cuda.synchronize()
    for _ in range(warmup):
        wl.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        wl.launch()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    # per-launch spread (events between launches add a small gap; diagnostic only)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        wl.launch()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    w = wl.w
    r = {"ms_per_step": total_ms / steps, "kernel_ms_avg": total_ms / steps,
         "kernel_ms_median": statistics.median(per), "kernel_ms_min": min(per),
         "kernel_ms_max": max(per), "wall_s": wall, "ramp_launches": n_ramp}
    r["tflops"] = w.flops / (r["ms_per_step"] * 1e-3) / 1e12
    r["kernel_tflops"] = w.flops / (r["kernel_ms_avg"] * 1e-3) / 1e12
    return r


def launch_stats(wl):
    """One launch with the kernel's statistics counters: the fraction of (wave, tile) steps
    after each wave's first that skipped the O rescale, and the mean shader clock over the
    workgroups' lifetimes (shader cycles / 100 MHz reference ticks)."""
    import torch
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    wl.launch(stats=stats)
    torch.cuda.synchronize()
    s, r, cycles, ticks = (int(x) for x in stats.cpu())
    skip = (1.0 - r / s) if s else None
    ghz = (cycles / ticks * 0.1) if ticks else None
    return skip, ghz


def rates():
    """Issue rates of the softmax's exponential options, the MFMA and the LDS reads, as
    nanoseconds per wave instruction per SIMD (best of 5 launches)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_forward_tiled_amd", "libattn_probes.so"))
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.probe_rate.argtypes = [P, I, I, I, P]
    lib.probe_mfma_rate.argtypes = [P, I, I, P]
    lib.probe_lds_rate.argtypes = [P, I, I, I, P]
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    simds = 4 * ncu

    def best(fn):
        assert fn() == 0
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = 1e9
        for _ in range(5):
            a.record()
            assert fn() == 0
            b.record()
            torch.cuda.synchronize()
            t = min(t, a.elapsed_time(b) * 1e6)   # ns
        return t

    out_rates = {}
    iters = 2048
    for wps in (2, 4):                  # 256-thread blocks: 4 waves, one per SIMD
        blocks = ncu * wps
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        waves_per_simd = blocks * 4 / simds
        for mode, name in ((0, "exp2_hw_plus_sub"), (1, "exp2_cubic_plus_sub"), (2, "fma")):
            ns = best(lambda: lib.probe_rate(out.data_ptr(), blocks, iters, mode, None))
            out_rates[f"{name}/waves_per_simd={wps}"] = ns / (waves_per_simd * iters * 8)
        ns = best(lambda: lib.probe_mfma_rate(out.data_ptr(), blocks, iters, None))
        per = ns / (waves_per_simd * iters * 4)
        out_rates[f"mfma_32x32x16_bf16/waves_per_simd={wps}"] = per
        out_rates[f"mfma_tflops/waves_per_simd={wps}"] = 32768 / per * simds / 1e3
        for mode, name, nbytes in ((0, "ds_read_b128_GBps_per_cu", 16),
                                   (1, "ds_read_b64_tr_b16_GBps_per_cu", 8)):
            ns = best(lambda: lib.probe_lds_rate(out.data_ptr(), blocks, iters, mode, None))
            out_rates[f"{name}/waves_per_simd={wps}"] = blocks * 256 * iters * 8 * nbytes / ns / ncu
        del out
    power = clock_under_load(lib, ncu)
    return {"unit": "ns per wave instruction per SIMD (element-step for the exp2 rows)",
            "rates": {k: round(v, 4) for k, v in out_rates.items()},
            "clock_under_load": power,
            "mfma_valu_overlap": mfma_valu_overlap(lib, ncu)}


def mfma_valu_overlap(lib, ncu, iters=20000):
    """SIMD cycles per bf16 MFMA (32x32x16) when each MFMA is followed by V independent fp32
    FMAs, at one and at two waves per SIMD: how much VALU work hides under the matrix unit.
    An MFMA alone takes 32 cycles; the FMAs alone take 4 cycles each."""
    import ctypes
    import torch
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.probe_overlap.argtypes = [P, P, I, I, I, I, P]
    out = torch.empty(ncu * 512, dtype=torch.float32, device="cuda")
    res = {}
    for threads in (256, 512):
        for v in (0, 4, 8, 12, 16):
            stats = torch.zeros(2, dtype=torch.int64, device="cuda")

            def go(st):
                assert lib.probe_overlap(out.data_ptr(), st.data_ptr(), ncu, threads, iters, v,
                                         None) == 0
            go(stats)
            torch.cuda.synchronize()
            best = 1e30
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                go(stats)
                b.record()
                torch.cuda.synchronize()
                best = min(best, a.elapsed_time(b))
            cyc, ticks = (int(x) for x in stats.cpu())
            ghz = cyc / ticks * 0.1
            per_simd = (threads // 256) * iters * 4
            res[f"waves_per_simd={threads // 256}/fma_per_mfma={v}"] = {
                "simd_cycles_per_mfma": round(best * 1e-3 * ghz * 1e9 / per_simd, 1),
                "clock_ghz": round(ghz, 3)}
    return res


def clock_under_load(lib, ncu, seconds=1.0, iters=8000):
    """The bf16 MFMA rate and the clock the chip holds with two waves per SIMD issuing MFMAs
    back to back on random-data operands (mode 0), with every A operand read from LDS
    (mode 1), and with about 5 softmax-like VALU instructions per MFMA on top (mode 2)."""
    import ctypes
    import numpy as np
    import torch
    import synth
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.probe_power.argtypes = [P, P, P, I, I, I, P]
    src = torch.from_numpy(synth.normal_bf16((16384,), 77, 1.0).view(np.int16)).cuda()
    out = torch.empty(ncu * 512, dtype=torch.float32, device="cuda")
    stats = torch.zeros(2, dtype=torch.int64, device="cuda")
    flops = ncu * 8 * iters * 8 * 32768.0
    res = {}
    for mode, name in ((0, "mfma_random_operands"), (1, "mfma_lds_operands"),
                       (2, "mfma_lds_operands_plus_5_valu")):
        def go(st=None):
            assert lib.probe_power(src.data_ptr(), out.data_ptr(),
                                   (st if st is not None else stats).data_ptr(), ncu, iters,
                                   mode, None) == 0
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(4):
                go()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            go()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 10
        st = torch.zeros(2, dtype=torch.int64, device="cuda")
        go(st)
        torch.cuda.synchronize()
        cyc, ticks = (int(x) for x in st.cpu())
        ghz = cyc / ticks * 0.1
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "clock_ghz": round(ghz, 3),
                     "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1),
                     "pct_of_peak_at_clock": round(100 * tf / (PEAK_BF16_TFLOPS * ghz /
                                                                PEAK_CLOCK_GHZ), 1)}
    return res


def lds_patterns():
    """Runs the LDS access-pattern probe (one wave, 4096 accesses each) over the MXFP8
    kernel's operand-read and staging-write maps, and over alternative layouts, one dispatch
    per pattern in the printed order.  Under `rocprofv3 --pmc SQ_LDS_BANK_CONFLICT` the
    counter of each dispatch / 4096 is the conflict cycles of one access."""
    import ctypes
    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_forward_tiled_amd", "libattn_probes.so"))
    lib.probe_lds_pattern.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p]
    lanes = np.arange(64)
    n32, half = lanes % 32, lanes // 32

    def krow8(mb, m):       # K row read by MFMA row m of key block mb (MXFP8 kernel)
        return 32 * mb + 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3)

    def kpos8(r):           # the MXFP8 kernel's reordered K row position
        return r ^ (((r >> 4) & 1) << 3)

    layouts = {"rows_reordered_144": lambda r, c: kpos8(r) * 144 + 16 * c,
               "rows_natural_144": lambda r, c: r * 144 + 16 * c}
    pats = [("linear", 0, 16 * lanes)]
    for name, f in layouts.items():
        for mb in (0, 1):
            for c0 in (0, 2, 4, 6):
                pats.append((f"K_read_{name}_block{mb}_chunk{c0}", 0,
                             np.array([f(krow8(mb, int(n)), c0 + int(hh))
                                       for n, hh in zip(n32, half)])))
        pats.append((f"K_write_{name}", 1, np.array([f(int(t >> 3), int(t & 7)) for t in lanes])))
    pats.append(("V_read_80", 0, n32 * 80 + 16 * half))
    pats.append(("V_write_80_consecutive_columns", 1,
                 np.array([(t >> 2) * 80 + 16 * (t & 3) for t in lanes])))
    pats.append(("V_write_80_columns_four_apart", 1,
                 np.array([(((t >> 4) & 3) + 4 * ((t >> 2) & 3) + 16 * (t >> 6)) * 80 +
                           16 * (t & 3) for t in lanes])))
    out = torch.zeros(64, dtype=torch.float32, device="cuda")
    for name, write, a in pats:
        a = np.asarray(a, dtype=np.int64)
        assert a.shape == (64,) and (a % 16 == 0).all() and a.min() >= 0 and a.max() < 32768
        at = torch.from_numpy(a.astype(np.int32)).cuda()
        assert lib.probe_lds_pattern(at.data_ptr(), out.data_ptr(), 4096, write, None) == 0
        torch.cuda.synchronize()
    return {"dispatch_order": [(name, "write" if w else "read") for name, w, _ in pats],
            "accesses_per_dispatch": 4096}


def cpu_baseline(w, budget_s=10.0):
    """The float64 oracle, as it stands, on whole (batch, head) slices of the same workload
    (the block-scaled workloads run the oracle's emulation of their quantisation)."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    if w.fmt == "bf16":
        qb, kb, vb = w.make()
        q, k, v = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))

        def one(b, h):
            oracle.attention_head(q, k, v, w.causal, w.scale, b, h)
    else:
        import numpy as np
        q, k, v = w.make()
        group = w.Hq // w.Hkv
        mod, rows_fn = ((oracle.mx, oracle.mx.directp_rows) if w.fmt == "mxfp4"
                        else (oracle.mxfp8, oracle.mxfp8.fp8p_rows))

        def one(b, h):
            t = mod.quantize_inputs(q[b:b + 1, h:h + 1], k[b:b + 1, h // group:h // group + 1],
                                    v[b:b + 1, h // group:h // group + 1])
            for r0 in range(0, w.N, 256):
                rows = np.arange(r0, min(w.N, r0 + 256))
                rows_fn(t["q"][0, 0, rows], t["k"][0, 0], t["v"][0, 0], rows, w.causal, w.scale)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b, h = heads[done % len(heads)]
        one(b, h)
        done += 1
    el = time.perf_counter() - t0
    flops = w.flops * done / len(heads)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} (batch, head) slices of {w.name} ({len(heads)} per step), "
                      f"float64 numpy, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--warmup-seconds", type=float, default=0.5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--exp", default="hw", choices=["hw", "poly", "mix"])
    ap.add_argument("--poly-frac", type=float, default=0.5,
                    help="with --exp mix: fraction of the exponentials on the cubic")
    ap.add_argument("--tau", type=float, default=8.0)
    ap.add_argument("--extra", default="3,5,6",
                    help="other workloads to time (comma list, '' for none), e.g. 2,3,5")
    ap.add_argument("--docs", type=int, default=0,
                    help="also time the workload split into this many equal packed documents "
                         "(every format; TFLOP/s count 4*d flop per visible pair)")
    ap.add_argument("--window", type=int, default=0,
                    help="also time the workload with this sliding window (every format); its "
                         "TFLOP/s count 4*d flop per visible (query, key) pair")
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="also time the workload with soft-capping C (bf16 only)")
    ap.add_argument("--alibi", action="store_true",
                    help="also time the workload with ALiBi slopes 2^(-8h/H) (bf16 only)")
    ap.add_argument("--bwd", action="store_true",
                    help="also time the bf16 backward (dQ, dK, dV) on the workload; TFLOP/s "
                         "count 2.5x the forward's FLOPs (five products)")
    ap.add_argument("--compare-exp", action="store_true",
                    help="also time the headline workload with the other exp modes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="bench",
                    choices=["bench", "launch", "copy", "rates", "lds-patterns"])
    ap.add_argument("--copy-mib", type=int, default=1024)
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

    if args.mode == "rates":
        print(json.dumps(rates()), flush=True)
        return

    if args.mode == "lds-patterns":
        print(json.dumps(lds_patterns()), flush=True)
        return

    if args.mode == "copy":
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_mib} MiB x {args.steps}")
        return

    w = synth.workload(args.config)

    if args.mode == "launch":
        off = ([round(x * w.N / args.docs) for x in range(args.docs + 1)] if args.docs
               else None)
        if args.bwd:
            wl = BwdWorkload(w, window=args.window, doc_offsets=off)
        elif (args.window or off) and w.fmt == "bf16":
            wl = Workload(w, args.exp, args.tau, args.poly_frac, window=args.window,
                          doc_offsets=off)
        else:
            wl = make_workload(w, args.exp, args.tau, args.poly_frac)
        for _ in range(args.steps):
            wl.launch()
        torch.cuda.synchronize()
        log(f"launched {w.name} x {args.steps}")
        return

    log(f"timing {w.name}: ramp {args.warmup_seconds} s, warmup {args.warmup}, steps {args.steps}")
    wl = make_workload(w, args.exp, args.tau, args.poly_frac)
    t = time_workload(wl, args.steps, args.warmup, args.warmup_seconds)
    skip, ghz = launch_stats(wl)
    acc = mx_accuracy(wl) if w.fmt != "bf16" else None
    del wl
    torch.cuda.empty_cache()
    kernel_tf = t["kernel_tflops"]
    props = torch.cuda.get_device_properties(0)

    extra = {"kernel_ms_avg": t["kernel_ms_avg"], "kernel_ms_median": t["kernel_ms_median"],
             "kernel_ms_min": t["kernel_ms_min"], "kernel_ms_max": t["kernel_ms_max"],
             "pct_of_bf16_peak": 100.0 * t["tflops"] / PEAK_BF16_TFLOPS,
             "skip_ratio": skip, "skip_ratio_model": skip_ratio_model(w.name)
                                   if args.tau == 8.0 else None,
             "clock_ghz": ghz,
             "pct_of_bf16_peak_at_clock": (100.0 * t["tflops"] / (PEAK_BF16_TFLOPS * ghz / PEAK_CLOCK_GHZ)
                                           if ghz else None),
             "exp_mode": {"bf16": args.exp, "mxfp4": "directp", "mxfp8": "hw"}[w.fmt],
             "poly_frac": args.poly_frac if args.exp == "mix" else None,
             "tau": args.tau, "kernel_hash": kernel_hash(w.fmt), "device": props.name,
             "compute_units": props.multi_processor_count, "workloads": {}}
    if w.fmt != "bf16":
        extra[f"pct_of_{w.fmt[2:]}_peak"] = 100.0 * t["tflops"] / PEAKS[w.fmt]
        extra["accuracy"] = acc
    if args.compare_exp and w.fmt == "bf16":
        for other, frac in (("hw", None), ("poly", None), ("mix", 0.25), ("mix", 0.5), ("mix", 0.75)):
            if other == args.exp and (other != "mix" or frac == args.poly_frac):
                continue
            tag = other if other != "mix" else f"mix{frac:g}"
            log(f"timing {w.name} with exp mode {tag}")
            wl = Workload(w, other, args.tau, frac)
            t2 = time_workload(wl, args.steps, args.warmup, args.warmup_seconds)
            _, g2 = launch_stats(wl)
            del wl
            extra["workloads"][f"{w.name}/exp={tag}"] = {
                "tflops": round(t2["tflops"], 2), "ms": round(t2["ms_per_step"], 4),
                "clock_ghz": g2}
    for idx in [int(x) for x in args.extra.split(",") if x.strip()]:
        wx = synth.workload(idx)
        if idx == args.config:
            continue
        log(f"timing {wx.name}")
        wl = make_workload(wx, args.exp, args.tau, args.poly_frac)
        tx = time_workload(wl, max(5, args.steps // 2), args.warmup, args.warmup_seconds)
        sx, gx = launch_stats(wl)
        ax = mx_accuracy(wl) if wx.fmt != "bf16" else None
        del wl
        torch.cuda.empty_cache()
        extra["workloads"][wx.name] = {
            "tflops": round(tx["tflops"], 2), "ms": round(tx["ms_per_step"], 4),
            "kernel_ms_avg": round(tx["kernel_ms_avg"], 4),
            "pct_of_bf16_peak": round(100.0 * tx["tflops"] / PEAK_BF16_TFLOPS, 2),
            "skip_ratio": sx,
            "skip_ratio_model": skip_ratio_model(wx.name) if args.tau == 8.0 else None,
            "clock_ghz": gx}
        if wx.fmt != "bf16":
            extra["workloads"][wx.name][f"pct_of_{wx.fmt[2:]}_peak"] = round(
                100.0 * tx["tflops"] / PEAKS[wx.fmt], 2)
            extra["workloads"][wx.name]["accuracy"] = ax

    masked_mx = {"mxfp4": Mxfp4Workload, "mxfp8": Mxfp8Workload}
    if args.window:
        log(f"timing {w.name} with window {args.window}")
        wl = (Workload(w, args.exp, args.tau, args.poly_frac, window=args.window)
              if w.fmt == "bf16" else masked_mx[w.fmt](w, args.tau, window=args.window))
        tw = time_workload(wl, args.steps, args.warmup, args.warmup_seconds)
        del wl
        torch.cuda.empty_cache()
        pairs = visible_pairs(w.N, w.causal, args.window)
        fl = 4.0 * w.d * w.B * w.Hq * pairs
        extra["workloads"][f"{w.name}/window={args.window}"] = {
            "tflops_visible": round(fl / (tw["kernel_ms_avg"] * 1e-3) / 1e12, 2),
            "kernel_ms_avg": round(tw["kernel_ms_avg"], 4),
            "visible_pairs_per_head": pairs,
            "time_vs_no_window": round(tw["kernel_ms_avg"] / t["kernel_ms_avg"], 4)}

    if args.docs:
        off = [round(x * w.N / args.docs) for x in range(args.docs + 1)]
        log(f"timing {w.name} as {args.docs} documents")
        wl = (Workload(w, args.exp, args.tau, args.poly_frac, doc_offsets=off)
              if w.fmt == "bf16" else masked_mx[w.fmt](w, args.tau, doc_offsets=off))
        td = time_workload(wl, args.steps, args.warmup, args.warmup_seconds)
        del wl
        torch.cuda.empty_cache()
        pairs = visible_pairs(w.N, w.causal, 0, off)
        fl = 4.0 * w.d * w.B * w.Hq * pairs
        extra["workloads"][f"{w.name}/docs={args.docs}"] = {
            "tflops_visible": round(fl / (td["kernel_ms_avg"] * 1e-3) / 1e12, 2),
            "kernel_ms_avg": round(td["kernel_ms_avg"], 4),
            "visible_pairs_per_head": pairs,
            "time_vs_one_document": round(td["kernel_ms_avg"] / t["kernel_ms_avg"], 4)}

    mods = []
    if args.softcap:
        mods.append((f"softcap={args.softcap:g}", {"softcap": args.softcap}))
    if args.alibi:
        mods.append(("alibi", {"alibi": True}))
    if args.softcap and args.alibi:
        mods.append((f"softcap={args.softcap:g}+alibi", {"softcap": args.softcap, "alibi": True}))
    if w.fmt == "bf16":
        for tag, kw in mods:
            log(f"timing {w.name} with {tag}")
            wl = Workload(w, "hw", args.tau, None, **kw)
            tm = time_workload(wl, args.steps, args.warmup, args.warmup_seconds)
            del wl
            torch.cuda.empty_cache()
            extra["workloads"][f"{w.name}/{tag}"] = {
                "tflops": round(tm["tflops"], 2),
                "kernel_ms_avg": round(tm["kernel_ms_avg"], 4),
                "time_vs_plain": round(tm["kernel_ms_avg"] / t["kernel_ms_avg"], 4)}

    if args.bwd and w.fmt == "bf16":
        log(f"timing the backward on {w.name}")
        wl = BwdWorkload(w)
        tb = time_workload(wl, args.steps, args.warmup, args.warmup_seconds)
        del wl
        torch.cuda.empty_cache()
        fl = 2.5 * w.flops
        extra["workloads"][f"{w.name}/bwd"] = {
            "tflops": round(fl / (tb["kernel_ms_avg"] * 1e-3) / 1e12, 2),
            "ms": round(tb["kernel_ms_avg"], 4),
            "pct_of_bf16_peak": round(100.0 * fl / (tb["kernel_ms_avg"] * 1e-3) / 1e12
                                      / PEAK_BF16_TFLOPS, 2),
            "flop_convention": "2.5x forward (dQ, dK, dV, S, dP); the kernels execute 3.5x "
                               "(S and dP recomputed in both the dK/dV and the dQ kernel)"}
        masked = []
        if args.window:
            masked.append((f"bwd/window={args.window}", args.window, None))
        if args.docs:
            masked.append((f"bwd/docs={args.docs}", 0,
                           [round(x * w.N / args.docs) for x in range(args.docs + 1)]))
        for tag, kw in mods:
            log(f"timing the backward on {w.name} with {tag}")
            wl = BwdWorkload(w, **kw)
            tm = time_workload(wl, args.steps, args.warmup, args.warmup_seconds)
            del wl
            torch.cuda.empty_cache()
            extra["workloads"][f"{w.name}/bwd/{tag}"] = {
                "tflops": round(2.5 * w.flops / (tm["kernel_ms_avg"] * 1e-3) / 1e12, 2),
                "ms": round(tm["kernel_ms_avg"], 4),
                "time_vs_plain_bwd": round(tm["kernel_ms_avg"] / tb["kernel_ms_avg"], 4)}
        for tag, win, off in masked:
            log(f"timing the backward on {w.name} with {tag[4:]}")
            wl = BwdWorkload(w, window=win, doc_offsets=off)
            tm = time_workload(wl, args.steps, args.warmup, args.warmup_seconds)
            del wl
            torch.cuda.empty_cache()
            pairs = visible_pairs(w.N, w.causal, win, off)
            fl = 2.5 * 4.0 * w.d * w.B * w.Hq * pairs
            extra["workloads"][f"{w.name}/{tag}"] = {
                "tflops_visible": round(fl / (tm["kernel_ms_avg"] * 1e-3) / 1e12, 2),
                "ms": round(tm["kernel_ms_avg"], 4),
                "visible_pairs_per_head": pairs,
                "time_vs_unmasked_bwd": round(tm["kernel_ms_avg"] / tb["kernel_ms_avg"], 4)}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host")
        cpu = cpu_baseline(w)

    peak = PEAKS[w.fmt]
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
        "dtype": w.fmt,
        "data": "synthetic",
        "config": dict(w.describe()),
        "roofline": {"bound": "mfma", "achieved": round(kernel_tf, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(kernel_tf / peak, 4),
                     "traffic": load_traffic(w.name, w.fmt)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Writes skip_ratio.json: the skip-ratio model (oracle.skipsim) run over every head of the
bf16 workloads, at tau = 8 and the kernel's grouping (32 query rows, 64-key tiles).

The bench reports this beside the kernel's own counters; it calls only oracle/ and synth/.
Run:  python tests/golden/make_skip_ratio.py
"""

import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import skipsim  # noqa: E402

TAU = 8.0


def main():
    out = {}
    for idx in (2, 3, 4):
        w = synth.workload(idx)
        t0 = time.perf_counter()
        qb, kb, vb = w.make()
        q, k = synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb)
        group = w.Hq // w.Hkv
        steps = fires = 0
        for b in range(w.B):
            for h in range(w.Hq):
                s, f = skipsim.skip_counts(q[b, h], k[b, h // group], w.scale, TAU, w.causal)
                steps += s
                fires += f
        out[w.name] = {"tau": TAU, "rows_per_group": 32, "keys_per_tile": 64,
                       "steps": steps, "rescales": fires, "skip_ratio": 1.0 - fires / steps}
        print(f"{w.name}: steps {steps} rescales {fires} skip {1 - fires / steps:.4f} "
              f"({time.perf_counter() - t0:.0f} s)", flush=True)
    with open(os.path.join(HERE, "skip_ratio.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()

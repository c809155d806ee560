"""Writes mx_reference_rows.npz: reference output rows of the MXFP4 and MXFP8 workloads
(B1 H24 N16384 d128, non-causal), for the bench's accuracy report.

For three heads and 40 fixed query rows of each workload it stores, as float32:
  exact     the exact attention rows (oracle.exact) on the unquantised fp32 inputs;
  emulated  the oracle's step-by-step emulation of the block-scaled path (oracle.mx
            Direct-P, oracle.mxfp8) on the quantised inputs.
The bench compares the GPU output with both: the mean row cosine against `exact` (the
explainer page's accuracy measure) and the relative error against `emulated` (parity).
Calls only oracle/ and synth/.  Run:  python tests/golden/make_mx_reference_rows.py
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import mx, mxfp8  # noqa: E402


def rows_for(n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 255, 256, n - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, n, 40 - len(fixed))]))


def main():
    out = {}
    for idx, mod, rows_fn in ((5, mx, mx.directp_rows), (6, mxfp8, mxfp8.fp8p_rows)):
        w = synth.workload(idx)
        q, k, v = w.make()
        heads = np.array([0, w.Hq // 2, w.Hq - 1])
        rows = rows_for(w.N, idx)
        exact = np.empty((len(heads), len(rows), w.d), np.float32)
        emul = np.empty_like(exact)
        for i, h in enumerate(heads):
            g = h // (w.Hq // w.Hkv)
            eo, _ = oracle.attention_rows(q[:, h:h + 1].astype(np.float64),
                                          k[:, g:g + 1].astype(np.float64),
                                          v[:, g:g + 1].astype(np.float64), w.causal, w.scale,
                                          0, 0, rows)
            exact[i] = eo
            t = mod.quantize_inputs(q[:, h:h + 1, rows], k[:, g:g + 1], v[:, g:g + 1])
            ro, _, _ = rows_fn(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], rows, w.causal,
                               w.scale)
            emul[i] = ro
            print(f"{w.name} head {h}: done", flush=True)
        out[f"{w.name}/heads"] = heads
        out[f"{w.name}/rows"] = rows
        out[f"{w.name}/exact"] = exact
        out[f"{w.name}/emulated"] = emul
    np.savez_compressed(os.path.join(HERE, "mx_reference_rows.npz"), **out)


if __name__ == "__main__":
    main()

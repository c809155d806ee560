"""Helpers for the GPU tests: device upload of synth inputs and parity metrics."""

import sys

import numpy as np


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cuda_ok():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def to_dev_bf16(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def rel_rms(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


# tolerances for the bf16 path (fixed by the workload definition)
BF16_O_RELRMS = 5e-3
BF16_LSE_ABS = 1e-3
# tolerance for the MXFP4 Direct-P path against the emulating oracle
MXFP4_O_RELRMS = 0.1

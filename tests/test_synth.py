"""The seeded input generator: bf16 rounding agrees with torch's fp32 -> bf16 conversion."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    x = synth.normal_f32((4096,), 5, 3.0)
    extra = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, -0.0, 65504.0, 1e-40],
                     dtype=np.float32)
    x = np.concatenate([x, extra])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_seeded_and_shaped():
    w = synth.workload(3)
    assert (w.B, w.Hq, w.Hkv, w.N, w.d, w.causal) == (1, 32, 8, 8192, 128, True)
    a = synth.normal_bf16((2, 3, 4), 11)
    b = synth.normal_bf16((2, 3, 4), 11)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    assert synth.workload(1).flops == 4 * 1 * 2 * 256 * 256 * 64
    assert synth.workload(2).flops == 2 * 4 * 16 * 2048 * 2048 * 128

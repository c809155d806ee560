"""The GPU parity gates themselves (CPU only): the per-row gate rejects what the whole-tensor
relative RMS lets through.

Worked case: the causal B1 H4 N1000 d128 shape of the bf16 shape sweep.  A copy of the
oracle's O with the noise the kernel's bf16 weights leave (relRMS 1.1e-3, as measured on the
device for this shape) passes both gates; one element moved by 1.0 (about 3x the typical
element) or one whole row moved by 0.09 per element still passes the relRMS gate of 5e-3,
and the per-row gate rejects both."""

import numpy as np

import oracle
import synth
from synth.configs import random_case
from gpu_util import BF16_O_RELRMS, BF16_O_ROW, gate, rel_rms, row_rel_max


def _correct_and_noisy():
    qb, kb, vb = random_case(4 + 4 + 1000 + 128 + 1 + 7, 1, 4, 4, 1000, 128, sigma=1.5)
    q, k, v = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    o, _ = oracle.attention(q, k, v, True, 128 ** -0.5)
    rng = np.random.default_rng(0)
    # each output moved by a relative 2^-9 / sqrt(3) = 1.1e-3 in RMS, the relRMS the kernel
    # measures on this shape
    noisy = o * (1.0 + rng.uniform(-2.0 ** -9, 2.0 ** -9, o.shape))
    return o, noisy


def test_correct_output_passes_both_gates():
    o, noisy = _correct_and_noisy()
    gate(noisy, o, BF16_O_RELRMS, BF16_O_ROW, "noisy copy")


def test_one_bad_element_is_rejected():
    o, noisy = _correct_and_noisy()
    bad = noisy.copy()
    bad[0, 2, 500, 17] += 1.0
    assert rel_rms(bad, o) <= BF16_O_RELRMS          # the whole-tensor gate misses it
    assert row_rel_max(bad, o) > BF16_O_ROW          # the per-row gate does not


def test_one_bad_row_is_rejected():
    o, noisy = _correct_and_noisy()
    bad = noisy.copy()
    bad[0, 1, 777, :] += 0.09
    assert rel_rms(bad, o) <= BF16_O_RELRMS
    assert row_rel_max(bad, o) > BF16_O_ROW


def test_small_rows_use_the_floor():
    """A row whose reference is near zero is measured against a tenth of the RMS row norm,
    so a tiny absolute error there is not an infinite relative one."""
    ref = np.ones((10, 8))
    ref[3] = 1e-12
    got = ref.copy()
    got[3] += 1e-6
    assert row_rel_max(got, ref) < 1e-4
    got[3] += 0.5
    assert row_rel_max(got, ref) > 0.5

"""bf16 forward on the GPU (through the C ABI) against the float64 oracle.

Tolerances: relative RMS of O <= 5e-3 and max |LSE error| <= 1e-3.  Small and
ragged shapes are compared element by element on every output; the full-size
workloads are compared on sampled query rows that the oracle computes one by
one, in the same launch configuration the bench times.
"""

import numpy as np
import pytest

import oracle
import synth
from synth.configs import random_case
from gpu_util import BF16_LSE_ABS, BF16_O_RELRMS, BF16_O_ROW, cuda_ok, gate, log, to_dev_bf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _run(qb, kb, vb, causal, scale, **kw):
    import torch
    import exact_attention_forward_tiled_amd as fa
    q, k, v = to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb)
    B, Hq, N, d = q.shape
    # pre-fill outputs with NaN so a tile the kernel forgot to write shows up
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd(q, k, v, causal=causal, scale=scale, out=(o, lse), **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _check(o, lse, ro, rl, what, lse_tol=BF16_LSE_ABS):
    """O: whole-tensor relRMS and the per-row gate; LSE: every row within lse_tol."""
    assert not np.isnan(o).any() and not np.isnan(lse).any(), f"{what}: unwritten outputs"
    gate(o, ro, BF16_O_RELRMS, BF16_O_ROW, f"{what} O")
    e = float(np.max(np.abs(lse - rl)))
    log(f"  {what}: max|dLSE|={e:.3e}")
    assert e <= lse_tol, (what, e)


SMALL = [
    # B, Hq, Hkv, N, d, causal
    (1, 2, 2, 256, 64, False),
    (1, 2, 2, 256, 64, True),
    (1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 128, True),
    (1, 3, 3, 65, 128, False),
    (2, 4, 2, 129, 64, True),
    (1, 2, 1, 200, 128, True),
    (1, 2, 2, 333, 128, False),
    (1, 8, 2, 512, 128, True),
    (2, 2, 2, 127, 128, True),
    (1, 4, 4, 1000, 128, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dHq%dHkv%dN%dd%d%s" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n"))
@pytest.mark.parametrize("mode", [("hw", 8.0), ("hw", 0.0), ("poly", 8.0), ("mix", 8.0)],
                         ids=lambda m: f"{m[0]}-tau{m[1]:g}")
def test_small_shapes(case, mode):
    B, Hq, Hkv, N, d, causal = case
    qb, kb, vb = random_case(sum(case[:5]) + 7, B, Hq, Hkv, N, d, sigma=1.5)
    scale = 1.0 / np.sqrt(d)
    log(f"case {case} mode {mode}")
    o, lse = _run(qb, kb, vb, causal, scale, exp_mode=mode[0], tau=mode[1],
                  poly_frac=0.5 if mode[0] == "mix" else None)
    ro, rl = oracle.attention(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                              synth.bf16_bits_to_f64(vb), causal, scale)
    _check(o, lse, ro, rl, f"{case} {mode}")


@pytest.mark.parametrize("frac", [0.25, 0.75])
def test_mix_fractions(frac):
    """The other two split points of the mixed exponential (0.5 runs in the shape sweep)."""
    qb, kb, vb = random_case(91, 1, 4, 2, 700, 128, sigma=1.5)
    scale = 1.0 / np.sqrt(128)
    log(f"mix poly_frac {frac}")
    for causal in (False, True):
        o, lse = _run(qb, kb, vb, causal, scale, exp_mode="mix", poly_frac=frac)
        ro, rl = oracle.attention(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                                  synth.bf16_bits_to_f64(vb), causal, scale)
        _check(o, lse, ro, rl, f"mix {frac} causal={causal}")


def test_workload_1_full():
    w = synth.workload(1)
    qb, kb, vb = w.make()
    log(f"workload {w.name}")
    o, lse = _run(qb, kb, vb, w.causal, w.scale)
    ro, rl = oracle.attention(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                              synth.bf16_bits_to_f64(vb), w.causal, w.scale)
    _check(o, lse, ro, rl, w.name)


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_full_size_sampled_rows(idx):
    """Full-size workloads: sampled rows of several heads against the oracle's row-wise definition."""
    w = synth.workload(idx)
    qb, kb, vb = w.make()
    log(f"workload {w.name}")
    o, lse = _run(qb, kb, vb, w.causal, w.scale)
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    rng = np.random.default_rng(idx)
    heads = [(0, 0), (w.B - 1, w.Hq - 1), (rng.integers(w.B), rng.integers(w.Hq))]
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, w.N - 1],
                                     rng.integers(0, w.N, 40)]))
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b, h in heads:
        ro, rl = oracle.attention_rows(q64, k64, v64, w.causal, w.scale, int(b), int(h), rows)
        got_o.append(o[b, h, rows]); got_l.append(lse[b, h, rows])
        ref_o.append(ro); ref_l.append(rl)
    _check(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o),
           np.concatenate(ref_l), w.name)
    assert not np.isnan(o).any() and not np.isnan(lse).any()


def test_constant_v_gives_one():
    qb, kb, _ = random_case(31, 1, 4, 2, 300, 128, sigma=2.0)
    vb = np.full((1, 2, 300, 128), 0x3F80, dtype=np.uint16)      # bf16 1.0
    for causal in (False, True):
        o, _ = _run(qb, kb, vb, causal, 0.09)
        assert np.max(np.abs(o - 1.0)) < 4e-3


def test_zero_query_prefix_mean():
    _, kb, vb = random_case(32, 1, 2, 2, 257, 64)
    qb = np.zeros((1, 2, 257, 64), dtype=np.uint16)
    v64 = synth.bf16_bits_to_f64(vb)
    for causal in (False, True):
        o, lse = _run(qb, kb, vb, causal, 0.125)
        if causal:
            ref = np.cumsum(v64, axis=2) / np.arange(1, 258)[None, None, :, None]
            ref_l = np.log(np.arange(1, 258))[None, None, :]
        else:
            ref = np.broadcast_to(v64.mean(axis=2, keepdims=True), v64.shape)
            ref_l = np.full((1, 2, 257), np.log(257.0))
        gate(o, ref, BF16_O_RELRMS, BF16_O_ROW, f"zero query causal={causal}")
        assert np.max(np.abs(lse - ref_l)) < 1e-4


def test_causal_first_row_is_first_value():
    qb, kb, vb = random_case(33, 1, 2, 2, 130, 128)
    o, lse = _run(qb, kb, vb, True, 0.088)
    v64 = synth.bf16_bits_to_f64(vb)
    q64, k64 = synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb)
    assert np.max(np.abs(o[:, :, 0] - v64[:, :, 0])) < 1e-6
    s0 = 0.088 * np.einsum("bhd,bhd->bh", q64[:, :, 0], k64[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - s0)) < 1e-5


def test_gqa_equals_repeated_heads_bitwise():
    qb, kb, vb = random_case(34, 1, 8, 2, 200, 128)
    for causal in (False, True):
        o1, l1 = _run(qb, kb, vb, causal, 0.088)
        o2, l2 = _run(qb, np.repeat(kb, 4, axis=1), np.repeat(vb, 4, axis=1), causal, 0.088)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_deterministic():
    qb, kb, vb = random_case(35, 2, 4, 4, 700, 128, sigma=3.0)
    runs = [_run(qb, kb, vb, True, 0.088) for _ in range(3)]
    for o, l in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(l, runs[0][1])


def test_scale_sign_and_zero():
    qb, kb, vb = random_case(36, 1, 2, 2, 150, 64)
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    for scale in (-0.125, 0.0, 0.5):
        for causal in (False, True):
            o, lse = _run(qb, kb, vb, causal, scale)
            ro, rl = oracle.attention(q64, k64, v64, causal, scale)
            _check(o, lse, ro, rl, f"scale={scale} causal={causal}")


def test_extreme_logits():
    """Logits far past 500 (the range-guard regime named in "Hardware-Aware FP4
    FlashAttention-4", section "1. Direct-P para Inferencia Directa").  The online softmax
    keeps every weight relative to the running max, so nothing under- or overflows and O
    keeps its tolerance.  The LSE moves with the scores' own fp32 summation error, which
    grows with their size: |dS| <= d u sum_k |q_k k_k| for any summation order (u = 2^-24),
    and |dLSE| <= scale max |dS|, so the LSE bound adds that term to the usual 1e-3."""
    qb, kb, vb = random_case(38, 1, 2, 2, 256, 128, sigma=6.0)
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    scale = 1.0
    logits = np.einsum("bhid,bhjd->bhij", q64, k64) * scale
    assert np.abs(logits).max() > 500
    absum = np.einsum("bhid,bhjd->bhij", np.abs(q64), np.abs(k64))
    bound = BF16_LSE_ABS + scale * 128 * 2.0 ** -24 * absum.max()
    log(f"max |logit| {np.abs(logits).max():.0f}; LSE bound {bound:.3e}")
    for causal in (False, True):
        o, lse = _run(qb, kb, vb, causal, scale)
        ro, rl = oracle.attention(q64, k64, v64, causal, scale)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        _check(o, lse, ro, rl, f"extreme logits causal={causal}", lse_tol=bound)


WINDOW_CASES = [
    # B, Hq, Hkv, N, d, causal, window
    (1, 2, 2, 256, 64, True, 1),
    (1, 2, 2, 256, 128, False, 1),
    (1, 2, 1, 333, 128, True, 31),
    (1, 2, 2, 517, 128, False, 64),
    (2, 4, 2, 700, 64, True, 100),
    (1, 2, 2, 1000, 128, True, 200),
    (1, 3, 3, 1000, 128, False, 257),
    (1, 2, 2, 1100, 128, True, 1099),
    (1, 1, 1, 2048, 128, True, 513),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "B%dHq%dHkv%dN%dd%d%sW%d" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6]))
def test_sliding_window(case):
    """Sliding window against the oracle's band mask (key j visible from query i only when
    i - W < j, and j < i + W without the causal mask)."""
    B, Hq, Hkv, N, d, causal, W = case
    qb, kb, vb = random_case(40 + W, B, Hq, Hkv, N, d)
    log(f"case {case}")
    o, lse = _run(qb, kb, vb, causal, d ** -0.5, window=W)
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ro, rl = oracle.attention(q64, k64, v64, causal, d ** -0.5, window=W)
    _check(o, lse, ro, rl, f"window {W}")


def test_sliding_window_large_sampled_rows():
    """A long causal GQA problem with a 1024-key window: sampled rows of several heads."""
    B, Hq, Hkv, N, d, W = 1, 8, 2, 8192, 128, 1024
    qb, kb, vb = random_case(49, B, Hq, Hkv, N, d)
    o, lse = _run(qb, kb, vb, True, d ** -0.5, window=W)
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    rng = np.random.default_rng(49)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 1023, 1024, 1025, N - 1],
                                     rng.integers(0, N, 24)]))
    for h in (0, 3, Hq - 1):
        ro, rl = oracle.attention_rows(q64, k64, v64, True, d ** -0.5, 0, h, rows, window=W)
        _check(o[0, h, rows], lse[0, h, rows], ro, rl, f"head {h}")


def test_long_sequence_sampled_rows():
    """One head of N = 2^18 keys (non-causal, 64 MiB of K and of V), far past the workloads'
    lengths: sampled rows, both ends and tile edges included, against the oracle's rows."""
    B, Hq, Hkv, N, d = 1, 1, 1, 1 << 18, 128
    qb, kb, vb = random_case(61, B, Hq, Hkv, N, d)
    o, lse = _run(qb, kb, vb, False, d ** -0.5)
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    rng = np.random.default_rng(61)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, N - 257, N - 65, N - 64, N - 1],
                                     rng.integers(0, N, 10)]))
    ro, rl = oracle.attention_rows(q64, k64, v64, False, d ** -0.5, 0, 0, rows)
    _check(o[0, 0, rows], lse[0, 0, rows], ro, rl, "N = 2^18")


def test_long_sequence_window_sampled_rows():
    """Causal GQA over N = 2^19 keys with a 2048-key window (the band bookkeeping and row
    offsets at half a million rows): sampled rows of both query heads."""
    B, Hq, Hkv, N, d, W = 1, 2, 1, 1 << 19, 128, 2048
    qb, kb, vb = random_case(62, B, Hq, Hkv, N, d)
    o, lse = _run(qb, kb, vb, True, d ** -0.5, window=W)
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    rng = np.random.default_rng(62)
    rows = np.unique(np.concatenate([[0, 1, W - 1, W, W + 1, N - 257, N - 1],
                                     rng.integers(0, N, 9)]))
    for h in range(Hq):
        ro, rl = oracle.attention_rows(q64, k64, v64, True, d ** -0.5, 0, h, rows, window=W)
        _check(o[0, h, rows], lse[0, h, rows], ro, rl, f"N = 2^19, W {W}, head {h}")


MOD_CASES = [
    # B, Hq, Hkv, N, d, causal, softcap, alibi, window
    (1, 2, 2, 256, 128, False, 5.0, False, 0),
    (1, 2, 2, 333, 128, True, 5.0, False, 0),
    (1, 4, 2, 300, 128, True, 0.0, True, 0),
    (1, 4, 4, 517, 128, False, 0.0, True, 0),
    (1, 4, 1, 700, 64, True, 20.0, True, 0),
    (2, 2, 2, 129, 64, False, 2.0, True, 0),
    (1, 4, 2, 1000, 128, True, 30.0, True, 200),
]


@pytest.mark.parametrize("case", MOD_CASES, ids=lambda c: "B%dHq%dHkv%dN%dd%d%scap%gal%dW%d" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6], c[7], c[8]))
def test_score_modifications(case):
    """ALiBi (score - a_h |i - j|, one slope per query head) and soft-capping
    (C tanh(score / C)) against the oracle, alone, together and with a window."""
    import torch
    B, Hq, Hkv, N, d, causal, cap, use_alibi, W = case
    qb, kb, vb = random_case(60 + N, B, Hq, Hkv, N, d, sigma=2.0)
    slopes = 0.5 ** (np.arange(1, Hq + 1) * 8.0 / Hq) if use_alibi else None
    log(f"case {case}")
    o, lse = _run(qb, kb, vb, causal, d ** -0.5, window=W, softcap=cap,
                  alibi=None if slopes is None else
                  torch.tensor(slopes, dtype=torch.float32, device="cuda"))
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    # the kernel reads the slopes in float32: the oracle gets the same values
    ref_slopes = None if slopes is None else slopes.astype(np.float32).astype(np.float64)
    ro, rl = oracle.attention(q64, k64, v64, causal, d ** -0.5, window=W, softcap=cap,
                              alibi=ref_slopes)
    _check(o, lse, ro, rl, f"softcap {cap} alibi {use_alibi} window {W}")


DOC_CASES = [
    # B, Hq, Hkv, N, d, causal, offsets, window, alibi
    (1, 2, 2, 256, 128, False, [0, 256], 0, False),
    (1, 2, 2, 333, 128, True, [0, 100, 101, 333], 0, False),
    (2, 4, 2, 700, 64, False, [0, 64, 128, 511, 700], 0, False),
    (1, 2, 1, 1000, 128, True, [0, 17, 300, 301, 302, 900, 1000], 0, False),
    (1, 4, 4, 1000, 128, False, [0, 250, 520, 1000], 100, False),
    (1, 4, 2, 777, 128, True, [0, 5, 400, 777], 0, True),
]


@pytest.mark.parametrize("case", DOC_CASES, ids=lambda c: "B%dHq%dHkv%dN%dd%d%sD%dW%dal%d" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", len(c[6]) - 1, c[7], c[8]))
def test_document_masking(case):
    """Packed documents (keys visible only within the query's document) against the
    oracle, with the masks, a window and ALiBi."""
    import torch
    B, Hq, Hkv, N, d, causal, off, W, use_alibi = case
    qb, kb, vb = random_case(70 + N, B, Hq, Hkv, N, d)
    slopes = 0.5 ** (np.arange(1, Hq + 1) * 8.0 / Hq) if use_alibi else None
    log(f"case {case}")
    o, lse = _run(qb, kb, vb, causal, d ** -0.5, window=W,
                  docs=torch.tensor(off, dtype=torch.int32, device="cuda"),
                  alibi=None if slopes is None else
                  torch.tensor(slopes, dtype=torch.float32, device="cuda"))
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    ref_slopes = None if slopes is None else slopes.astype(np.float32).astype(np.float64)
    ro, rl = oracle.attention(q64, k64, v64, causal, d ** -0.5, window=W, docs=off,
                              alibi=ref_slopes)
    _check(o, lse, ro, rl, f"documents {off} window {W}")


def test_document_masking_large_sampled_rows():
    """N = 8192 holding 7 documents of mixed lengths, causal: sampled rows of several heads."""
    import torch
    B, Hq, Hkv, N, d = 1, 4, 2, 8192, 128
    off = [0, 1000, 1001, 3000, 4096, 4200, 7777, 8192]
    qb, kb, vb = random_case(79, B, Hq, Hkv, N, d)
    o, lse = _run(qb, kb, vb, True, d ** -0.5,
                  docs=torch.tensor(off, dtype=torch.int32, device="cuda"))
    q64, k64, v64 = (synth.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    rng = np.random.default_rng(79)
    rows = np.unique(np.concatenate([off[:-1], [x - 1 for x in off[1:]], rng.integers(0, N, 16)]))
    for h in (0, Hq - 1):
        ro, rl = oracle.attention_rows(q64, k64, v64, True, d ** -0.5, 0, h, rows, docs=off)
        _check(o[0, h, rows], lse[0, h, rows], ro, rl, f"head {h}")


def test_skip_ratio_stats():
    """The rescale counter against the skip-ratio model (oracle.skipsim: the tau rule over
    32-row groups and 64-key tiles in float64): the step count exactly, the rescale count
    within a few decisions (scores are fp32 in the kernel, so a tile max within rounding of
    m + tau can decide differently).  tau = 0 rescales on most steps, tau = 8 skips most."""
    import torch
    from oracle import skipsim
    w = synth.workload(4)
    qb, kb, vb = random_case(37, 1, 2, 2, 4096, 128, sigma=w.sigma_qk)
    q64, k64 = synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb)
    ratios = {}
    for tau in (0.0, 8.0):
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        import exact_attention_forward_tiled_amd as fa
        fa.fwd(to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb), causal=False,
               scale=w.scale, tau=tau, stats=stats)
        torch.cuda.synchronize()
        steps, resc, cycles, ticks = (int(x) for x in stats.cpu())
        assert steps == 2 * (4096 // 32) * (4096 // 64 - 1)
        # shader clock over the workgroups' lifetimes (100 MHz reference ticks)
        ghz = cycles / ticks * 0.1
        log(f"  mean shader clock {ghz:.3f} GHz")
        assert 0.3 < ghz < 3.0
        ratios[tau] = 1.0 - resc / steps
        m_steps = m_fires = 0
        for h in range(2):
            st, fi = skipsim.skip_counts(q64[0, h], k64[0, h], w.scale, tau, False)
            m_steps += st
            m_fires += fi
        log(f"  tau={tau}: steps={steps} rescales={resc} skip={ratios[tau]:.4f}; "
            f"model rescales={m_fires} skip={1 - m_fires / m_steps:.4f}")
        assert m_steps == steps
        assert abs(resc - m_fires) <= max(3, 0.002 * steps), (resc, m_fires)
    assert ratios[8.0] > ratios[0.0]


def test_skip_ratio_causal_model():
    """Causal GQA: the step count of the per-wave diagonal bookkeeping and the rescale count
    against the model."""
    import torch
    import exact_attention_forward_tiled_amd as fa
    from oracle import skipsim
    qb, kb, vb = random_case(39, 1, 4, 2, 2000, 128, sigma=2.0)
    q64, k64 = synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb)
    for tau in (0.0, 8.0):
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        fa.fwd(to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb), causal=True,
               scale=128 ** -0.5, tau=tau, stats=stats)
        torch.cuda.synchronize()
        steps, resc = (int(x) for x in stats.cpu()[:2])
        m_steps = m_fires = 0
        for h in range(4):
            st, fi = skipsim.skip_counts(q64[0, h], k64[0, h // 2], 128 ** -0.5, tau, True)
            m_steps += st
            m_fires += fi
        log(f"  causal tau={tau}: steps={steps} rescales={resc}; model {m_steps} {m_fires}")
        assert m_steps == steps
        assert abs(resc - m_fires) <= max(3, 0.002 * steps), (resc, m_fires)

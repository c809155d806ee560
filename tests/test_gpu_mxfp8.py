"""MXFP8 path on the GPU (through the C ABI) against the float64 oracle.

* The quantisation kernels must reproduce the oracle's OCP MXFP8 codes and
  scales bit for bit (byte work: exact equality).
* The FP8 forward is compared with the oracle's step-by-step emulation of the
  same quantisation (oracle.mxfp8.fp8_attention) on the dequantised operands:
  relative RMS of O <= 5e-3, and |dLSE| within the shift the E4M3 MFMA's own
  accumulation error can cause (gpu_util.mxfp8_lse_tol states the measured
  basis).
* Exact invariants: V = 1 gives O = 1 (the normaliser is summed from the same
  rounded weights as PV); Q = 0 gives the mean of the dequantised V rows; GQA
  equals repeated kv heads bit for bit.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from oracle import mxfp8 as m8
from gpu_util import (MXFP8_O_RELRMS, MXFP8_O_ROW, cuda_ok, gate, log, mxfp8_lse_tol, rel_rms,
                      to_dev_f32)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _gpu_quantize(q, k, v):
    import exact_attention_forward_tiled_amd as fa
    qd, kd, vd = to_dev_f32(q), to_dev_f32(k), to_dev_f32(v)
    q8, qs = fa.quantize_mxfp8_rows(qd)
    k8, ks = fa.quantize_mxfp8_rows(kd)
    vt8, vts = fa.quantize_mxfp8_cols_t(vd)
    return q8, qs, k8, ks, vt8, vts


def _run(q, k, v, causal, scale, **kw):
    import torch
    import exact_attention_forward_tiled_amd as fa
    q8, qs, k8, ks, vt8, vts = _gpu_quantize(q, k, v)
    B, Hq, N, d = q.shape
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd_mxfp8(q8, qs, k8, ks, vt8, vts, causal=causal, scale=scale, out=(o, lse), **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _case(seed, B, Hq, Hkv, N, d=128, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, Hq, N, d)) * sigma).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, N, d)) * sigma).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    return q, k, v


def _reference(q, k, v, causal, scale):
    """(O, LSE, LSE tolerance) of the emulation on the same quantised inputs."""
    t = m8.quantize_inputs(q, k, v)
    o, lse = m8.fp8_attention(t["q"], t["k"], t["v"], causal, scale)
    return o, lse, mxfp8_lse_tol(t["q"], t["k"], scale)


def test_quantizers_bit_exact():
    import torch
    import exact_attention_forward_tiled_amd as fa
    rng = np.random.default_rng(31)
    x = rng.standard_normal((3, 96, 128)).astype(np.float32)
    x[0, 5, 32:64] = 0.0                                   # an all-zero block
    mags = m8.E4M3_MAGNITUDES
    ties = ((mags[:-1] + mags[1:]) / 2)[rng.permutation(126)[:31]]
    x[1, 7, :32] = np.concatenate([[300.0], ties]).astype(np.float32) * np.float32(2.0 ** -4)
    x[1, 8, :32] = np.float32(470.0)                        # block max in [448, 512): saturates
    x[1, 8, 3] = np.float32(-1e-9)                          # rounds to -0 -> stored +0
    x[2, 9, :32] *= 1e6                                     # large exponents
    x[2, 10, :32] *= 1e-30                                  # tiny exponents
    xd = to_dev_f32(x)
    log("quantize8 rows / cols_t")
    c, s = fa.quantize_mxfp8_rows(xd)
    torch.cuda.synchronize()
    rc, rs = m8.quantize(x.astype(np.float64), axis=-1)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert np.array_equal(s.cpu().numpy(), rs)
    ct, st = fa.quantize_mxfp8_cols_t(xd)
    torch.cuda.synchronize()
    rct, rst = m8.quantize(x.astype(np.float64), axis=-2)          # blocks along rows
    assert np.array_equal(ct.cpu().numpy(), np.swapaxes(rct, -1, -2))
    assert np.array_equal(st.cpu().numpy(), np.swapaxes(rst, -1, -2))


SMALL = [
    # B, Hq, Hkv, N, causal
    (1, 2, 2, 256, False),
    (1, 2, 2, 256, True),
    (1, 1, 1, 32, False),
    (1, 1, 1, 32, True),
    (1, 2, 2, 96, True),
    (2, 4, 2, 160, False),
    (1, 8, 2, 512, True),
    (1, 3, 3, 320, False),
    (1, 2, 1, 800, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dHq%dHkv%dN%d%s" % (
    c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
@pytest.mark.parametrize("tau", [8.0, 0.0])
def test_fp8_small(case, tau):
    B, Hq, Hkv, N, causal = case
    q, k, v = _case(sum(case[:4]) + 7, B, Hq, Hkv, N)
    scale = 1.0 / math.sqrt(128)
    log(f"mxfp8 case {case} tau {tau}")
    o, lse = _run(q, k, v, causal, scale, tau=tau)
    ro, rl, tol = _reference(q, k, v, causal, scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    gate(o, ro, MXFP8_O_RELRMS, MXFP8_O_ROW, f"{case} tau {tau} O")
    e = float(np.max(np.abs(lse - rl)))
    log(f"  max|dLSE|={e:.3e} (gate {tol:.3e})")
    assert e <= tol, e


def test_fp8_scale_sign_and_large_logits():
    q, k, v = _case(41, 1, 2, 2, 192, sigma=3.0)
    for scale in (-0.2, 0.3):
        log(f"mxfp8 scale {scale}")
        o, lse = _run(q, k, v, False, scale)
        ro, rl, tol = _reference(q, k, v, False, scale)
        gate(o, ro, MXFP8_O_RELRMS, MXFP8_O_ROW, f"scale {scale} O")
        e = float(np.max(np.abs(lse - rl)))
        log(f"  max|dLSE|={e:.3e} (gate {tol:.3e})")
        assert e <= tol


def test_fp8_extreme_logits():
    """Logits far past 500 (the range-guard regime of "Hardware-Aware FP4 FlashAttention-4",
    section "1. Direct-P para Inferencia Directa"): the integer reference max follows the true
    running max, and blocks whose exponent would fall below -127 are flushed by the stated
    rule in the kernel and the emulation alike."""
    q, k, v = _case(45, 1, 2, 2, 256, sigma=6.0)
    scale = 1.0
    t = m8.quantize_inputs(q, k, v)
    logits = np.einsum("bhid,bhjd->bhij", t["q"], t["k"]) * scale
    assert np.abs(logits).max() > 500
    for causal in (False, True):
        log(f"mxfp8 extreme logits causal={causal}")
        o, lse = _run(q, k, v, causal, scale)
        ro, rl, tol = _reference(q, k, v, causal, scale)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        gate(o, ro, MXFP8_O_RELRMS, MXFP8_O_ROW, f"extreme causal={causal} O")
        e = float(np.max(np.abs(lse - rl)))
        log(f"  max|dLSE|={e:.3e} (gate {tol:.3e})")
        assert e <= tol


def test_fp8_constant_v_gives_one():
    q, k, _ = _case(42, 1, 4, 2, 256, sigma=2.0)
    v = np.ones((1, 2, 256, 128), np.float32)
    for causal in (False, True):
        log(f"mxfp8 constant V causal={causal}")
        o, _ = _run(q, k, v, causal, 0.09)
        assert np.max(np.abs(o - 1.0)) < 1e-6


def test_fp8_zero_query_is_mean_of_v():
    _, k, v = _case(43, 1, 2, 2, 128)
    q = np.zeros((1, 2, 128, 128), np.float32)
    t = m8.quantize_inputs(q, k, v)
    log("mxfp8 zero query")
    o, lse = _run(q, k, v, False, 0.1)
    ref = np.broadcast_to(t["v"].mean(axis=2, keepdims=True), o.shape)
    assert rel_rms(o, ref) < 1e-5
    assert np.max(np.abs(lse - math.log(128))) < 1e-5


def test_fp8_gqa_equals_repeated_heads():
    q, k, v = _case(44, 1, 8, 2, 192)
    for causal in (False, True):
        log(f"mxfp8 gqa causal={causal}")
        o1, l1 = _run(q, k, v, causal, 0.09)
        o2, l2 = _run(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), causal, 0.09)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("idx", [6, 7])
def test_fp8_workload_sampled_rows(idx):
    """The MXFP8 bench workloads at full size (B1 H24 N16384 non-causal; causal GQA B1 Hq32
    Hkv8 N8192), in the bench's launch configuration: sampled rows of several heads against
    the emulation, and the cosine against exact attention on the unquantised inputs (the
    explainer page quotes about 0.990 for its FP8 path; context only)."""
    w = synth.workload(idx)
    q, k, v = w.make()
    log(f"mxfp8 workload {w.name}")
    o, lse = _run(q, k, v, w.causal, w.scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    rng = np.random.default_rng(idx)
    group = w.Hq // w.Hkv
    heads = [0, w.Hq - 1, int(rng.integers(w.Hq))]
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, 255, 256, w.N - 1],
                                     rng.integers(0, w.N, 27)]))
    got, ref, exact = [], [], []
    for h in heads:
        g = h // group
        t = m8.quantize_inputs(q[:, h:h + 1, rows], k[:, g:g + 1], v[:, g:g + 1])
        tol = mxfp8_lse_tol(t["q"], t["k"], w.scale)
        ro, rl, _ = m8.fp8p_rows(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], rows, w.causal,
                                 w.scale)
        got.append(o[0, h, rows])
        ref.append(ro)
        eo, _ = oracle.attention_rows(q[:, h:h + 1].astype(np.float64),
                                      k[:, g:g + 1].astype(np.float64),
                                      v[:, g:g + 1].astype(np.float64), w.causal, w.scale,
                                      0, 0, rows)
        exact.append(eo)
        e = float(np.max(np.abs(lse[0, h, rows] - rl)))
        log(f"  head {h}: max|dLSE|={e:.3e} (gate {tol:.3e})")
        assert e <= tol
    got, ref, exact = (np.concatenate(x) for x in (got, ref, exact))
    gate(got, ref, MXFP8_O_RELRMS, MXFP8_O_ROW, "sampled rows vs emulation O")
    cos = np.mean(np.sum(got * exact, -1) / np.linalg.norm(got, axis=-1) /
                  np.linalg.norm(exact, axis=-1))
    log(f"  mean row cosine vs unquantised exact {cos:.5f}")



def test_fp8_long_sequence_sampled_rows():
    """One head of N = 2^18 keys (non-causal), far past the workloads' lengths: sampled rows,
    both ends and scale-block edges included, against the emulation."""
    N = 1 << 18
    scale = 1.0 / math.sqrt(128)
    q, k, v = _case(63, 1, 1, 1, N)
    log("mxfp8 N = 2^18")
    o, lse = _run(q, k, v, False, scale)
    rng = np.random.default_rng(63)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 255, 256, N - 257, N - 33, N - 32, N - 1],
                                     rng.integers(0, N, 10)]))
    t = m8.quantize_inputs(q[:, :, rows], k, v)
    tol = mxfp8_lse_tol(t["q"], t["k"], scale)
    ro, rl, _ = m8.fp8p_rows(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], rows, False, scale)
    e = float(np.max(np.abs(lse[0, 0, rows] - rl)))
    log(f"  max|dLSE|={e:.3e} (gate {tol:.3e})")
    assert e <= tol
    gate(o[0, 0, rows], ro, MXFP8_O_RELRMS, MXFP8_O_ROW, "N = 2^18 rows vs emulation O")

MASKED = [
    # B, Hq, Hkv, N, causal, window, docs
    (1, 2, 2, 512, True, 100, None),
    (1, 2, 2, 320, False, 64, None),
    (1, 4, 2, 256, True, 0, [0, 100, 101, 256]),
    (1, 2, 2, 384, False, 0, [0, 64, 200, 384]),
    (1, 2, 2, 512, True, 130, [0, 300, 512]),
    (1, 2, 2, 128, True, 1, None),       # a window of 1: every row sees only itself
    (1, 2, 2, 256, False, 256, None),    # a window N wide hides nothing
]


def _masked_check(q, k, v, causal, scale, window, docs, rows=None):
    import torch
    dd = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda")
    o, lse = _run(q, k, v, causal, scale, window=window, docs=dd)
    t = m8.quantize_inputs(q, k, v)
    tol = mxfp8_lse_tol(t["q"], t["k"], scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    if rows is None:
        ro, rl = m8.fp8_attention(t["q"], t["k"], t["v"], causal, scale, window=window,
                                  docs=docs)
    else:   # sampled rows of every head
        B, Hq = q.shape[:2]
        group = Hq // k.shape[1]
        ro = np.empty((B, Hq, len(rows), q.shape[3]))
        rl = np.empty((B, Hq, len(rows)))
        for b in range(B):
            for h in range(Hq):
                ro[b, h], rl[b, h], _ = m8.fp8p_rows(t["q"][b, h, rows], t["k"][b, h // group],
                                                     t["v"][b, h // group], rows, causal, scale,
                                                     window=window, docs=docs)
        o, lse = o[:, :, rows], lse[:, :, rows]
    gate(o, ro, MXFP8_O_RELRMS, MXFP8_O_ROW, "masked O")
    e = float(np.max(np.abs(lse - rl)))
    log(f"  max|dLSE|={e:.3e} (gate {tol:.3e})")
    assert e <= tol, e


@pytest.mark.parametrize("case", MASKED, ids=lambda c: "Hq%dHkv%dN%d%sW%d%s" % (
    c[1], c[2], c[3], "c" if c[4] else "n", c[5], "docs" if c[6] else ""))
def test_fp8_masked(case):
    """Sliding window and packed documents on the MXFP8 forward (tiles outside a block's band
    skipped) against the emulation under the same masks."""
    B, Hq, Hkv, N, causal, window, docs = case
    q, k, v = _case(N + window + 3 * Hq, B, Hq, Hkv, N)
    log(f"mxfp8 masked case {case}")
    _masked_check(q, k, v, causal, 1.0 / math.sqrt(128), window, docs)


def test_fp8_masked_long_sampled_rows():
    """Causal GQA N 4096 with a 1024 window over two documents: sampled rows (both document
    edges, the window's reach, the last rows) of every head."""
    q, k, v = _case(61, 1, 4, 2, 4096)
    rows = np.array([0, 1, 31, 1023, 1024, 1500, 2047, 2048, 2049, 3071, 3072, 4094, 4095])
    log("mxfp8 masked N4096 W1024 docs")
    _masked_check(q, k, v, True, 1.0 / math.sqrt(128), 1024, [0, 2048, 4096], rows=rows)


def _visible_tile_steps(N, causal, window=0, docs=None):
    """Steps the counters report: per 32-row wave, the 64-key tiles holding a key visible to
    one of its rows, minus the wave's first (from the oracle's visibility definition)."""
    vis = oracle.exact.visible(np.arange(N), N, causal, window, docs)
    steps = 0
    for r0 in range(0, N, 32):
        w = vis[r0:r0 + 32]
        tiles = [bool(w[:, t0:t0 + 64].any()) for t0 in range(0, N, 64)]
        steps += max(0, sum(tiles) - 1)
    return steps


@pytest.mark.parametrize("causal,window,docs", [(False, 0, None), (True, 0, None),
                                                (True, 300, None), (False, 200, [0, 700, 1024])])
def test_fp8_skip_ratio_stats(causal, window, docs):
    """The MXFP8 kernel's counters (steps in closed form, rescales counted where they are
    applied): the step count exactly against the visible tiles of every wave, and, without
    a band, the rescale count against the skip-ratio model with the integer reference rule
    on the dequantised operands (within a few decisions: fp32 scores in the kernel)."""
    import torch
    from oracle import skipsim
    N, H = 1024, 2
    q, k, v = _case(27, 1, H, H, N, sigma=3.0)
    t = m8.quantize_inputs(q, k, v)
    dd = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda")
    for tau in (0.0, 8.0):
        stats = torch.zeros(4, dtype=torch.int64, device="cuda")
        log(f"mxfp8 stats causal={causal} window={window} docs={docs} tau={tau}")
        _run(q, k, v, causal, 1.0 / math.sqrt(128), tau=tau, stats=stats, window=window,
             docs=dd)
        steps, resc = (int(x) for x in stats.cpu()[:2])
        want_steps = H * _visible_tile_steps(N, causal, window, docs)
        log(f"  steps {steps} (visible tiles {want_steps}) rescales {resc}")
        assert steps == want_steps
        if window == 0 and docs is None:
            m_fires = sum(skipsim.skip_counts(t["q"][0, h], t["k"][0, h], 1.0 / math.sqrt(128),
                                              tau, causal, integer_ref=True)[1] for h in range(H))
            log(f"  model rescales {m_fires}")
            assert abs(resc - m_fires) <= max(3, 0.002 * steps)

"""MXFP4 path on the GPU (through the C ABI) against the float64 oracle.

* The quantisation kernels must reproduce the oracle's OCP MX codes and scales
  bit for bit (byte work: exact equality).
* The Direct-P forward is compared with the oracle's step-by-step emulation of
  the same quantisation (oracle.mx.directp_attention) on the dequantised
  operands: relative RMS of O <= 0.1 (the stated tolerance for this path).
  Because the emulation follows the same integer-reference rule, the two agree
  far closer than that unless an exponential lands on an E2M1 midpoint; the
  measured error is printed.
* Exact invariants: V = 1 gives O = 1 (the normaliser is summed from the same
  codes and scales as PV); Q = 0 gives the mean of the dequantised V rows.
* Sliding window and packed documents against the emulation under the same
  masks, and the step counter against the visible tiles of every wave.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from oracle import mx
from gpu_util import MXFP4_O_RELRMS, MXFP4_O_ROW, cuda_ok, gate, log, rel_rms, to_dev_f32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _pack(codes):
    """One 4-bit code per element along the last axis -> bytes (element 2i in the low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _gpu_quantize(q, k, v):
    import exact_attention_forward_tiled_amd as fa
    qd, kd, vd = to_dev_f32(q), to_dev_f32(k), to_dev_f32(v)
    q4, qs = fa.quantize_mxfp4_rows(qd)
    k4, ks = fa.quantize_mxfp4_rows(kd)
    vt4, vts = fa.quantize_mxfp4_cols_t(vd)
    return q4, qs, k4, ks, vt4, vts


def _run(q, k, v, causal, scale, **kw):
    import torch
    import exact_attention_forward_tiled_amd as fa
    q4, qs, k4, ks, vt4, vts = _gpu_quantize(q, k, v)
    B, Hq, N, d = q.shape
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd_mxfp4(q4, qs, k4, ks, vt4, vts, causal=causal, scale=scale, out=(o, lse), **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _case(seed, B, Hq, Hkv, N, d=128, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, Hq, N, d)) * sigma).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, N, d)) * sigma).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    return q, k, v


def test_quantizers_bit_exact():
    import torch
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 96, 128)).astype(np.float32)
    x[0, 5, 32:64] = 0.0                                  # an all-zero block
    x[1, 7, :32] = np.float32(2.0 ** -3) * np.array(     # exact ties in block units
        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0] * 4, np.float32)
    x[2, 9, :32] *= 1e6                                   # large exponents
    x[2, 10, :32] *= 1e-30                                # tiny exponents
    import exact_attention_forward_tiled_amd as fa
    xd = to_dev_f32(x)
    c, s = fa.quantize_mxfp4_rows(xd)
    torch.cuda.synchronize()
    rc, rs = mx.quantize(x.astype(np.float64), axis=-1)
    assert np.array_equal(c.cpu().numpy(), _pack(rc))
    assert np.array_equal(s.cpu().numpy(), rs)
    ct, st = fa.quantize_mxfp4_cols_t(xd)
    torch.cuda.synchronize()
    rct, rst = mx.quantize(x.astype(np.float64), axis=-2)        # blocks along rows
    assert np.array_equal(ct.cpu().numpy(), _pack(np.swapaxes(rct, -1, -2)))
    assert np.array_equal(st.cpu().numpy(), np.swapaxes(rst, -1, -2))


def _reference(q, k, v, causal, scale):
    t = mx.quantize_inputs(q, k, v)
    return mx.directp_attention(t["q"], t["k"], t["v"], causal, scale)


SMALL = [
    # B, Hq, Hkv, N, causal
    (1, 2, 2, 256, False),
    (1, 2, 2, 256, True),
    (1, 1, 1, 32, False),
    (1, 2, 2, 96, True),
    (2, 4, 2, 160, False),
    (1, 8, 2, 512, True),
    (1, 3, 3, 320, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dHq%dHkv%dN%d%s" % (
    c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
@pytest.mark.parametrize("tau", [8.0, 0.0])
def test_directp_small(case, tau):
    B, Hq, Hkv, N, causal = case
    q, k, v = _case(sum(case[:4]) + 3, B, Hq, Hkv, N)
    scale = 1.0 / math.sqrt(128)
    log(f"case {case} tau {tau}")
    o, lse = _run(q, k, v, causal, scale, tau=tau)
    ro, rl = _reference(q, k, v, causal, scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    gate(o, ro, MXFP4_O_RELRMS, MXFP4_O_ROW, f"{case} tau {tau} O")
    e = float(np.max(np.abs(lse - rl)))
    log(f"  max|dLSE|={e:.3e}")
    assert e <= 0.05, e


def test_directp_scale_sign_and_large_logits():
    q, k, v = _case(21, 1, 2, 2, 192, sigma=3.0)
    for scale in (-0.2, 0.3):
        log(f"scale {scale}")
        o, lse = _run(q, k, v, False, scale)
        ro, rl = _reference(q, k, v, False, scale)
        gate(o, ro, MXFP4_O_RELRMS, MXFP4_O_ROW, f"scale {scale} O")
        log(f"  max|dLSE|={float(np.max(np.abs(lse - rl))):.3e}")


def test_directp_extreme_logits():
    """Logits far past 500, the regime of the range guard in "Hardware-Aware FP4
    FlashAttention-4", section "1. Direct-P para Inferencia Directa" (Protección de Rango).
    Here the integer reference max follows the true running max, so the leading blocks of a
    row never underflow.  Blocks more than about 125 binades below it have E < -127 and are
    flushed to zero by the stated rule, in the kernel and in the emulation alike.  The inputs
    are checked to be extreme (|logit| > 500) and to exercise the flush."""
    q, k, v = _case(25, 1, 2, 2, 256, sigma=6.0)
    scale = 1.0
    t = mx.quantize_inputs(q, k, v)
    logits = np.einsum("bhid,bhjd->bhij", t["q"], t["k"]) * scale
    assert np.abs(logits).max() > 500
    tl = logits * mx.LOG2E
    m = np.ceil(tl.max(-1, keepdims=True))
    e_blk = np.floor(tl.reshape(*tl.shape[:-1], -1, mx.BLOCK).max(-1) - m) - 2
    log(f"max |logit| {np.abs(logits).max():.0f}; flushed (row, block) pairs "
        f"{np.mean(e_blk < -127):.2f}")
    assert np.mean(e_blk < -127) > 0.1
    # fp32 summation error of the scores themselves (any order; u = 2^-24), in log units
    absum = np.einsum("bhid,bhjd->bhij", np.abs(t["q"]), np.abs(t["k"]))
    ds = scale * 128 * 2.0 ** -24 * absum.max()
    for causal in (False, True):
        o, lse = _run(q, k, v, causal, scale)
        ro, rl = _reference(q, k, v, causal, scale)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        gate(o, ro, MXFP4_O_RELRMS, MXFP4_O_ROW, f"extreme causal={causal} O")
        e = float(np.max(np.abs(lse - rl)))
        log(f"  causal={causal}: max|dLSE|={e:.3e} (bound {0.05 + ds:.3e})")
        assert e <= 0.05 + ds


def test_directp_constant_v_gives_one():
    q, k, _ = _case(22, 1, 4, 2, 256, sigma=2.0)
    v = np.ones((1, 2, 256, 128), np.float32)
    for causal in (False, True):
        o, _ = _run(q, k, v, causal, 0.09)
        assert np.max(np.abs(o - 1.0)) < 1e-6


def test_directp_zero_query_is_mean_of_v():
    _, k, v = _case(23, 1, 2, 2, 128)
    q = np.zeros((1, 2, 128, 128), np.float32)
    t = mx.quantize_inputs(q, k, v)
    o, lse = _run(q, k, v, False, 0.1)
    ref = np.broadcast_to(t["v"].mean(axis=2, keepdims=True), o.shape)
    assert rel_rms(o, ref) < 1e-5
    assert np.max(np.abs(lse - math.log(128))) < 1e-5


def test_directp_gqa_equals_repeated_heads():
    q, k, v = _case(24, 1, 8, 2, 192)
    for causal in (False, True):
        o1, l1 = _run(q, k, v, causal, 0.09)
        o2, l2 = _run(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), causal, 0.09)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_directp_workload_sampled_rows():
    """The full-size MXFP4 workload: sampled rows of several heads against the emulation, and
    the cosine against exact attention on the unquantised inputs (context only)."""
    w = synth.workload(5)
    q, k, v = w.make()
    log(f"workload {w.name}")
    o, lse = _run(q, k, v, w.causal, w.scale)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    rng = np.random.default_rng(5)
    heads = [0, w.Hq - 1, int(rng.integers(w.Hq))]
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, w.N - 1], rng.integers(0, w.N, 29)]))
    got, ref, exact = [], [], []
    for h in heads:
        t = mx.quantize_inputs(q[:, h:h + 1, rows], k[:, h:h + 1], v[:, h:h + 1])
        ro, rl, _ = mx.directp_rows(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], rows, False, w.scale)
        got.append(o[0, h, rows])
        ref.append(ro)
        eo, _ = oracle.attention(q[:, h:h + 1, rows].astype(np.float64),
                                 k[:, h:h + 1].astype(np.float64),
                                 v[:, h:h + 1].astype(np.float64), False, w.scale)
        exact.append(eo[0, 0])
        assert np.max(np.abs(lse[0, h, rows] - rl)) < 0.05
    got, ref, exact = (np.concatenate(x) for x in (got, ref, exact))
    gate(got, ref, MXFP4_O_RELRMS, MXFP4_O_ROW, "sampled rows vs emulation O")
    cos = np.mean(np.sum(got * exact, -1) / np.linalg.norm(got, axis=-1) /
                  np.linalg.norm(exact, axis=-1))
    log(f"  mean row cosine vs unquantised exact {cos:.4f}")



def test_directp_long_sequence_sampled_rows():
    """One head of N = 2^18 keys (non-causal), far past the workloads' lengths: sampled rows,
    both ends and block edges included, against the Direct-P emulation."""
    N = 1 << 18
    scale = 1.0 / math.sqrt(128)
    q, k, v = _case(64, 1, 1, 1, N)
    log("mxfp4 N = 2^18")
    o, lse = _run(q, k, v, False, scale)
    rng = np.random.default_rng(64)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 255, 256, N - 257, N - 33, N - 32, N - 1],
                                     rng.integers(0, N, 10)]))
    t = mx.quantize_inputs(q[:, :, rows], k, v)
    ro, rl, _ = mx.directp_rows(t["q"][0, 0], t["k"][0, 0], t["v"][0, 0], rows, False, scale)
    assert np.max(np.abs(lse[0, 0, rows] - rl)) < 0.05
    gate(o[0, 0, rows], ro, MXFP4_O_RELRMS, MXFP4_O_ROW, "N = 2^18 rows vs emulation O")

def test_directp_skip_ratio_stats():
    """The MXFP4 kernel's counters (steps in closed form, rescales counted where they are
    applied) against the skip-ratio model with the integer reference rule, on the
    dequantised operands: the step count exactly, the rescale count within a few
    decisions (scores are fp32 sums in the kernel)."""
    import torch
    from oracle import skipsim
    for causal in (False, True):
        q, k, v = _case(26, 1, 2, 2, 2048, sigma=3.0)
        t = mx.quantize_inputs(q, k, v)
        for tau in (0.0, 8.0):
            stats = torch.zeros(4, dtype=torch.int64, device="cuda")
            log(f"mxfp4 stats causal={causal} tau={tau}")
            _run(q, k, v, causal, 1.0 / math.sqrt(128), tau=tau, stats=stats)
            steps, resc = (int(x) for x in stats.cpu()[:2])
            m_steps = m_fires = 0
            for h in range(2):
                st, fi = skipsim.skip_counts(t["q"][0, h], t["k"][0, h], 1.0 / math.sqrt(128),
                                             tau, causal, integer_ref=True)
                m_steps += st
                m_fires += fi
            log(f"  steps {steps} rescales {resc}; model {m_steps} {m_fires}")
            assert steps == m_steps
            assert abs(resc - m_fires) <= max(3, 0.002 * steps)


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
    t = mx.quantize_inputs(q, k, v)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    if rows is None:
        ro, rl = mx.directp_attention(t["q"], t["k"], t["v"], causal, scale, window=window,
                                      docs=docs)
    else:   # sampled rows of every head
        B, Hq = q.shape[:2]
        group = Hq // k.shape[1]
        ro = np.empty((B, Hq, len(rows), q.shape[3]))
        rl = np.empty((B, Hq, len(rows)))
        for b in range(B):
            for h in range(Hq):
                ro[b, h], rl[b, h], _ = mx.directp_rows(t["q"][b, h, rows], t["k"][b, h // group],
                                                        t["v"][b, h // group], rows, causal, scale,
                                                        window=window, docs=docs)
        o, lse = o[:, :, rows], lse[:, :, rows]
    gate(o, ro, MXFP4_O_RELRMS, MXFP4_O_ROW, "masked O")
    e = float(np.max(np.abs(lse - rl)))
    log(f"  max|dLSE|={e:.3e}")
    assert e <= 0.05, e


@pytest.mark.parametrize("case", MASKED, ids=lambda c: "Hq%dHkv%dN%d%sW%d%s" % (
    c[1], c[2], c[3], "c" if c[4] else "n", c[5], "docs" if c[6] else ""))
def test_directp_masked(case):
    """Sliding window and packed documents on the MXFP4 Direct-P forward (tiles outside a
    block's band skipped) against the emulation under the same masks."""
    B, Hq, Hkv, N, causal, window, docs = case
    q, k, v = _case(N + window + 5 * Hq, B, Hq, Hkv, N)
    log(f"mxfp4 masked case {case}")
    _masked_check(q, k, v, causal, 1.0 / math.sqrt(128), window, docs)


def test_directp_masked_long_sampled_rows():
    """Causal GQA N 4096 with a 1024 window over two documents: sampled rows (both document
    edges, the window's reach, the last rows) of every head."""
    q, k, v = _case(62, 1, 4, 2, 4096)
    rows = np.array([0, 1, 31, 1023, 1024, 1500, 2047, 2048, 2049, 3071, 3072, 4094, 4095])
    log("mxfp4 masked N4096 W1024 docs")
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


@pytest.mark.parametrize("causal,window,docs", [(True, 300, None), (False, 200, [0, 700, 1024])])
def test_directp_masked_step_counter(causal, window, docs):
    """With a band the kernel's step counter (closed form) equals the visible tiles of every
    wave."""
    import torch
    N, H = 1024, 2
    q, k, v = _case(28, 1, H, H, N, sigma=3.0)
    dd = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    log(f"mxfp4 stats causal={causal} window={window} docs={docs}")
    _run(q, k, v, causal, 1.0 / math.sqrt(128), stats=stats, window=window, docs=dd)
    steps = int(stats.cpu()[0])
    want = H * _visible_tile_steps(N, causal, window, docs)
    log(f"  steps {steps} (visible tiles {want})")
    assert steps == want


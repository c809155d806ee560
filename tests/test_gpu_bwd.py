"""bf16 backward on the GPU (through the C ABI) against the float64 oracle.

The backward takes the forward's O and LSE.  Two feeds are tested: the oracle's own O and
LSE (the backward kernels alone) and the GPU forward's (the forward + backward pair as a
caller runs it).  Gates: relRMS(dV) <= 5e-3, relRMS(dQ), relRMS(dK) <= 1e-2 (gpu_util
states the arithmetic); invariants from the definition (the dK rows of a kv head sum to 0,
the dV rows sum to the group's dO rows); bitwise determinism (no atomics).
"""

import math

import numpy as np
import pytest

import oracle
import synth
from oracle import backward as bw
from gpu_util import (BWD_DQK_RELRMS, BWD_DQK_ROW, BWD_DV_RELRMS, BWD_DV_ROW, cuda_ok, log,
                      rel_rms, row_rel_max, to_dev_bf16, to_dev_f32)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


def _case(seed, B, Hq, Hkv, N, d=128):
    """bf16 bits of q, k, v, dO and their exact float64 values."""
    qb, kb, vb = synth.configs.random_case(seed, B, Hq, Hkv, N, d)
    gb = synth.normal_bf16((B, Hq, N, d), 7919 + seed, 1.0)
    return (qb, kb, vb, gb), tuple(synth.bf16_bits_to_f64(x) for x in (qb, kb, vb, gb))


def _run(bits, causal, scale, o=None, lse=None, window=0, docs=None, alibi=None, softcap=0.0):
    """GPU backward; o, lse: float64 arrays to feed, else the GPU forward's outputs (with the
    same window, documents, ALiBi slopes and soft-capping)."""
    import torch
    import exact_attention_forward_tiled_amd as fa
    q, k, v, g = (to_dev_bf16(x) for x in bits)
    dd = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda")
    al = None if alibi is None else torch.tensor(alibi, dtype=torch.float32, device="cuda")
    if o is None:
        od, ld = fa.fwd(q, k, v, causal=causal, scale=scale, window=window, docs=dd, alibi=al,
                        softcap=softcap)
    else:
        od, ld = to_dev_f32(o), to_dev_f32(lse)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nan = float("nan")
    dq = torch.full((B, Hq, N, d), nan, dtype=torch.float32, device="cuda")
    dk = torch.full((B, Hkv, N, d), nan, dtype=torch.float32, device="cuda")
    dv = torch.full((B, Hkv, N, d), nan, dtype=torch.float32, device="cuda")
    fa.bwd(q, k, v, od, ld, g, causal=causal, scale=scale, out=(dq, dk, dv), window=window,
           docs=dd, alibi=al, softcap=softcap)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


# Where every query sees a single key (a window of 1, one-token documents everywhere) dQ and
# dK are exactly 0: P = 1 and dP - D cancels.  The kernels compute dP and D in fp32 from
# unit-scale bf16 operands, so the residue is a few fp32 ulps of dP (~1e-6), far below this.
ZERO_GRAD_ABS = 1e-4


def _check(got, ref, tag):
    """relRMS and the per-row gate on each gradient (rows: the last axis)."""
    rq, rk, rv = (rel_rms(a, b) for a, b in zip(got, ref))
    wq, wk, wv = (row_rel_max(a, b) for a, b in zip(got, ref))
    log(f"  {tag}: relRMS dQ={rq:.2e} dK={rk:.2e} dV={rv:.2e}; "
        f"rowmax dQ={wq:.2e} dK={wk:.2e} dV={wv:.2e}")
    for a in got:
        assert not np.isnan(a).any()
    assert rv <= BWD_DV_RELRMS, rv
    assert wv <= BWD_DV_ROW, wv
    for a, b, r, w in ((got[0], ref[0], rq, wq), (got[1], ref[1], rk, wk)):
        if np.sqrt(np.mean(np.square(b))) < 1e-9:    # an exactly zero gradient
            assert np.abs(a).max() <= ZERO_GRAD_ABS, np.abs(a).max()
        else:
            assert r <= BWD_DQK_RELRMS, (rq, rk)
            assert w <= BWD_DQK_ROW, (wq, wk)


SMALL = [
    # B, Hq, Hkv, N, causal[, d]
    (1, 2, 2, 128, False),
    (1, 2, 2, 256, False, 64),
    (1, 4, 2, 190, True, 64),
    (1, 1, 1, 1, True, 64),
    (1, 2, 2, 128, True),
    (1, 1, 1, 1, False),
    (1, 1, 1, 1, True),
    (1, 2, 2, 33, True),
    (2, 4, 2, 200, False),
    (1, 8, 2, 256, True),
    (1, 2, 2, 300, False),
    (1, 2, 1, 161, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dHq%dHkv%dN%d%sd%d" % (
    c[0], c[1], c[2], c[3], "c" if c[4] else "n", c[5] if len(c) > 5 else 128))
def test_bwd_small(case):
    B, Hq, Hkv, N, causal = case[:5]
    d = case[5] if len(case) > 5 else 128
    bits, (q, k, v, g) = _case(sum(case[:4]) + 11, B, Hq, Hkv, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal, scale)
    ref = bw.attention_backward(q, k, v, g, causal, scale, o=o, lse=lse)
    log(f"bwd case {case}")
    _check(_run(bits, causal, scale, o, lse), ref, "oracle O/LSE")
    _check(_run(bits, causal, scale), ref, "GPU forward O/LSE")


def test_bwd_negative_scale_and_large_logits():
    bits, (q, k, v, g) = _case(51, 1, 2, 2, 192)
    for scale in (-0.2, 0.3):
        o, lse = oracle.attention(q, k, v, False, scale)
        ref = bw.attention_backward(q, k, v, g, False, scale, o=o, lse=lse)
        log(f"bwd scale {scale}")
        _check(_run(bits, False, scale, o, lse), ref, f"scale {scale}")


def test_bwd_deterministic_and_invariants():
    bits, (q, k, v, g) = _case(52, 1, 4, 2, 256)
    scale = 1.0 / math.sqrt(128)
    log("bwd determinism")
    a = _run(bits, True, scale)
    b = _run(bits, True, scale)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    dq, dk, dv = a
    # dK rows of each kv head sum to ~0; dV rows sum to the group's dO rows
    assert np.abs(dk.sum(axis=2)).max() <= 1e-2 * np.abs(dk).sum(axis=2).max()
    want = g.reshape(1, 2, 2, 256, 128).sum(axis=(2, 3))
    assert np.allclose(dv.sum(axis=2), want, rtol=1e-2, atol=1e-2 * np.abs(want).max())


def test_bwd_headline_shape_two_heads():
    """Causal B4 H16 N2048 d128 (the forward's headline shape) in the launch configuration a
    caller uses: all heads run on the GPU, two heads are checked against the oracle in full."""
    w = synth.workload(2)
    qb, kb, vb = w.make()
    gb = synth.normal_bf16((w.B, w.Hq, w.N, w.d), 2917, 1.0)
    log(f"bwd on {w.name}")
    dq, dk, dv = _run((qb, kb, vb, gb), w.causal, w.scale)
    for b, h in ((0, 0), (w.B - 1, w.Hq - 1)):
        q, k, v, g = (synth.bf16_bits_to_f64(x[b, h]) for x in (qb, kb, vb, gb))
        ref = bw.backward_head(q, k, v, g, w.causal, w.scale)
        _check((dq[b, h], dk[b, h], dv[b, h]), ref, f"(b, h) = ({b}, {h})")


MASKED = [
    # B, Hq, Hkv, N, causal, window, docs, d
    (1, 4, 2, 300, True, 70, None, 128),
    (1, 2, 2, 257, False, 100, None, 128),
    (1, 2, 2, 150, True, 1, None, 128),
    (1, 2, 2, 150, False, 1, None, 64),
    (1, 2, 2, 100, True, 100, None, 128),           # a window N wide hides nothing
    (1, 2, 1, 400, True, 0, [0, 37, 170, 171, 400], 128),
    (2, 4, 2, 333, False, 0, [0, 100, 333], 64),
    (1, 2, 2, 512, True, 50, [0, 200, 512], 128),
    (1, 2, 2, 260, False, 33, [0, 129, 260], 64),
    (1, 2, 2, 64, False, 0, [0, 1, 2, 64], 128),    # one-token documents
]


@pytest.mark.parametrize("case", MASKED, ids=lambda c: "Hq%dHkv%dN%d%sW%d%sd%d" % (
    c[1], c[2], c[3], "c" if c[4] else "n", c[5], "docs" if c[6] else "", c[7]))
def test_bwd_masked(case):
    """Sliding window and packed documents: the band kernels (tiles outside the band are
    skipped) against the oracle under the same masks, fed the oracle's and the GPU
    forward's O / LSE."""
    B, Hq, Hkv, N, causal, window, docs, d = case
    bits, (q, k, v, g) = _case(N + 7 * Hq + window, B, Hq, Hkv, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal, scale, window=window, docs=docs)
    ref = bw.attention_backward(q, k, v, g, causal, scale, o=o, lse=lse, window=window,
                                docs=docs)
    log(f"bwd masked case {case}")
    _check(_run(bits, causal, scale, o, lse, window, docs), ref, "oracle O/LSE")
    _check(_run(bits, causal, scale, window=window, docs=docs), ref, "GPU forward O/LSE")


def test_bwd_masked_long_sequence():
    """Causal GQA N 2048 with a 256 window over three documents: most tiles lie outside
    the band; every head checked against the oracle."""
    B, Hq, Hkv, N = 1, 4, 2, 2048
    docs = [0, 700, 1500, 2048]
    bits, (q, k, v, g) = _case(77, B, Hq, Hkv, N)
    scale = 1.0 / math.sqrt(128)
    log("bwd masked N2048 W256 docs")
    got = _run(bits, True, scale, window=256, docs=docs)
    ref = bw.attention_backward(q, k, v, g, True, scale, window=256, docs=docs)
    _check(got, ref, "N2048 W256 docs")


MODIFIED = [
    # B, Hq, Hkv, N, causal, window, docs, d, softcap, ALiBi (slopes 2^(-8 h / Hq) * a)
    (1, 4, 2, 300, True, 0, None, 128, 2.0, 0.0),
    (1, 2, 2, 257, False, 0, None, 128, 0.0, 1.0),
    (1, 4, 2, 200, True, 0, None, 128, 1.5, 0.5),
    (1, 2, 2, 190, False, 64, None, 64, 3.0, 1.0),
    (1, 2, 1, 300, True, 0, [0, 100, 300], 128, 2.0, 0.0),
    (2, 2, 2, 130, False, 0, None, 64, 1.0, 0.0),
    (1, 2, 2, 96, True, 0, None, 64, 0.0, 2.0),
    # ALiBi alone at d = 128 (the two-wave dQ kernel with the cap path compiled out): causal
    # GQA, a window, documents
    (1, 4, 2, 300, True, 0, None, 128, 0.0, 1.0),
    (1, 2, 2, 333, False, 90, None, 128, 0.0, 0.7),
    (1, 4, 2, 290, True, 0, [0, 120, 121, 290], 128, 0.0, 1.5),
]


@pytest.mark.parametrize("case", MODIFIED, ids=lambda c: "Hq%dHkv%dN%d%sW%d%sd%dC%gA%g" % (
    c[1], c[2], c[3], "c" if c[4] else "n", c[5], "docs" if c[6] else "", c[7], c[8], c[9]))
def test_bwd_score_modifications(case):
    """Soft-capping and ALiBi (alone, together, with a window or documents): P rebuilt from
    the modified score and dS times the cap's derivative, against the oracle."""
    B, Hq, Hkv, N, causal, window, docs, d, softcap, a = case
    bits, (q, k, v, g) = _case(3 * N + Hq + d, B, Hq, Hkv, N, d)
    scale = 1.0 / math.sqrt(d)
    alibi = [a * 2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)] if a else None
    o, lse = oracle.attention(q, k, v, causal, scale, window=window, docs=docs, softcap=softcap,
                              alibi=alibi)
    ref = bw.attention_backward(q, k, v, g, causal, scale, o=o, lse=lse, window=window,
                                docs=docs, softcap=softcap, alibi=alibi)
    log(f"bwd modified case {case}")
    _check(_run(bits, causal, scale, o, lse, window, docs, alibi, softcap), ref, "oracle O/LSE")
    _check(_run(bits, causal, scale, window=window, docs=docs, alibi=alibi, softcap=softcap),
           ref, "GPU forward O/LSE")


DELTA_CASES = [
    # causal, window, docs, d, softcap: every form of the dQ kernel that writes D
    (True, 0, None, 128, 0.0),
    (False, 40, None, 128, 0.0),
    (True, 0, [0, 1, 120, 300], 128, 0.0),
    (False, 0, None, 64, 0.0),
    (False, 0, None, 128, 30.0),    # soft-capping at d = 128: the one-wave dQ kernel
]


@pytest.mark.parametrize("case", DELTA_CASES, ids=lambda c: "{}_w{}_{}_d{}_cap{}".format(
    "c" if c[0] else "n", c[1], "docs" if c[2] else "", c[3], c[4]))
def test_bwd_delta_workspace(case):
    """The caller's workspace, filled with NaN beforehand, ends holding D_i = dO_i . O_i for
    every row (written by the first kernel, whatever the mask), which the oracle pins as
    sum_j P_ij dP_ij."""
    import torch
    import exact_attention_forward_tiled_amd as fa
    causal, window, docs, d, softcap = case
    bits, (q, k, v, g) = _case(53 + d, 1, 4, 2, 300, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, causal, scale, window=window, docs=docs, softcap=softcap)
    qd, kd, vd, gd = (to_dev_bf16(x) for x in bits)
    dd = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda")
    delta = torch.full((1, 4, 300), float("nan"), dtype=torch.float32, device="cuda")
    log(f"bwd delta workspace {case}")
    fa.bwd(qd, kd, vd, to_dev_f32(o), to_dev_f32(lse), gd, causal=causal, scale=scale,
           delta=delta, window=window, docs=dd, softcap=softcap)
    torch.cuda.synchronize()
    got = delta.cpu().numpy()
    # O is fed in fp32 and dO is exact in bf16: D is an fp32 dot product of d terms
    want = bw.delta(o.astype(np.float32).astype(np.float64), g)
    bound = d * 2.0 ** -24 * np.sum(np.abs(o * g), axis=-1) + 1e-7
    assert np.all(np.abs(got - want) <= bound)


def _full_size_sampled(idx, seed):
    """Backward at a full workload size, all heads on the GPU (from the GPU forward's O and
    LSE, as a caller runs it); two (batch, kv head) groups checked on sampled query rows
    (dQ) and key rows (dK, dV, summed over the group's query heads) against the oracle."""
    w = synth.workload(idx)
    qb, kb, vb = w.make()
    gb = synth.normal_bf16((w.B, w.Hq, w.N, w.d), seed, 1.0)
    log(f"bwd on {w.name}")
    dq, dk, dv = _run((qb, kb, vb, gb), w.causal, w.scale)
    group = w.Hq // w.Hkv
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, w.N - 2, w.N - 1],
                                     rng.integers(0, w.N, 24)]))
    for b, hk in ((0, 0), (w.B - 1, w.Hkv - 1)):
        k, v = (synth.bf16_bits_to_f64(x[b, hk]) for x in (kb, vb))
        got_q, ref_q = [], []
        ref_k = np.zeros((len(rows), w.d))
        ref_v = np.zeros((len(rows), w.d))
        for h in range(hk * group, (hk + 1) * group):
            q, g = (synth.bf16_bits_to_f64(x[b, h]) for x in (qb, gb))
            o, lse = oracle.attention_head(q[None, None], k[None, None], v[None, None],
                                           w.causal, w.scale, 0, 0)
            rq, rk, rv = bw.backward_rows(q, k, v, g, w.causal, w.scale, o, lse, rows, rows)
            got_q.append(dq[b, h, rows])
            ref_q.append(rq)
            ref_k += rk
            ref_v += rv
        _check((np.concatenate(got_q), dk[b, hk, rows], dv[b, hk, rows]),
               (np.concatenate(ref_q), ref_k, ref_v), f"(b, kv head) = ({b}, {hk})")


def test_bwd_full_size_noncausal_long():
    """Non-causal B2 H16 N16384 d128 (the unrolled non-causal dK/dV path)."""
    _full_size_sampled(4, 4917)


def test_bwd_full_size_causal_gqa():
    """Causal GQA B1 Hq32 Hkv8 N8192 d128 (dK, dV summed over four query heads)."""
    _full_size_sampled(3, 3917)

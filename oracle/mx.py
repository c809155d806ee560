"""MXFP4 quantisation and a step-by-step Direct-P emulation, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Format.  "Hardware-Aware FP4 FlashAttention-4", section "Planteamiento del
Problema" (Rango Numérico) names the 4-bit E2M1 payload of NVFP4/MXFP4, and
section "1. Direct-P para Inferencia Directa" (Selección de Formato) gives
MXFP4 power-of-two block scales to P and V.  The element and scale encodings
themselves are those of the OCP Microscaling (MX) v1.0 specification, which
the pages do not print:

* E2M1 element: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; the
  eight non-negative magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (code 0..7),
  the sign is bit 3 of the 4-bit code.
* E8M0 block scale: a byte holding E + 127, the block value being 2^E.
* Block of 32 elements; shared exponent E = floor(log2(amax)) - 2, where 2 is
  the exponent of the largest E2M1 normal; elements are x / 2^E rounded to
  the nearest magnitude, ties to the even code, saturating at 6.

Readings of points the pages leave open (each listed in the design notes):
an all-zero block gets E = 0 (scale byte 127) and zero codes; a value that
rounds to magnitude 0 is stored as +0 (code 0); E is clamped to [-127, 127].

Direct-P (same page, section "1. Direct-P para Inferencia Directa"): the
normalised log-scores are mapped straight onto the eight E2M1 magnitudes
(Mapeo Directo), and the softmax denominator is accumulated from exactly the
rounded codes and block scales that the PV product consumes (Normalización
Consistente).  Emulated here as:

    t_ij  = scale * q~_i . k~_j * log2(e)           (-inf where masked: causal, and
                                                     the sliding window and packed
                                                     documents of the FlexAttention
                                                     patterns, oracle.exact.visible)
    m_i   = ceil(max_j t_ij)                        integer reference max
    per row i and 32-key block b:
      M_ib = max of t_ij over the block
      E_ib = floor(M_ib - m_i) - 2                  P block scale exponent
      code = RNE_E2M1(2^(t_ij - m_i - E_ib))        no separate exponential
      p~_ij = |code| * 2^E_ib                       (block flushed to 0 when
                                                     fully masked or E_ib < -127)
    l_i   = sum_j p~_ij
    O_i   = sum_j p~_ij v~_j / l_i
    LSE_i = ln(2) * m_i + ln(l_i)

Because m_i is an integer, the codes do not depend on which integer
reference max is held when a block is classified, so one emulation serves
any tile order and any rescale threshold (pinned by a test).
"""

import math

import numpy as np

from .exact import visible

BLOCK = 32
E2M1_EMAX = 2
# code -> magnitude, OCP MX v1.0 FP4 (E2M1)
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
LOG2E = 1.0 / math.log(2.0)


def e2m1_round(y):
    """Nearest E2M1 magnitude code (0..7) for y >= 0; ties go to the even code; saturates at 6."""
    y = np.asarray(y, dtype=np.float64)
    dist = np.abs(y[..., None] - E2M1_MAGNITUDES)
    nearest = dist == dist.min(axis=-1, keepdims=True)
    even = nearest & (np.arange(8) % 2 == 0)
    pick_even = even.any(axis=-1)
    code = np.where(pick_even, np.argmax(even, axis=-1), np.argmax(nearest, axis=-1))
    return code.astype(np.uint8)


def shared_exponent(amax):
    """E = floor(log2(amax)) - 2, exactly (frexp); 0 for an all-zero block; clamped to [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    mant, ex = np.frexp(amax)            # amax = mant * 2^ex, mant in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - E2M1_EMAX
    e = np.where(amax > 0, e, 0)
    return np.clip(e, -127, 127)


def quantize(x, axis):
    """Quantise along `axis` in blocks of 32.

    Returns (codes, scale_bytes): codes has x's shape (uint8, one 4-bit code
    per element, sign in bit 3); scale_bytes has the block axis shortened by
    32x (uint8, E + 127).
    """
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    if n % BLOCK:
        raise ValueError("quantised axis must be a multiple of 32")
    blocks = xm.reshape(xm.shape[:-1] + (n // BLOCK, BLOCK))
    e = shared_exponent(np.abs(blocks).max(axis=-1))
    y = np.ldexp(np.abs(blocks), -e[..., None])
    mag = e2m1_round(y)
    neg = (blocks < 0) & (mag != 0)
    codes = (mag | (neg.astype(np.uint8) << 3)).reshape(xm.shape)
    scales = (e + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def dequantize(codes, scale_bytes, axis):
    """Exact float64 values of MXFP4 codes with their block scales."""
    codes = np.moveaxis(np.asarray(codes, dtype=np.uint8), axis, -1)
    sb = np.moveaxis(np.asarray(scale_bytes, dtype=np.int64), axis, -1)
    mag = E2M1_MAGNITUDES[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    n = codes.shape[-1]
    val = val.reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    val = np.ldexp(val, (sb - 127)[..., None])
    return np.moveaxis(val.reshape(codes.shape), -1, axis)


def directp_rows(qt_rows, kt, vt, row_ids, causal, scale, ref_max=None, window=0, docs=None):
    """Direct-P output for some query rows of one head, on dequantised operands.

    qt_rows [r, d], kt and vt [N, d] (float64, already dequantised).
    ref_max optionally overrides the integer reference max m_i (a test hook
    showing that the result does not depend on it).  window, docs: the exact
    forward's sliding window and packed documents (oracle.exact.visible); a
    hidden key's score is -inf before the block maxima, as with the causal
    mask.  Returns (O, LSE, p~).
    """
    n_keys = kt.shape[0]
    if n_keys % BLOCK:
        raise ValueError("the key count must be a multiple of 32")
    t = (scale * (qt_rows @ kt.T)) * LOG2E
    if causal or window or docs is not None:
        t = np.where(visible(np.asarray(row_ids), n_keys, causal, window, docs), t, -np.inf)
    row_max = t.max(axis=1)
    live_row = np.isfinite(row_max)
    m = np.where(live_row, np.ceil(np.where(live_row, row_max, 0.0)), 0.0)
    if ref_max is not None:
        m = np.asarray(ref_max, dtype=np.float64)
    p = np.zeros_like(t)
    for b0 in range(0, n_keys, BLOCK):
        tb = t[:, b0:b0 + BLOCK]
        mb = tb.max(axis=1)
        live = np.isfinite(mb)
        e = np.where(live, np.floor(np.where(live, mb, 0.0) - m) - 2.0, 0.0)
        live &= e >= -127
        with np.errstate(invalid="ignore"):
            x = tb - m[:, None] - e[:, None]
        y = np.where(np.isfinite(x), np.exp2(np.where(np.isfinite(x), x, 0.0)), 0.0)
        code = e2m1_round(y)
        pb = np.ldexp(E2M1_MAGNITUDES[code], e.astype(np.int64)[:, None])
        p[:, b0:b0 + BLOCK] = np.where(live[:, None], pb, 0.0)
    l = p.sum(axis=1)
    ok = l > 0
    l_safe = np.where(ok, l, 1.0)
    o = (p @ vt) / l_safe[:, None]
    o[~ok] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(ok, math.log(2.0) * m + np.log(l_safe), -np.inf)
    return o, lse, p


def directp_attention(qt, kt, vt, causal, scale, chunk=256, window=0, docs=None):
    """Direct-P forward over [B, H, N, d] dequantised operands: returns (O, LSE).  window,
    docs: as for directp_rows."""
    qt = np.asarray(qt, dtype=np.float64)
    B, Hq, N, d = qt.shape
    group = Hq // kt.shape[1]
    o = np.empty(qt.shape[:3] + (vt.shape[3],))
    lse = np.empty(qt.shape[:3])
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(N, r0 + chunk))
                o[b, h, rows], lse[b, h, rows], _ = directp_rows(
                    qt[b, h, rows], kt[b, g], vt[b, g], rows, causal, scale, window=window,
                    docs=docs)
    return o, lse


def quantize_inputs(q, k, v):
    """The workload's input quantisation: Q and K in 32-blocks along d, V in
    32-blocks along the key axis (one scale per 32 keys per column).

    Returns dict of codes/scales and the dequantised float64 operands.
    """
    qc, qs = quantize(q, axis=-1)
    kc, ks = quantize(k, axis=-1)
    vc, vs = quantize(v, axis=-2)
    return {
        "q_codes": qc, "q_scales": qs,
        "k_codes": kc, "k_scales": ks,
        "v_codes": vc, "v_scales": vs,
        "q": dequantize(qc, qs, axis=-1),
        "k": dequantize(kc, ks, axis=-1),
        "v": dequantize(vc, vs, axis=-2),
    }

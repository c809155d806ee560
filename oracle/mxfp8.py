"""MXFP8 (E4M3) quantisation and a step-by-step emulation of the FP8 forward, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages give.  "Hardware-Aware FP4 FlashAttention-4", section
"Resultados", compares its FP4 fast path with an FP8 path ("NV/FP8", mean
cosine about 0.990 against BF16); section "2. Causal Backward Cuantizado" puts
P and V in FP8 because MXFP4 P/V diverged in training; the aigc.bar page,
section "从V1到V4", credits FlashAttention-3 with FP8 support.  None of them
prints the format details or how P is scaled, so this module takes:

* E4M3 element (the OCP 8-bit floating-point format "E4M3FN"): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, subnormal when the exponent
  field is 0, no infinities, the all-ones exponent-and-mantissa pattern is
  NaN; largest magnitude 448, smallest subnormal 2^-9.
* MX block scaling (OCP Microscaling v1.0, as for MXFP4): one E8M0 scale
  byte per 32 elements, E = floor(log2(amax)) - 8 (8 = the exponent of E4M3's
  largest normal binade), elements x / 2^E rounded to the nearest E4M3
  magnitude, ties to the even code, saturating at 448.  An all-zero block
  gets E = 0; a value that rounds to 0 is stored as +0; E is clamped to
  [-127, 127].  Q and K are blocked along d, V along the key axis (the
  contraction axes of the two products), as on the MXFP4 path.
* P: the softmax weights relative to an integer reference max m_i are put on
  the same MX footing, one power-of-two scale per 32 keys:

      t_ij  = scale * q~_i . k~_j * log2(e)          (-inf where masked)
      m_i   = ceil(max_j t_ij)
      per row i and 32-key block b:
        M_ib  = max of t_ij over the block
        E_ib  = floor(M_ib - m_i) - 7                block max in [128, 256) * 2^E
        code  = RNE_E4M3(2^(t_ij - m_i - E_ib))
        p~_ij = val(code) * 2^E_ib                   (block flushed to 0 when
                                                      fully masked or E_ib < -127)
      l_i   = sum_j p~_ij                            from the rounded weights
      O_i   = sum_j p~_ij v~_j / l_i
      LSE_i = ln(2) * m_i + ln(l_i)

  The block maximum lands one binade below E4M3's top binade, so no weight
  ever saturates; weights more than 2^-16 below their block maximum round to
  0.  The denominator is taken from the very rounded weights the PV product
  consumes, as the same page's Direct-P section does for FP4 (Normalización
  Consistente).  Because m_i is an integer, the codes do not depend on which
  integer reference max is held when a block is rounded, so one emulation
  serves every tile order and rescale threshold (pinned by a test).
"""

import math

import numpy as np

from .exact import visible

BLOCK = 32
E4M3_EMAX = 8          # exponent of the largest normal binade (448 = 1.75 * 2^8)
E4M3_MAX = 448.0
P_EXP_OFFSET = 7       # P block exponent: floor(block max) - 7
LOG2E = 1.0 / math.log(2.0)


def e4m3_value(code):
    """Value of an E4M3 byte from its bit fields (NaN for the two NaN codes)."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64)))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# magnitudes of the non-negative codes 0..126 (127 is NaN), increasing with the code
E4M3_MAGNITUDES = e4m3_value(np.arange(127))


def e4m3_round(y):
    """Nearest E4M3 magnitude code (0..126) for y >= 0; ties to the even code; saturates at 448.

    Within a binade [2^e, 2^(e+1)) (e >= -6) the magnitudes are spaced 2^(e-3);
    below 2^-6 they are the subnormals, spaced 2^-9.  y / spacing rounded half
    to even is the even-code tie rule (the code's last bit is the mantissa's);
    a value rounding up to the next binade gets that binade's first code.
    """
    y = np.asarray(y, dtype=np.float64)
    pos = y > 0
    _, ex = np.frexp(np.where(pos, y, 1.0))       # y = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)    # binade exponent, subnormals share -6
    spacing_exp = e - 3
    k = np.rint(np.ldexp(np.where(pos, y, 0.0), -spacing_exp))   # multiple of the spacing
    q = np.ldexp(k, spacing_exp)
    q = np.minimum(q, E4M3_MAX)
    return magnitude_code(q)


def magnitude_code(q):
    """Code of an exactly representable non-negative E4M3 magnitude."""
    q = np.asarray(q, dtype=np.float64)
    idx = np.searchsorted(E4M3_MAGNITUDES, q)
    idx = np.minimum(idx, 126)
    if not np.all(E4M3_MAGNITUDES[idx] == q):
        raise ValueError("not an E4M3 magnitude")
    return idx.astype(np.uint8)


def shared_exponent(amax):
    """E = floor(log2(amax)) - 8, exactly (frexp); 0 for an all-zero block; clamped to [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    e = (ex.astype(np.int64) - 1) - E4M3_EMAX
    e = np.where(amax > 0, e, 0)
    return np.clip(e, -127, 127)


def quantize(x, axis):
    """Quantise along `axis` in blocks of 32: (codes uint8 like x, scale bytes E + 127)."""
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    if n % BLOCK:
        raise ValueError("quantised axis must be a multiple of 32")
    blocks = xm.reshape(xm.shape[:-1] + (n // BLOCK, BLOCK))
    e = shared_exponent(np.abs(blocks).max(axis=-1))
    mag = e4m3_round(np.ldexp(np.abs(blocks), -e[..., None]))
    neg = (blocks < 0) & (mag != 0)
    codes = (mag | (neg.astype(np.uint8) << 7)).reshape(xm.shape)
    scales = (e + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def dequantize(codes, scale_bytes, axis):
    """Exact float64 values of MXFP8 codes with their block scales."""
    codes = np.moveaxis(np.asarray(codes, dtype=np.uint8), axis, -1)
    sb = np.moveaxis(np.asarray(scale_bytes, dtype=np.int64), axis, -1)
    val = e4m3_value(codes)
    n = codes.shape[-1]
    val = val.reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    val = np.ldexp(val, (sb - 127)[..., None])
    return np.moveaxis(val.reshape(codes.shape), -1, axis)


def quantize_inputs(q, k, v):
    """Q and K in 32-blocks along d, V in 32-blocks along the key axis.

    Returns a dict of codes/scales and the dequantised float64 operands.
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


def fp8p_rows(qt_rows, kt, vt, row_ids, causal, scale, ref_max=None, window=0, docs=None):
    """FP8 forward for some query rows of one head, on dequantised operands.

    qt_rows [r, d], kt and vt [N, d] (float64).  ref_max optionally overrides
    the integer reference max (a test hook).  window, docs: the exact forward's
    sliding window and packed documents (oracle.exact.visible); a hidden key's
    score is -inf before the block maxima, as with the causal mask.  Returns
    (O, LSE, p~).
    """
    n_keys = kt.shape[0]
    if n_keys % BLOCK:
        raise ValueError("the key count must be a multiple of 32")
    t = (scale * (qt_rows @ kt.T)) * LOG2E
    if causal or window or docs is not None:
        t = np.where(visible(row_ids, n_keys, causal, window, docs), t, -np.inf)
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
        e = np.where(live, np.floor(np.where(live, mb, 0.0) - m) - P_EXP_OFFSET, 0.0)
        live &= e >= -127
        with np.errstate(invalid="ignore"):
            x = tb - m[:, None] - e[:, None]
        y = np.where(np.isfinite(x), np.exp2(np.where(np.isfinite(x), x, 0.0)), 0.0)
        code = e4m3_round(y)
        pb = np.ldexp(E4M3_MAGNITUDES[code], e.astype(np.int64)[:, None])
        p[:, b0:b0 + BLOCK] = np.where(live[:, None], pb, 0.0)
    l = p.sum(axis=1)
    ok = l > 0
    l_safe = np.where(ok, l, 1.0)
    o = (p @ vt) / l_safe[:, None]
    o[~ok] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(ok, math.log(2.0) * m + np.log(l_safe), -np.inf)
    return o, lse, p


def fp8_attention(qt, kt, vt, causal, scale, chunk=256, window=0, docs=None):
    """FP8 forward over [B, H, N, d] dequantised operands: returns (O, LSE)."""
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
                o[b, h, rows], lse[b, h, rows], _ = fp8p_rows(
                    qt[b, h, rows], kt[b, g], vt[b, g], rows, causal, scale, window=window,
                    docs=docs)
    return o, lse

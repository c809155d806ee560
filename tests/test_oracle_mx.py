"""Pins for the MXFP4 quantiser and the Direct-P emulation in oracle.mx."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mx


# ---- E2M1 / E8M0 encodings ---------------------------------------------------------

def test_e2m1_table_from_bit_fields():
    """The magnitude table equals the E2M1 bit-field definition: 2 exponent bits with bias 1,
    1 mantissa bit, subnormal when the exponent field is 0."""
    for code in range(8):
        e, m = code >> 1, code & 1
        val = (m / 2.0) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        assert mx.E2M1_MAGNITUDES[code] == val


def test_rne_ties_go_to_even_code():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for y, want in ties.items():
        assert mx.E2M1_MAGNITUDES[mx.e2m1_round(y)] == want, y


def test_round_to_nearest_dense_grid():
    """Away from ties the result is the nearest magnitude (brute-force scan of the 8 values)."""
    y = np.linspace(0.0, 9.0, 90001)
    got = mx.E2M1_MAGNITUDES[mx.e2m1_round(y)]
    for yy, g in zip(y[::97], got[::97]):
        best = min(mx.E2M1_MAGNITUDES, key=lambda m: (abs(m - yy), m))
        if not any(abs(abs(m - yy) - abs(best - yy)) < 1e-12 and m != best
                   for m in mx.E2M1_MAGNITUDES):
            assert g == best, yy
    assert np.all(got[y > 6.0] == 6.0)   # saturation


def _bruteforce_floor_log2(a):
    k = 0
    while 2.0 ** k > a:
        k -= 1
    while 2.0 ** (k + 1) <= a:
        k += 1
    return k


def test_shared_exponent():
    for a in [1.0, 2.0, 0.5, 3.999, 4.0, 1e-3, 6.1e4, 2.0 ** -100, 7.0]:
        assert mx.shared_exponent(a) == _bruteforce_floor_log2(a) - 2, a
    assert mx.shared_exponent(0.0) == 0
    assert mx.shared_exponent(2.0 ** 200) == 127 and mx.shared_exponent(2.0 ** -200) == -127
    # powers of two: the E8M0 byte of 2^k / 4 (torch's own e8m0 conversion is exact there)
    for k in range(-20, 21):
        want = torch.tensor([2.0 ** (k - 2)]).to(torch.float8_e8m0fnu).view(torch.uint8).item()
        assert int(mx.shared_exponent(2.0 ** k)) + 127 == want


def test_quantize_round_trip_exact_values():
    """Blocks made of representable values times 2^E, whose amax fixes that E, come back bit-exact."""
    rng = np.random.default_rng(1)
    for E in (-5, -1, 0, 3):
        vals = rng.choice(np.concatenate([mx.E2M1_MAGNITUDES, -mx.E2M1_MAGNITUDES[1:]]), 32)
        vals[7] = 4.0                      # amax in [4, 8) -> shared exponent is E
        x = np.ldexp(vals, E)
        codes, sc = mx.quantize(x[None, :], axis=-1)
        assert sc[0, 0] == E + 127
        assert np.array_equal(mx.dequantize(codes, sc, axis=-1)[0], x)


def test_quantize_error_bound_and_layout():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 64, 96)).astype(np.float32).astype(np.float64)
    for axis in (-1, -2):
        codes, sc = mx.quantize(x, axis=axis)
        xt = mx.dequantize(codes, sc, axis=axis)
        xm = np.moveaxis(x, axis, -1).reshape(-1, 32)
        tm = np.moveaxis(xt, axis, -1).reshape(-1, 32)
        e = np.moveaxis(sc.astype(np.int64) - 127, axis, -1).reshape(-1)
        scale = np.ldexp(1.0, e)[:, None]
        a = np.abs(xm) / scale
        # half the gap between neighbouring magnitudes; beyond 6 the error is the clip
        half_gap = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
        bound = np.where(a > 6, a - 6, half_gap) * scale
        assert np.all(np.abs(xm - tm) <= bound + 1e-15)
        assert np.all(np.sign(tm) * np.sign(xm) >= 0)
        # amax / 2^E lies in [4, 8)
        amax = np.abs(xm).max(axis=1)
        assert np.all((amax / scale[:, 0] >= 4) & (amax / scale[:, 0] < 8))


def test_zero_block_and_zero_sign():
    x = np.zeros((1, 32))
    x[0, 3] = -0.0
    codes, sc = mx.quantize(x, axis=-1)
    assert sc[0, 0] == 127 and np.all(codes == 0)
    y = np.full((1, 32), 1e-9)
    y[0, 0] = 4.0
    y[0, 1] = -1e-9
    codes, _ = mx.quantize(y, axis=-1)
    assert codes[0, 1] == 0                  # magnitude 0 is stored as +0


# ---- Direct-P emulation ----------------------------------------------------------

def _mx_case(seed, B, H, N, d):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3))
    return mx.quantize_inputs(q, k, v)


def test_directp_constant_v_gives_one():
    """Consistent normalisation: the denominator is the sum of the same codes PV uses, so V = 1 gives 1."""
    t = _mx_case(10, 1, 2, 96, 32)
    v = np.ones_like(t["v"])
    for causal in (False, True):
        o, _ = mx.directp_attention(t["q"], t["k"], v, causal, 0.5)
        assert np.allclose(o, 1.0, atol=1e-14)


def test_directp_zero_query():
    """Q = 0: t = 0, m = 0, E = -2, every key gets code 4.0 * 2^-2 = 1, so O is the mean of V~."""
    t = _mx_case(11, 1, 2, 64, 32)
    q = np.zeros_like(t["q"])
    o, lse = mx.directp_attention(q, t["k"], t["v"], False, 0.5)
    assert np.allclose(o, t["v"].mean(axis=2, keepdims=True), atol=1e-14)
    assert np.allclose(lse, math.log(64), atol=1e-14)
    _, _, p = mx.directp_rows(q[0, 0], t["k"][0, 0], t["v"][0, 0], np.arange(64), False, 0.5)
    assert np.all(p == 1.0)


def test_directp_single_visible_key():
    t = _mx_case(12, 1, 1, 32, 32)
    o, _ = mx.directp_attention(t["q"], t["k"], t["v"], True, 0.5)
    assert np.allclose(o[0, 0, 0], t["v"][0, 0, 0], atol=1e-15)


def test_directp_exact_when_weights_are_representable():
    """When every 2^(t - m - E) is an E2M1 magnitude, Direct-P equals the exact oracle."""
    N, d = 64, 1
    rng = np.random.default_rng(13)
    # logits in log2 units chosen so each block's values sit on the grid {4, 2, 1, 0.5} * 2^E
    t_vals = -rng.integers(0, 4, size=N).astype(np.float64)
    t_vals[0] = 0.0
    t_vals[32] = -1.0
    q = np.ones((1, 1, 1, d))
    k = (t_vals / mx.LOG2E).reshape(1, 1, N, d)     # scale * q.k * log2e = t
    v = rng.standard_normal((1, 1, N, 5))
    o, lse, p = mx.directp_rows(q[0, 0], k[0, 0], v[0, 0], np.array([0]), False, 1.0)
    oe, le = oracle.attention(q, k, v, False, 1.0)
    assert np.allclose(p[0], 2.0 ** t_vals, rtol=1e-12)
    assert np.allclose(o[0], oe[0, 0, 0], atol=1e-12)
    assert abs(lse[0] - le[0, 0, 0]) < 1e-12


def test_directp_independent_of_integer_reference():
    """Shifting the integer reference max by any integer leaves O and LSE unchanged."""
    t = _mx_case(14, 1, 1, 128, 64)
    qr, kh, vh = t["q"][0, 0, :16], t["k"][0, 0], t["v"][0, 0]
    rows = np.arange(16)
    o0, l0, p0 = mx.directp_rows(qr, kh, vh, rows, False, 0.3)
    m0 = np.ceil((0.3 * qr @ kh.T * mx.LOG2E).max(axis=1))
    for shift in (-3, 2, 7):
        o1, l1, p1 = mx.directp_rows(qr, kh, vh, rows, False, 0.3, ref_max=m0 + shift)
        assert np.allclose(p1 * 2.0 ** shift, p0, rtol=0, atol=0)
        assert np.allclose(o1, o0, atol=1e-15) and np.allclose(l1, l0, atol=1e-12)


def test_directp_codes_are_rne_of_exp():
    """Each weight is an E2M1 magnitude times a power of two, within the rounding bound of 2^(t-m)."""
    t = _mx_case(15, 1, 1, 64, 32)
    qr, kh = t["q"][0, 0, :8], t["k"][0, 0]
    _, _, p = mx.directp_rows(qr, kh, t["v"][0, 0], np.arange(8), False, 0.5)
    tt = 0.5 * qr @ kh.T * mx.LOG2E
    m = np.ceil(tt.max(axis=1))
    exact = 2.0 ** (tt - m[:, None])
    for b0 in range(0, 64, 32):
        blk = exact[:, b0:b0 + 32]
        E = np.floor(np.log2(blk.max(axis=1))) - 2
        y = blk / 2.0 ** E[:, None]
        err = np.abs(p[:, b0:b0 + 32] / 2.0 ** E[:, None] - np.minimum(y, 6.0))
        half_gap = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
        assert np.all(err <= half_gap + 1e-12)


def test_directp_close_to_exact_on_gaussian_inputs():
    """Gaussian softmax test: the Direct-P output tracks exact attention on the same dequantised
    operands.  FP4 weights carry one mantissa bit, so the per-row error is a few percent; the
    mean row cosine stays near 0.99 (the explainer page quotes about 0.944 for its fast path)."""
    t = _mx_case(16, 1, 2, 256, 64)
    o, lse = mx.directp_attention(t["q"], t["k"], t["v"], False, 0.125)
    oe, le = oracle.attention(t["q"], t["k"], t["v"], False, 0.125)
    rel = np.linalg.norm(o - oe) / np.linalg.norm(oe)
    cos = (o * oe).sum(-1) / np.linalg.norm(o, axis=-1) / np.linalg.norm(oe, axis=-1)
    assert rel < 0.2 and cos.mean() > 0.98
    assert np.max(np.abs(lse - le)) < 0.5


def test_directp_gqa_matches_repeated_heads():
    t = _mx_case(17, 1, 4, 64, 32)
    k2, v2 = t["k"][:, :2], t["v"][:, :2]
    o, l = mx.directp_attention(t["q"], k2, v2, True, 0.3)
    om, lm = mx.directp_attention(t["q"], np.repeat(k2, 2, axis=1), np.repeat(v2, 2, axis=1),
                                  True, 0.3)
    assert np.array_equal(o, om) and np.array_equal(l, lm)


@pytest.mark.parametrize("bad", ["no_consistent_norm", "float_ref_max", "no_block_scale"])
def test_planted_directp_mistakes_are_caught(bad, monkeypatch):
    """Planted mistakes in the Direct-P emulation fail the pins above."""
    orig_rows = mx.directp_rows

    def mutated(qt_rows, kt, vt, row_ids, causal, scale, ref_max=None, window=0, docs=None):
        assert window == 0 and docs is None   # the pins below use neither
        if bad == "no_consistent_norm":
            o, lse, p = orig_rows(qt_rows, kt, vt, row_ids, causal, scale, ref_max)
            t = scale * qt_rows @ kt.T * mx.LOG2E
            if causal:
                t = np.where(np.arange(kt.shape[0])[None] > np.asarray(row_ids)[:, None],
                             -np.inf, t)
            m = np.ceil(t.max(axis=1))
            l_exact = np.exp2(t - m[:, None]).sum(axis=1)
            return (p @ vt) / l_exact[:, None], lse, p
        if bad == "float_ref_max":
            t = scale * qt_rows @ kt.T * mx.LOG2E
            m = t.max(axis=1) if ref_max is None else np.asarray(ref_max) + 0.37
            return orig_rows(qt_rows, kt, vt, row_ids, causal, scale, ref_max=m)
        o, lse, p = orig_rows(qt_rows, kt, vt, row_ids, causal, scale, ref_max)
        pz = np.where(p > 0, 2.0 ** np.round(np.log2(np.where(p > 0, p, 1.0))), 0.0)
        return (pz @ vt) / pz.sum(axis=1)[:, None], lse, pz
    monkeypatch.setattr(mx, "directp_rows", mutated)
    pins = [test_directp_constant_v_gives_one, test_directp_zero_query,
            test_directp_independent_of_integer_reference, test_directp_codes_are_rne_of_exp,
            test_directp_exact_when_weights_are_representable]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0


@pytest.mark.parametrize("causal", [False, True])
def test_directp_documents_are_independent_sequences(causal):
    """Packed documents whose offsets are multiples of 32 (the P blocks then coincide): each
    document's rows equal the emulation run on that document alone."""
    t = _mx_case(31, 1, 2, 256, 32)
    docs = [0, 64, 160, 256]
    o, lse = mx.directp_attention(t["q"], t["k"], t["v"], causal, 0.2, docs=docs)
    for a, b in zip(docs[:-1], docs[1:]):
        oa, la = mx.directp_attention(t["q"][:, :, a:b], t["k"][:, :, a:b], t["v"][:, :, a:b],
                                      causal, 0.2)
        assert np.array_equal(o[:, :, a:b], oa) and np.array_equal(lse[:, :, a:b], la)


@pytest.mark.parametrize("causal", [False, True])
def test_directp_window_edges(causal):
    """A narrow window W = 8: the emulation stays within its quantisation error of the exact
    windowed attention, and is far from the exact attention with W - 1 or W + 1 (one key more
    or less per row), so the window's edges are where the definition puts them.  A window of
    N or more is no window."""
    t = _mx_case(32, 1, 2, 128, 32)
    o, _ = mx.directp_attention(t["q"], t["k"], t["v"], causal, 0.2, window=8)

    def rel(x, y):
        return np.linalg.norm(x - y) / np.linalg.norm(y)

    oe, _ = oracle.attention(t["q"], t["k"], t["v"], causal, 0.2, window=8)
    assert rel(o, oe) < 0.12
    for w in (7, 9):
        ow, _ = oracle.attention(t["q"], t["k"], t["v"], causal, 0.2, window=w)
        assert rel(o, ow) > 2 * rel(o, oe)
    o_all, l_all = mx.directp_attention(t["q"], t["k"], t["v"], causal, 0.2, window=128)
    o_none, l_none = mx.directp_attention(t["q"], t["k"], t["v"], causal, 0.2)
    assert np.array_equal(o_all, o_none) and np.array_equal(l_all, l_none)


def test_directp_window_of_one_returns_v():
    """Causal with a window of 1: each row sees only its own key, whose block maximum is its
    score, so x = t - m - E lies in [2, 3), the code is 4 or 6 and O_i = v~_i exactly; the
    LSE is ln 2 (m_i + E_i) + ln code."""
    t = _mx_case(33, 1, 2, 96, 32)
    o, lse = mx.directp_attention(t["q"], t["k"], t["v"], True, 0.3, window=1)
    assert np.array_equal(o, t["v"])
    s = 0.3 * np.einsum("bhnd,bhnd->bhn", t["q"], t["k"]) * mx.LOG2E
    m = np.ceil(s)
    e = np.floor(s - m) - 2.0
    code_val = mx.E2M1_MAGNITUDES[mx.e2m1_round(np.exp2(s - m - e))]
    assert np.all((code_val == 4.0) | (code_val == 6.0))
    assert np.allclose(lse, math.log(2.0) * (m + e) + np.log(code_val), atol=1e-12)


@pytest.mark.parametrize("bad", ["window_one_wider", "documents_ignored"])
def test_planted_mask_mistakes_are_caught(bad, monkeypatch):
    """Planted mistakes in the emulation's masks fail the mask pins above."""
    orig_rows = mx.directp_rows

    def mutated(qt_rows, kt, vt, row_ids, causal, scale, ref_max=None, window=0, docs=None):
        if bad == "window_one_wider" and window:
            window += 1
        if bad == "documents_ignored":
            docs = None
        return orig_rows(qt_rows, kt, vt, row_ids, causal, scale, ref_max, window, docs)
    monkeypatch.setattr(mx, "directp_rows", mutated)
    pins = [lambda: test_directp_documents_are_independent_sequences(True),
            lambda: test_directp_window_edges(True), test_directp_window_of_one_returns_v]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0


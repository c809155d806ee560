"""The exact float64 oracle against its pins, and planted mistakes against the pins."""

import numpy as np
import pytest

import oracle
from oracle import exact
import pins_exact


@pytest.mark.parametrize("pin", pins_exact.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.attention)


@pytest.mark.parametrize("pin", pins_exact.WINDOW_PINS, ids=lambda p: p.__name__)
def test_oracle_window_pin(pin):
    pin(oracle.attention)


@pytest.mark.parametrize("pin", pins_exact.MOD_PINS, ids=lambda p: p.__name__)
def test_oracle_score_mod_pin(pin):
    pin(oracle.attention)


@pytest.mark.parametrize("pin", pins_exact.DOC_PINS, ids=lambda p: p.__name__)
def test_oracle_document_pin(pin):
    pin(oracle.attention)


def test_document_offsets_are_checked():
    with pytest.raises(ValueError):
        exact.document_ids([0, 5, 5, 10], 10)
    with pytest.raises(ValueError):
        exact.document_ids([0, 5, 9], 10)


# planted document-mask mistakes: each must fail at least one document pin
def _dmut_off_by_one(monkeypatch):
    orig = exact.document_ids
    monkeypatch.setattr(exact, "document_ids",
                        lambda off, n: np.minimum(orig(off, n) + (np.arange(n) == np.asarray(off)[1] - 1),
                                                  len(off) - 2))


def _dmut_ignored(monkeypatch):
    monkeypatch.setattr(exact, "document_ids", lambda off, n: np.zeros(n, dtype=np.int64))


def _dmut_keys_only(monkeypatch):
    orig = exact.visible

    def bad(row_ids, n_keys, causal, window=0, docs=None):
        ok = orig(row_ids, n_keys, causal, window, None)
        if docs is not None:   # hides keys of other documents than the first, for every row
            doc = exact.document_ids(docs, n_keys)
            ok &= (doc == 0)[None, :]
        return ok
    monkeypatch.setattr(exact, "visible", bad)


@pytest.mark.parametrize("mutant", [_dmut_off_by_one, _dmut_ignored, _dmut_keys_only],
                         ids=lambda m: m.__name__)
def test_planted_document_mistake_is_caught(mutant, monkeypatch):
    mutant(monkeypatch)
    failures = []
    for pin in pins_exact.DOC_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.attention)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, "a planted document-mask mistake passed every pin"


# planted score-modification mistakes: each must fail at least one score-mod pin
def _smut_alibi_signed(monkeypatch):
    orig = exact.modify_scores

    def bad(s, row_ids, softcap=0.0, alibi_slope=None):
        out = orig(s, row_ids, softcap, None)
        if alibi_slope is not None:   # i - j instead of |i - j|
            out = out - alibi_slope * (np.asarray(row_ids)[:, None] - np.arange(s.shape[1])[None, :])
        return out
    monkeypatch.setattr(exact, "modify_scores", bad)


def _smut_alibi_sign(monkeypatch):
    orig = exact.modify_scores
    monkeypatch.setattr(exact, "modify_scores",
                        lambda s, r, softcap=0.0, alibi_slope=None:
                        orig(s, r, softcap, None if alibi_slope is None else -alibi_slope))


def _smut_softcap_unscaled(monkeypatch):
    orig = exact.modify_scores

    def bad(s, row_ids, softcap=0.0, alibi_slope=None):
        if softcap:
            s = np.tanh(s / softcap) * softcap ** 0.5
        return orig(s, row_ids, 0.0, alibi_slope)
    monkeypatch.setattr(exact, "modify_scores", bad)


def _smut_softcap_after_bias(monkeypatch):
    orig = exact.modify_scores

    def bad(s, row_ids, softcap=0.0, alibi_slope=None):
        s = orig(s, row_ids, 0.0, alibi_slope)
        return softcap * np.tanh(s / softcap) if softcap else s
    monkeypatch.setattr(exact, "modify_scores", bad)


@pytest.mark.parametrize("mutant", [_smut_alibi_signed, _smut_alibi_sign, _smut_softcap_unscaled,
                                    _smut_softcap_after_bias], ids=lambda m: m.__name__)
def test_planted_score_mod_mistake_is_caught(mutant, monkeypatch):
    mutant(monkeypatch)
    failures = []
    for pin in pins_exact.MOD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.attention)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, "a planted score-modification mistake passed every pin"


# planted window mistakes: each must fail at least one window pin
def _wmut_edge_off_by_one(monkeypatch):
    orig = exact.visible

    def bad(row_ids, n_keys, causal, window=0, docs=None):
        return orig(row_ids, n_keys, causal, window + 1 if window else 0, docs)
    monkeypatch.setattr(exact, "visible", bad)


def _wmut_causal_band_both_sides(monkeypatch):
    orig = exact.visible

    def bad(row_ids, n_keys, causal, window=0, docs=None):
        ok = orig(row_ids, n_keys, causal, window, docs)
        if causal and window:   # forgets the causal side inside the band
            i = np.asarray(row_ids)[:, None]
            j = np.arange(n_keys)[None, :]
            ok = ok | ((j > i) & (j < i + window))
        return ok
    monkeypatch.setattr(exact, "visible", bad)


def _wmut_window_ignored(monkeypatch):
    orig = exact.visible
    monkeypatch.setattr(exact, "visible", lambda r, n, c, window=0, docs=None: orig(r, n, c, 0, docs))


@pytest.mark.parametrize("mutant", [_wmut_edge_off_by_one, _wmut_causal_band_both_sides,
                                    _wmut_window_ignored], ids=lambda m: m.__name__)
def test_planted_window_mistake_is_caught(mutant, monkeypatch):
    mutant(monkeypatch)
    failures = []
    for pin in pins_exact.WINDOW_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle.attention)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, "a planted window mistake passed every window pin"


def test_rows_match_full():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 4, 40, 8))
    k = rng.standard_normal((1, 2, 40, 8))
    v = rng.standard_normal((1, 2, 40, 8))
    o, lse = oracle.attention(q, k, v, True, 0.4, chunk=7)
    rows = np.array([0, 5, 39, 17])
    orow, lrow = oracle.attention_rows(q, k, v, True, 0.4, 0, 3, rows)
    assert np.array_equal(orow, o[0, 3, rows]) or np.allclose(orow, o[0, 3, rows], atol=1e-14)
    assert np.allclose(lrow, lse[0, 3, rows], atol=1e-14)


def test_fully_masked_row_reading():
    """A row with no visible key (not reachable with equal Q/K lengths) gives O = 0, LSE = -inf."""
    m, e, l = exact.softmax_parts(np.full((1, 4), -np.inf))
    o, lse = exact.finish(m, e, l, np.ones((4, 3)))
    assert np.all(o == 0) and np.isneginf(lse[0])


# ---- planted mistakes: each must fail at least one pin -------------------------------

def _mut_drop_scale(monkeypatch):
    monkeypatch.setattr(exact, "scores", lambda qr, kh, scale: qr @ kh.T)


def _mut_mask_diagonal(monkeypatch):
    def bad(s, rows, causal, window=0, docs=None):
        if not causal:
            return s
        cols = np.arange(s.shape[1])
        return np.where(cols[None, :] >= rows[:, None], -np.inf, s)
    monkeypatch.setattr(exact, "apply_mask", bad)


def _mut_gqa_modulo(monkeypatch):
    monkeypatch.setattr(exact, "kv_head", lambda hq, Hq, Hkv: hq % Hkv)


def _mut_lse_log2(monkeypatch):
    orig = exact.finish

    def bad(m, e, l, vh):
        o, lse = orig(m, e, l, vh)
        return o, m + np.log2(np.where(l > 0, l, 1.0))
    monkeypatch.setattr(exact, "finish", bad)


def _mut_sign(monkeypatch):
    def bad(s):
        m = s.max(axis=1)
        m_safe = np.where(np.isfinite(m), m, 0.0)
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(m_safe[:, None] - s)
        e = np.where(np.isfinite(s), e, 0.0)
        return m, e, e.sum(axis=1)
    monkeypatch.setattr(exact, "softmax_parts", bad)


def _mut_transposed_operand(monkeypatch):
    orig = exact.attention_rows

    def bad(q, k, v, causal, scale, b, hq, rows, *mods):
        return orig(q, k, k if k.shape == v.shape else v, causal, scale, b, hq, rows, *mods)
    monkeypatch.setattr(exact, "attention_rows", bad)


def _mut_lse_without_max(monkeypatch):
    orig = exact.finish

    def bad(m, e, l, vh):
        o, lse = orig(m, e, l, vh)
        return o, np.log(np.where(l > 0, l, 1.0))
    monkeypatch.setattr(exact, "finish", bad)


def _mut_unnormalised(monkeypatch):
    def bad(m, e, l, vh):
        live = l > 0
        return e @ vh, np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    monkeypatch.setattr(exact, "finish", bad)


MUTANTS = [_mut_drop_scale, _mut_mask_diagonal, _mut_gqa_modulo, _mut_lse_log2, _mut_sign,
           _mut_transposed_operand, _mut_lse_without_max, _mut_unnormalised]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistake_is_caught(mutant, monkeypatch):
    mutant(monkeypatch)
    with np.errstate(all="ignore"):
        failures = pins_exact.run_all(oracle.attention)
    assert failures, "a planted mistake passed every pin"

"""Pins for the float64 attention backward in oracle.backward."""

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bw


def _case(seed, B, Hq, Hkv, N, d, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d)) * sigma
    k = rng.standard_normal((B, Hkv, N, d)) * sigma
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, Hq, N, d))
    return q, k, v, do


def _mask(n, causal, window, docs):
    """Boolean [n, n] visibility written out from the mask rules (independent of the oracle):
    causal j <= i; window i - W < j (and j < i + W when not causal); same document."""
    m = torch.ones(n, n, dtype=torch.bool)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    if causal:
        m &= j <= i
    if window:
        m &= j > i - window
        if not causal:
            m &= j < i + window
    if docs is not None:
        doc = torch.zeros(n, dtype=torch.long)
        for d_idx in range(len(docs) - 1):
            doc[docs[d_idx]:docs[d_idx + 1]] = d_idx
        m &= doc[:, None] == doc[None, :]
    return m


def _torch_grads(q, k, v, do, causal, scale, window=0, docs=None, softcap=0.0, alibi=None):
    """Autograd of a plain float64 softmax attention (GQA by repeating K/V heads), with the
    soft-capping C tanh(s / C) and the ALiBi bias -a_h |i - j| written out."""
    g = q.shape[1] // k.shape[1]
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(g, dim=1)
    vv = tv.repeat_interleave(g, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous())
    if softcap:
        s = softcap * torch.tanh(s / softcap)
    if alibi is not None:
        n = q.shape[2]
        dist = (torch.arange(n)[:, None] - torch.arange(n)[None, :]).abs().to(torch.float64)
        s = s - torch.tensor(alibi, dtype=torch.float64)[None, :, None, None] * dist
    if causal or window or docs is not None:
        s = s.masked_fill(~_mask(q.shape[2], causal, window, docs), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("shape", [(1, 2, 2, 9, 4), (2, 4, 2, 16, 8), (1, 6, 2, 33, 16),
                                   (1, 1, 1, 1, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd(shape, causal):
    B, Hq, Hkv, N, d = shape
    q, k, v, do = _case(sum(shape), B, Hq, Hkv, N, d)
    scale = 0.7
    got = bw.attention_backward(q, k, v, do, causal, scale)
    ref = _torch_grads(q, k, v, do, causal, scale)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, atol=1e-12, rtol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window,docs", [(3, None), (0, [0, 5, 6, 13, 20]), (4, [0, 9, 20])])
def test_masked_matches_torch_autograd(causal, window, docs):
    """Sliding window and packed documents: the same masks as the forward, against autograd."""
    q, k, v, do = _case(31, 1, 4, 2, 20, 8)
    got = bw.attention_backward(q, k, v, do, causal, 0.6, window=window, docs=docs)
    ref = _torch_grads(q, k, v, do, causal, 0.6, window, docs)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, atol=1e-12, rtol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("softcap,alibi,window", [(2.5, None, 0), (0.0, [0.3, 0.05, 0.7, 0.0], 0),
                                                  (1.5, [0.2, 0.4, 0.1, 0.9], 5)])
def test_modified_scores_match_torch_autograd(causal, softcap, alibi, window):
    """Soft-capping and ALiBi (with a window too): the chain rule through the cap, against
    autograd; large logits (sigma 2) so that the cap bends the scores."""
    q, k, v, do = _case(41, 1, 4, 2, 18, 8, sigma=2.0)
    got = bw.attention_backward(q, k, v, do, causal, 0.5, window=window, softcap=softcap,
                                alibi=alibi)
    ref = _torch_grads(q, k, v, do, causal, 0.5, window, None, softcap, alibi)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, atol=1e-12, rtol=1e-10)


def test_modified_scores_finite_differences():
    """Central differences through the cap and the bias on a tiny case."""
    q, k, v, do = _case(42, 1, 1, 1, 6, 2, sigma=2.0)
    alibi = [0.25]
    dq, dk, dv = bw.attention_backward(q, k, v, do, True, 0.9, softcap=1.2, alibi=alibi)

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, True, 0.9, softcap=1.2, alibi=alibi)
        return float(np.sum(o * do))

    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (loss(*[xp if y is x else y for y in (q, k, v)]) -
                  loss(*[xm if y is x else y for y in (q, k, v)])) / (2 * h)
            assert abs(fd - g[idx]) < 1e-7, (idx, fd, g[idx])


def test_dropped_cap_derivative_is_caught(monkeypatch):
    """A backward that forgets the 1 - tanh^2 factor fails the autograd pin."""
    orig = bw.backward_head

    def no_cap_factor(q, k, v, do, causal, scale, o=None, lse=None, window=0, docs=None,
                      softcap=0.0, alibi_slope=None):
        dq, dk, dv = orig(q, k, v, do, causal, scale, o, lse, window, docs, softcap,
                          alibi_slope)
        if softcap:   # undo the factor: recompute with the cap only in P
            rows = np.arange(q.shape[0])
            raw = oracle.exact.scores(q, k, scale)
            fac = 1.0 - np.tanh(raw / softcap) ** 2
            s = oracle.exact.apply_mask(oracle.exact.modify_scores(raw, rows, softcap,
                                                                   alibi_slope),
                                        rows, causal, window, docs)
            p = np.exp(s - lse[:, None])
            ds = p * (do @ v.T - np.sum(do * o, axis=1)[:, None])
            assert np.all(fac > 0)
            return scale * ds @ k, scale * ds.T @ q, dv
        return dq, dk, dv

    monkeypatch.setattr(bw, "backward_head", no_cap_factor)
    with pytest.raises(AssertionError):
        test_modified_scores_match_torch_autograd(False, 2.5, None, 0)


def test_masked_finite_differences_and_isolation():
    """Central differences on a tiny windowed, documented case; and a key outside every
    query's window and document band gets no gradient at all."""
    q, k, v, do = _case(32, 1, 1, 1, 7, 2)
    docs = [0, 3, 7]
    dq, dk, dv = bw.attention_backward(q, k, v, do, False, 0.8, window=2, docs=docs)

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, False, 0.8, window=2, docs=docs)
        return float(np.sum(o * do))

    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (loss(*[xp if y is x else y for y in (q, k, v)]) -
                  loss(*[xm if y is x else y for y in (q, k, v)])) / (2 * h)
            assert abs(fd - g[idx]) < 1e-7, (idx, fd, g[idx])
    # documents of one position see only themselves: their dQ is 0 and their K row is
    # reached by no other query
    q2, k2, v2, do2 = _case(33, 1, 1, 1, 6, 3)
    dq2, dk2, dv2 = bw.attention_backward(q2, k2, v2, do2, False, 0.5, docs=[0, 2, 3, 6])
    assert np.allclose(dq2[0, 0, 2], 0.0, atol=1e-15) and np.allclose(dk2[0, 0, 2], 0.0)
    assert np.allclose(dv2[0, 0, 2], do2[0, 0, 2], atol=1e-14)


def test_finite_differences():
    """Central differences of L = sum(O * dO) against the gradients, element by element on a
    tiny causal GQA case (the forward is the pinned oracle.exact)."""
    q, k, v, do = _case(7, 1, 2, 1, 5, 3)
    scale = 0.9
    dq, dk, dv = bw.attention_backward(q, k, v, do, True, scale)

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, True, scale)
        return float(np.sum(o * do))

    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-7, (idx, fd, g[idx])


def test_shift_and_sum_invariants():
    """Closed forms: adding a constant vector to every key leaves the loss unchanged, so the dK
    rows of each kv head sum to 0 (also under the causal mask, every row keeps its keys);
    the softmax rows sum to 1, so the dV rows of a kv head sum to the dO rows of its query
    heads."""
    q, k, v, do = _case(8, 2, 4, 2, 24, 8)
    for causal in (False, True):
        dq, dk, dv = bw.attention_backward(q, k, v, do, causal, 0.5)
        assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        want = do.reshape(2, 2, 2, 24, 8).sum(axis=(2, 3))
        assert np.allclose(dv.sum(axis=2), want, atol=1e-12)


def test_single_key_row_gets_no_q_gradient():
    """Causal row 0 sees one key: its output is v_0 whatever q_0 is, so dQ_0 = 0."""
    q, k, v, do = _case(9, 1, 2, 2, 12, 4)
    dq, _, _ = bw.attention_backward(q, k, v, do, True, 0.8)
    assert np.allclose(dq[:, :, 0], 0.0, atol=1e-14)


def test_given_forward_outputs_equal_recomputed():
    q, k, v, do = _case(10, 1, 2, 2, 20, 6)
    o, lse = oracle.attention(q, k, v, True, 0.4)
    a = bw.attention_backward(q, k, v, do, True, 0.4, o=o, lse=lse)
    b = bw.attention_backward(q, k, v, do, True, 0.4)
    for x, y in zip(a, b):
        assert np.allclose(x, y, atol=1e-14)
    assert np.allclose(bw.delta(o, do), np.sum(o * do, axis=-1))


@pytest.mark.parametrize("bad", ["no_delta", "no_scale_dk", "gqa_last_head", "p_unnormalised"])
def test_planted_mistakes_are_caught(bad, monkeypatch):
    orig = bw.backward_head

    def mutated(q, k, v, do, causal, scale, o=None, lse=None, window=0, docs=None,
                softcap=0.0, alibi_slope=None):
        dq, dk, dv = orig(q, k, v, do, causal, scale, o, lse, window, docs, softcap,
                          alibi_slope)
        if bad == "no_delta":
            rows = np.arange(q.shape[0])
            s = oracle.exact.apply_mask(scale * q @ k.T, rows, causal, window, docs)
            p = np.exp(s - lse[:, None])
            ds = p * (do @ v.T)
            return scale * ds @ k, scale * ds.T @ q, dv
        if bad == "no_scale_dk":
            return dq, dk / scale, dv
        if bad == "p_unnormalised":
            return dq, dk, dv * 1.5
        return dq, dk, dv

    monkeypatch.setattr(bw, "backward_head", mutated)
    if bad == "gqa_last_head":
        orig_all = bw.attention_backward

        def keep_last(q, k, v, do, causal, scale, o=None, lse=None, window=0, docs=None,
                      softcap=0.0, alibi=None):
            dq, dk, dv = orig_all(q, k, v, do, causal, scale, o, lse, window, docs, softcap,
                                  alibi)
            g = q.shape[1] // k.shape[1]
            if g > 1:   # as if only the group's last query head were counted
                for hk in range(k.shape[1]):
                    _, dk1, dv1 = orig(q[0, hk * g + g - 1], k[0, hk], v[0, hk],
                                       do[0, hk * g + g - 1], causal, scale)
                    dk[0, hk], dv[0, hk] = dk1, dv1
            return dq, dk, dv
        monkeypatch.setattr(bw, "attention_backward", keep_last)
    pins = [lambda: test_matches_torch_autograd((2, 4, 2, 16, 8), True),
            test_shift_and_sum_invariants]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0


def test_delta_is_sum_of_p_times_dp_brute_force():
    """D_i = dO_i . O_i equals sum_j P_ij dP_ij with P the softmax of the scores and
    dP_ij = dO_i . v_j, both written out as scalar loops (math.exp), independent of how
    the oracle forms O."""
    import math
    q, k, v, do = _case(21, 1, 2, 1, 9, 5)
    for causal in (False, True):
        scale = 0.7
        o, _ = oracle.attention(q, k, v, causal, scale)
        got = bw.delta(o, do)
        for h in range(2):
            for i in range(9):
                keys = [j for j in range(9) if not (causal and j > i)]
                s = [scale * sum(q[0, h, i, c] * k[0, 0, j, c] for c in range(5)) for j in keys]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = sum(e)
                want = sum(e[n] / tot * sum(do[0, h, i, c] * v[0, 0, j, c] for c in range(5))
                           for n, j in enumerate(keys))
                assert abs(got[0, h, i] - want) <= 1e-12 * max(1.0, abs(want))


def test_planted_delta_mistakes_are_caught(monkeypatch):
    """A sign flip or a missing row of the product in delta fails the brute-force pin."""
    orig = bw.delta
    for bad in ("sign", "drop_last_column"):
        def mutated(o, do, bad=bad):
            if bad == "sign":
                return -orig(o, do)
            return orig(o[..., :-1], do[..., :-1])
        monkeypatch.setattr(bw, "delta", mutated)
        with pytest.raises(AssertionError):
            test_delta_is_sum_of_p_times_dp_brute_force()
    monkeypatch.setattr(bw, "delta", orig)


@pytest.mark.parametrize("mask", ["none", "causal", "window", "docs_mods"])
def test_backward_rows_equal_full_backward(mask):
    """Sampled rows and columns of the gradients equal the full backward's, under every mask
    and the score modifications (the row function forms only those rows and columns)."""
    q, k, v, do = _case(22, 1, 1, 1, 40, 6)
    kw = dict(causal=False, window=0, docs=None, softcap=0.0, alibi_slope=None)
    if mask == "causal":
        kw["causal"] = True
    elif mask == "window":
        kw.update(causal=True, window=7)
    elif mask == "docs_mods":
        kw.update(docs=[0, 13, 14, 40], softcap=1.5, alibi_slope=0.3)
    scale = 0.6
    alibi = None if kw["alibi_slope"] is None else [kw["alibi_slope"]]
    o, lse = oracle.attention(q, k, v, kw["causal"], scale, window=kw["window"], docs=kw["docs"],
                              softcap=kw["softcap"], alibi=alibi)
    full = bw.backward_head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], kw["causal"], scale, o[0, 0],
                            lse[0, 0], kw["window"], kw["docs"], kw["softcap"], kw["alibi_slope"])
    qrows, krows = np.array([0, 5, 13, 39]), np.array([1, 13, 14, 38, 39])
    dq, dk, dv = bw.backward_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], kw["causal"], scale,
                                  o[0, 0], lse[0, 0], qrows, krows, kw["window"], kw["docs"],
                                  kw["softcap"], kw["alibi_slope"])
    assert np.allclose(dq, full[0][qrows], rtol=1e-12, atol=1e-14)
    assert np.allclose(dk, full[1][krows], rtol=1e-12, atol=1e-14)
    assert np.allclose(dv, full[2][krows], rtol=1e-12, atol=1e-14)

"""Pins for an exact attention-forward implementation `attn(q, k, v, causal, scale) -> (O, LSE)`.

Each pin ties the function to something other than itself: brute force on
tiny inputs, torch's CPU attention routine in float64 (an independent library
implementation that also returns the log-sum-exp), closed forms and
invariants of softmax attention.  The pins take the function as an argument
so that the mutation tests can show that a planted mistake in the oracle
fails at least one of them.
"""

import numpy as np
import scipy.special
import torch

from oracle import attention_brute

TOL = 1e-11


def _rand(rng, shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


def _case(seed, B, Hq, Hkv, N, d, sigma=1.0):
    rng = np.random.default_rng(seed)
    return (_rand(rng, (B, Hq, N, d), sigma), _rand(rng, (B, Hkv, N, d), sigma),
            _rand(rng, (B, Hkv, N, d)))


def pin_brute(attn):
    """Agreement with scalar loops + math.exp on tiny shapes, both masks, MHA/GQA."""
    shapes = [(1, 1, 1, 1, 1), (1, 2, 2, 2, 4), (1, 2, 1, 3, 8), (2, 4, 2, 7, 4),
              (1, 4, 1, 16, 8), (1, 2, 2, 5, 1)]
    for n, (B, Hq, Hkv, N, d) in enumerate(shapes):
        q, k, v = _case(100 + n, B, Hq, Hkv, N, d, sigma=1.5)
        for causal in (False, True):
            scale = 0.37 + 0.1 * n
            o, lse = attn(q, k, v, causal, scale)
            ob, lseb = attention_brute(q, k, v, causal, scale)
            assert np.max(np.abs(o - ob)) < TOL, ("brute O", B, Hq, Hkv, N, d, causal)
            assert np.max(np.abs(lse - lseb)) < TOL, ("brute LSE", B, Hq, Hkv, N, d, causal)


def pin_torch(attn):
    """Agreement with torch's CPU attention (float64) including its log-sum-exp."""
    op = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu
    for n, (B, Hq, Hkv, N, d) in enumerate([(2, 4, 4, 33, 16), (1, 8, 2, 64, 32),
                                             (1, 2, 1, 100, 64)]):
        q, k, v = _case(200 + n, B, Hq, Hkv, N, d)
        g = Hq // Hkv
        kt = torch.from_numpy(np.repeat(k, g, axis=1))
        vt = torch.from_numpy(np.repeat(v, g, axis=1))
        for causal in (False, True):
            scale = 1.0 / np.sqrt(d) * (1.0 + 0.25 * n)
            ref_o, ref_lse = op(torch.from_numpy(q), kt, vt, 0.0, causal, scale=scale)
            o, lse = attn(q, k, v, causal, scale)
            assert np.max(np.abs(o - ref_o.numpy())) < 1e-10, ("torch O", causal, n)
            assert np.max(np.abs(lse - ref_lse.numpy())) < 1e-10, ("torch LSE", causal, n)


def pin_zero_query(attn):
    """Q = 0: every logit is 0, so O is the mean of the visible V rows and LSE = ln(count)."""
    B, H, N, d = 1, 2, 12, 8
    _, k, v = _case(300, B, H, H, N, d)
    q = np.zeros((B, H, N, d))
    o, lse = attn(q, k, v, False, 0.7)
    assert np.allclose(o, v.mean(axis=2, keepdims=True).repeat(N, axis=2), atol=TOL)
    assert np.allclose(lse, np.log(N), atol=TOL)
    o, lse = attn(q, k, v, True, 0.7)
    prefix = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.allclose(o, prefix, atol=TOL)
    assert np.allclose(lse, np.log(np.arange(1, N + 1))[None, None, :], atol=TOL)


def pin_single_key(attn):
    """One visible key: O is that key's V row and LSE is its logit scale*q.k."""
    q, k, v = _case(400, 1, 3, 3, 1, 16)
    o, lse = attn(q, k, v, False, 0.3)
    assert np.allclose(o, v, atol=TOL)
    assert np.allclose(lse, 0.3 * np.einsum("bhnd,bhnd->bhn", q, k), atol=TOL)
    q, k, v = _case(401, 1, 2, 2, 9, 16)
    o, lse = attn(q, k, v, True, 0.3)
    assert np.allclose(o[:, :, 0], v[:, :, 0], atol=TOL)
    assert np.allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                       atol=TOL)


def pin_two_keys(attn):
    """d = 1, two keys: O = v0 + (v1 - v0) * logistic(s1 - s0) and LSE = logaddexp(s0, s1)."""
    q = np.array([[[[1.3]]]])
    k = np.array([[[[0.4], [-1.1]]]])
    v = np.array([[[[2.0], [-3.0]]]])
    q2 = np.concatenate([q, -q], axis=2)
    for scale in (0.5, 2.0):
        o, lse = attn(q2, k, v, False, scale)
        for i, qi in enumerate((1.3, -1.3)):
            s0, s1 = scale * qi * 0.4, scale * qi * -1.1
            w1 = scipy.special.expit(s1 - s0)
            assert abs(o[0, 0, i, 0] - (2.0 + (-3.0 - 2.0) * w1)) < TOL
            assert abs(lse[0, 0, i] - np.logaddexp(s0, s1)) < TOL


def pin_constant_v(attn):
    """V = 1 everywhere gives O = 1 (the weights of each row sum to 1)."""
    q, k, _ = _case(500, 1, 4, 2, 20, 8, sigma=2.0)
    v = np.ones((1, 2, 20, 8))
    for causal in (False, True):
        o, _ = attn(q, k, v, causal, 0.9)
        assert np.allclose(o, 1.0, atol=TOL)


def pin_identity_v(attn):
    """V = identity (d = N): O is P itself, so rows are >= 0, sum to 1, and vanish above the diagonal."""
    N = 10
    q, k, _ = _case(600, 1, 1, 1, N, 6, sigma=1.5)
    v = np.eye(N)[None, None]
    for causal in (False, True):
        p, lse = attn(q, k, v, causal, 0.8)
        assert np.all(p >= 0)
        assert np.allclose(p.sum(axis=-1), 1.0, atol=TOL)
        s = 0.8 * q[0, 0] @ k[0, 0].T
        # softmax ratios are exp of logit differences
        i, j1, j2 = 7, 2, 5
        assert abs(np.log(p[0, 0, i, j1] / p[0, 0, i, j2]) - (s[i, j1] - s[i, j2])) < 1e-9
        # each weight is exp(s - LSE)
        assert np.allclose(p[0, 0, i, j1], np.exp(s[i, j1] - lse[0, 0, i]), atol=TOL)
        if causal:
            assert np.all(np.triu(p[0, 0], 1) == 0)


def pin_shift(attn):
    """k_j += w for every j: O is unchanged and LSE_i grows by scale * q_i . w."""
    q, k, v = _case(700, 1, 2, 2, 15, 8)
    w = np.random.default_rng(7).standard_normal(8)
    for causal in (False, True):
        o0, l0 = attn(q, k, v, causal, 0.6)
        o1, l1 = attn(q, k + w, v, causal, 0.6)
        assert np.allclose(o0, o1, atol=1e-10)
        assert np.allclose(l1 - l0, 0.6 * q @ w, atol=1e-10)


def pin_permutations(attn):
    """Non-causal: permuting keys with values changes nothing; permuting queries permutes the rows."""
    q, k, v = _case(800, 1, 2, 2, 13, 8)
    rng = np.random.default_rng(8)
    pk, pq = rng.permutation(13), rng.permutation(13)
    o, lse = attn(q, k, v, False, 0.5)
    o1, l1 = attn(q, k[:, :, pk], v[:, :, pk], False, 0.5)
    assert np.allclose(o, o1, atol=TOL) and np.allclose(lse, l1, atol=TOL)
    o2, l2 = attn(q[:, :, pq], k, v, False, 0.5)
    assert np.allclose(o[:, :, pq], o2, atol=TOL) and np.allclose(lse[:, :, pq], l2, atol=TOL)


def pin_linear_in_v(attn):
    """O is linear in V: O(a V1 + b V2) = a O(V1) + b O(V2)."""
    q, k, v1 = _case(900, 1, 2, 1, 11, 8)
    v2 = np.random.default_rng(9).standard_normal(v1.shape)
    for causal in (False, True):
        o1, _ = attn(q, k, v1, causal, 0.5)
        o2, _ = attn(q, k, v2, causal, 0.5)
        o3, _ = attn(q, k, 2.5 * v1 - 0.75 * v2, causal, 0.5)
        assert np.allclose(o3, 2.5 * o1 - 0.75 * o2, atol=1e-10)


def pin_gqa(attn):
    """GQA equals MHA with each K/V head repeated for its Hq/Hkv query heads."""
    q, k, v = _case(1000, 2, 6, 2, 9, 8)
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.5)
        om, lm = attn(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), causal, 0.5)
        assert np.allclose(o, om, atol=TOL) and np.allclose(lse, lm, atol=TOL)


def pin_causal_prefix(attn):
    """Causal row i equals non-causal attention of query i over keys 0..i."""
    q, k, v = _case(1100, 1, 2, 2, 10, 8)
    oc, lc = attn(q, k, v, True, 0.5)
    for i in (0, 3, 9):
        on, ln = attn(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], False, 0.5)
        assert np.allclose(oc[:, :, i], on[:, :, 0], atol=TOL)
        assert np.allclose(lc[:, :, i], ln[:, :, 0], atol=TOL)


def pin_dominant_logit(attn):
    """A key whose logit exceeds the others by 50 takes all the weight."""
    q, k, v = _case(1200, 1, 1, 1, 8, 4)
    q[0, 0, 3] = np.array([1.0, 0.0, 0.0, 0.0])
    k[0, 0, :, 0] = 0.0
    k[0, 0, 5, 0] = 50.0
    o, lse = attn(q, k, v, False, 1.0)
    assert np.allclose(o[0, 0, 3], v[0, 0, 5], atol=1e-12)
    assert abs(lse[0, 0, 3] - 50.0) < 1e-12


# ---- sliding window (attn(..., window=W)) -----------------------------------------------

def _visible_range(i, N, causal, W):
    """[lo, hi] of the keys query i sees under window W (W = 0: no window)."""
    lo = max(0, i - W + 1) if W else 0
    hi = i if causal else (min(N - 1, i + W - 1) if W else N - 1)
    return lo, hi


def pin_window_brute(attn):
    """Agreement with the scalar loops on tiny shapes, windows 1..N+1, both masks."""
    for n, (B, Hq, Hkv, N, d) in enumerate([(1, 2, 1, 7, 4), (1, 1, 1, 9, 3), (2, 2, 2, 5, 2)]):
        q, k, v = _case(300 + n, B, Hq, Hkv, N, d, sigma=1.3)
        for W in (1, 2, 3, N - 1, N + 1):
            for causal in (False, True):
                o, lse = attn(q, k, v, causal, 0.6, window=W)
                ob, lseb = attention_brute(q, k, v, causal, 0.6, window=W)
                assert np.max(np.abs(o - ob)) < TOL, ("window brute O", n, W, causal)
                assert np.max(np.abs(lse - lseb)) < TOL, ("window brute LSE", n, W, causal)


def pin_window_one(attn):
    """W = 1: every query sees only its own key, so O_i = v_i and LSE_i = scale q_i.k_i."""
    q, k, v = _case(310, 1, 4, 2, 12, 8)
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.45, window=1)
        kk, vv = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
        assert np.max(np.abs(o - vv)) < TOL
        assert np.max(np.abs(lse - 0.45 * np.sum(q * kk, axis=-1))) < TOL


def pin_window_zero_query(attn):
    """Q = 0: O_i is the mean of exactly the visible V rows and LSE_i = ln(their count)."""
    N = 23
    _, k, v = _case(311, 1, 2, 2, N, 4)
    q = np.zeros((1, 2, N, 4))
    for W in (1, 4, 9, 40):
        for causal in (False, True):
            o, lse = attn(q, k, v, causal, 0.8, window=W)
            for i in range(N):
                lo, hi = _visible_range(i, N, causal, W)
                assert np.max(np.abs(o[0, :, i] - v[0, :, lo:hi + 1].mean(axis=1))) < TOL, (W, i)
                assert abs(lse[0, 0, i] - np.log(hi - lo + 1)) < TOL, (W, i)


def pin_window_torch(attn):
    """Agreement with torch's CPU attention (float64) given the band as an explicit mask."""
    q, k, v = _case(312, 1, 4, 4, 50, 16)
    for W in (3, 17):
        for causal in (False, True):
            i = np.arange(50)[:, None]
            j = np.arange(50)[None, :]
            band = (j > i - W) & ((j <= i) if causal else (j < i + W))
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                attn_mask=torch.from_numpy(band), scale=0.3)
            o, _ = attn(q, k, v, causal, 0.3, window=W)
            assert np.max(np.abs(o - ref.numpy())) < 1e-10, ("window torch", W, causal)


def pin_window_wide_is_plain(attn):
    """A window at least N wide hides nothing beyond the causal mask."""
    q, k, v = _case(313, 1, 2, 1, 31, 8)
    for causal in (False, True):
        o0, l0 = attn(q, k, v, causal, 0.5)
        for W in (31, 32, 1000):
            o, l = attn(q, k, v, causal, 0.5, window=W)
            assert np.max(np.abs(o - o0)) < TOL and np.max(np.abs(l - l0)) < TOL


WINDOW_PINS = [pin_window_brute, pin_window_one, pin_window_zero_query, pin_window_torch,
               pin_window_wide_is_plain]


# ---- score modifications (attn(..., softcap=C, alibi=slopes)) -----------------------------

def _slopes(H):
    return 0.5 ** (np.arange(1, H + 1) * 8.0 / H)   # a geometric sequence of per-head slopes


def pin_mod_brute(attn):
    """Agreement with the scalar loops: soft-capping, ALiBi, both, with the masks and a window."""
    for n, (B, Hq, Hkv, N, d) in enumerate([(1, 2, 1, 7, 4), (1, 4, 2, 9, 3), (2, 2, 2, 5, 2)]):
        q, k, v = _case(400 + n, B, Hq, Hkv, N, d, sigma=2.0)
        for causal in (False, True):
            for cap, alibi, W in ((3.0, None, 0), (0.0, _slopes(Hq), 0), (2.5, _slopes(Hq), 0),
                                  (4.0, _slopes(Hq), 3)):
                o, lse = attn(q, k, v, causal, 0.7, window=W, softcap=cap, alibi=alibi)
                ob, lb = attention_brute(q, k, v, causal, 0.7, window=W, softcap=cap, alibi=alibi)
                assert np.max(np.abs(o - ob)) < TOL and np.max(np.abs(lse - lb)) < TOL, \
                    ("mod brute", n, causal, cap, alibi is not None, W)


def pin_mod_torch(attn):
    """torch's CPU attention (float64) fed the modified scores as an additive mask with
    Q = 0 (ALiBi: the bias; soft-capping: the capped scores themselves)."""
    q, k, v = _case(410, 1, 4, 4, 40, 8, sigma=2.0)
    i = np.arange(40)[:, None]
    j = np.arange(40)[None, :]
    for causal in (False, True):
        hide = (j > i) if causal else np.zeros((40, 40), bool)
        for cap, alibi in ((3.0, None), (0.0, _slopes(4)), (2.0, _slopes(4))):
            s = 0.5 * np.einsum("bhid,bhjd->bhij", q, k)
            if cap:
                s = cap * np.tanh(s / cap)
            if alibi is not None:
                s = s - alibi[None, :, None, None] * np.abs(i - j)[None, None]
            s = np.where(hide[None, None], -np.inf, s)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.zeros(1, 4, 40, 8, dtype=torch.float64), torch.from_numpy(k),
                torch.from_numpy(v), attn_mask=torch.from_numpy(s))
            o, _ = attn(q, k, v, causal, 0.5, softcap=cap, alibi=alibi)
            assert np.max(np.abs(o - ref.numpy())) < 1e-10, ("mod torch", causal, cap)


def pin_alibi_zero_query(attn):
    """Q = 0 with ALiBi: the weights are exp(-a |i - j|), so O_i and LSE_i are explicit
    geometric sums over the visible keys."""
    N = 19
    _, k, v = _case(411, 1, 2, 2, N, 4)
    q = np.zeros((1, 2, N, 4))
    slopes = np.array([0.3, 1.7])
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.9, alibi=slopes)
        for h in range(2):
            for r in range(N):
                js = np.arange(0, r + 1 if causal else N)
                w = np.exp(-slopes[h] * np.abs(r - js))
                assert np.max(np.abs(o[0, h, r] - (w @ v[0, h, js]) / w.sum())) < TOL
                assert abs(lse[0, h, r] - np.log(w.sum())) < TOL


def pin_softcap_limits(attn):
    """A cap far above every score leaves attention unchanged (to the cap's cubic term);
    scores far above the cap saturate at it, so rows of huge equal logits become uniform."""
    q, k, v = _case(412, 1, 2, 2, 17, 8)
    for causal in (False, True):
        o0, l0 = attn(q, k, v, causal, 0.3)
        o, l = attn(q, k, v, causal, 0.3, softcap=1e6)   # |C tanh(s/C) - s| <= |s|^3 / (3 C^2)
        assert np.max(np.abs(o - o0)) < 1e-9 and np.max(np.abs(l - l0)) < 1e-9
    k2 = np.ones_like(k)
    q2 = np.full_like(q, 50.0)                # every score 0.3 * 8 * 50 = 120 >> cap
    o, l = attn(q2, k2, v, False, 0.3, softcap=2.0)
    assert np.max(np.abs(o - v.mean(axis=2, keepdims=True))) < 1e-9
    assert np.max(np.abs(l - (2.0 * np.tanh(60.0) + np.log(17)))) < 1e-9


MOD_PINS = [pin_mod_brute, pin_mod_torch, pin_alibi_zero_query, pin_softcap_limits]


# ---- document masking (attn(..., docs=offsets)) -------------------------------------------

def pin_docs_brute(attn):
    """Agreement with the scalar loops, with the masks, a window and score modifications."""
    q, k, v = _case(500, 1, 2, 1, 11, 4, sigma=1.5)
    for docs in ([0, 11], [0, 4, 11], [0, 1, 2, 7, 11], [0, 5, 6, 11]):
        for causal in (False, True):
            for W, cap in ((0, 0.0), (3, 0.0), (0, 2.0)):
                o, lse = attn(q, k, v, causal, 0.6, window=W, softcap=cap, docs=docs)
                ob, lb = attention_brute(q, k, v, causal, 0.6, window=W, softcap=cap, docs=docs)
                assert np.max(np.abs(o - ob)) < TOL and np.max(np.abs(lse - lb)) < TOL, \
                    ("docs brute", docs, causal, W, cap)


def pin_docs_are_independent_sequences(attn):
    """Each document attends like a separate sequence: the result equals plain attention run
    on every document's slice on its own."""
    q, k, v = _case(501, 2, 4, 2, 40, 8)
    docs = [0, 7, 8, 25, 40]
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.4, docs=docs)
        for a, b in zip(docs[:-1], docs[1:]):
            os_, ls_ = attn(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], causal, 0.4)
            assert np.max(np.abs(o[:, :, a:b] - os_)) < TOL
            assert np.max(np.abs(lse[:, :, a:b] - ls_)) < TOL


def pin_docs_zero_query(attn):
    """Q = 0: O_i is the mean of the V rows of i's document (causal: up to i), LSE_i the log
    of their count."""
    N = 21
    _, k, v = _case(502, 1, 2, 2, N, 4)
    q = np.zeros((1, 2, N, 4))
    docs = [0, 3, 4, 13, 21]
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.8, docs=docs)
        for a, b in zip(docs[:-1], docs[1:]):
            for i in range(a, b):
                hi = i if causal else b - 1
                assert np.max(np.abs(o[0, :, i] - v[0, :, a:hi + 1].mean(axis=1))) < TOL
                assert abs(lse[0, 1, i] - np.log(hi - a + 1)) < TOL


def pin_docs_torch(attn):
    """torch's CPU attention (float64) with the block-diagonal mask spelled out."""
    q, k, v = _case(503, 1, 2, 2, 30, 16)
    docs = [0, 10, 11, 30]
    doc = np.repeat(np.arange(3), np.diff(docs))
    for causal in (False, True):
        m = doc[:, None] == doc[None, :]
        if causal:
            m &= np.arange(30)[None, :] <= np.arange(30)[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=torch.from_numpy(m), scale=0.35)
        o, _ = attn(q, k, v, causal, 0.35, docs=docs)
        assert np.max(np.abs(o - ref.numpy())) < 1e-10


DOC_PINS = [pin_docs_brute, pin_docs_are_independent_sequences, pin_docs_zero_query,
            pin_docs_torch]


ALL_PINS = [pin_brute, pin_torch, pin_zero_query, pin_single_key, pin_two_keys,
            pin_constant_v, pin_identity_v, pin_shift, pin_permutations, pin_linear_in_v,
            pin_gqa, pin_causal_prefix, pin_dominant_logit]


def run_all(attn):
    failures = []
    for pin in ALL_PINS:
        try:
            pin(attn)
        except (AssertionError, ValueError, IndexError) as exc:
            failures.append((pin.__name__, exc))
    return failures

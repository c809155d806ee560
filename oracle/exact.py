"""Exact attention forward in float64: the plain definition, no tiling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed (the series' forward, "FlashAttention-4发布：原生支持
Blackwell…", section "从V1到V4", FlashAttention (2022) entry: tiling and
recomputation reach the same output without storing the N x N matrix):

    s_ij   = scale * sum_c q[i, c] * k[j, c]
    s_ij   = -inf            if causal and j > i
    m_i    = max_j s_ij
    l_i    = sum_j exp(s_ij - m_i)
    O[i,:] = sum_j exp(s_ij - m_i) * v[j, :] / l_i
    LSE_i  = m_i + ln(l_i)                      (natural log)

Sliding window (the FlexAttention news page, body: sliding window attention is
one of the patterns the FA4 backend serves; the page prints no definition).
Reading: with a window W >= 1, key j is visible from query i only when
i - W < j, and, without the causal mask, also j < i + W (a band of half-width
W - 1 around the diagonal).  W = 0 means no window.

Document masking (same page, same list; no definition printed).  Reading: the
sequence holds documents packed back to back, given by offsets 0 = o_0 < o_1 < ... <
o_D = N (document d is positions o_d .. o_{d+1} - 1, the same layout for every batch
entry), and key j is visible from query i only when both lie in the same document.
It combines with the causal mask and the window.

Score modifications (the same page names ALiBi and soft-capping among the patterns the
FA4 backend serves, again without definitions).  Readings, applied to the scaled score
before the mask, soft-capping first:

    soft-capping with cap C > 0:    s_ij <- C * tanh(s_ij / C)
    ALiBi with per-head slope a_h:  s_ij <- s_ij - a_h * |i - j|

(|i - j| = i - j under the causal mask.)  The slopes are an input, one per query head.

Grouped-query attention (named in the same section's FlashAttention-2 entry)
maps query head hq to key/value head hq // (Hq / Hkv).  A row whose keys are
all masked (never reached with the causal mask when Q and K have the same
length) gets O = 0 and LSE = -inf.

Inputs are float64 arrays q [B, Hq, N, d], k and v [B, Hkv, N, d]; bf16
inputs are widened exactly by the caller.
"""

import math

import numpy as np


def kv_head(hq, Hq, Hkv):
    """Key/value head serving query head hq: contiguous groups of Hq/Hkv heads."""
    return hq // (Hq // Hkv)


def scores(q_rows, k_head, scale):
    """scale * q_rows @ k^T  ->  [rows, N_k]."""
    return scale * (q_rows @ k_head.T)


def modify_scores(s, row_ids, softcap=0.0, alibi_slope=None):
    """Soft-capping C*tanh(s/C) (C > 0), then the ALiBi bias -slope*|i - j|."""
    if softcap:
        s = softcap * np.tanh(s / softcap)
    if alibi_slope is not None:
        dist = np.abs(np.asarray(row_ids)[:, None] - np.arange(s.shape[1])[None, :])
        s = s - alibi_slope * dist
    return s


def document_ids(doc_offsets, n):
    """Document index of each of the n positions, from the offsets o_0 = 0 < ... < o_D = n."""
    off = np.asarray(doc_offsets, dtype=np.int64)
    if off[0] != 0 or off[-1] != n or np.any(np.diff(off) <= 0):
        raise ValueError("document offsets must rise strictly from 0 to N")
    return np.searchsorted(off, np.arange(n), side="right") - 1


def visible(row_ids, n_keys, causal, window=0, docs=None):
    """Boolean [rows, n_keys]: key j visible from query i (causal: j <= i; window W:
    i - W < j, and j < i + W when not causal; documents: same document)."""
    i = np.asarray(row_ids)[:, None]
    j = np.arange(n_keys)[None, :]
    ok = np.ones((i.shape[0], n_keys), dtype=bool)
    if causal:
        ok &= j <= i
    if window:
        ok &= j > i - window
        if not causal:
            ok &= j < i + window
    if docs is not None:
        doc = document_ids(docs, n_keys)
        ok &= doc[np.asarray(row_ids)][:, None] == doc[None, :]
    return ok


def apply_mask(s, row_ids, causal, window=0, docs=None):
    """Additive -inf mask on the keys that `visible` hides."""
    if not causal and not window and docs is None:
        return s
    return np.where(visible(row_ids, s.shape[1], causal, window, docs), s, -np.inf)


def softmax_parts(s):
    """Row max m, unnormalised weights e = exp(s - m) and their sum l."""
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    return m, e, l


def finish(m, e, l, v_head):
    """O = (e @ v) / l and LSE = m + ln l; all-masked rows give O = 0, LSE = -inf."""
    live = l > 0
    l_safe = np.where(live, l, 1.0)
    o = (e @ v_head) / l_safe[:, None]
    o[~live] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(live, m + np.log(l_safe), -np.inf)
    return o, lse


def attention_rows(q, k, v, causal, scale, b, hq, rows, window=0, softcap=0.0, alibi=None,
                   docs=None):
    """O and LSE for the listed query rows of one (batch, query head) slice.  alibi: the
    per-query-head slopes (length Hq) or None."""
    B, Hq, N, d = q.shape
    hk = kv_head(hq, Hq, k.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    s = scores(q[b, hq, rows, :], k[b, hk], scale)
    s = modify_scores(s, rows, softcap, None if alibi is None else float(alibi[hq]))
    s = apply_mask(s, rows, causal, window, docs)
    m, e, l = softmax_parts(s)
    return finish(m, e, l, v[b, hk])


def attention_head(q, k, v, causal, scale, b, hq, chunk=512, window=0, softcap=0.0, alibi=None,
                   docs=None):
    """All rows of one (batch, query head) slice, in chunks of whole rows."""
    N = q.shape[2]
    o = np.empty((N, v.shape[3]), dtype=np.float64)
    lse = np.empty((N,), dtype=np.float64)
    for r0 in range(0, N, chunk):
        rows = np.arange(r0, min(N, r0 + chunk))
        o[rows], lse[rows] = attention_rows(q, k, v, causal, scale, b, hq, rows, window,
                                            softcap, alibi, docs)
    return o, lse


def attention(q, k, v, causal, scale, chunk=512, window=0, softcap=0.0, alibi=None, docs=None):
    """Exact forward over the whole [B, Hq, N, d] problem: returns (O, LSE)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    if k.shape[1] == 0 or Hq % k.shape[1] != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    o = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.empty(q.shape[:3], dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            o[b, hq], lse[b, hq] = attention_head(q, k, v, causal, scale, b, hq, chunk, window,
                                                  softcap, alibi, docs)
    return o, lse


def attention_brute(q, k, v, causal, scale, window=0, softcap=0.0, alibi=None, docs=None):
    """The same definition as scalar Python loops with math.exp (tiny inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    group = Hq // Hkv
    doc_of = None
    if docs is not None:                  # position -> document, by walking the offsets
        doc_of = []
        for dd in range(len(docs) - 1):
            doc_of += [dd] * (int(docs[dd + 1]) - int(docs[dd]))
    o = np.zeros((B, Hq, N, dv))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(N):
                s = []
                for j in range(Nk):
                    if causal and j > i:
                        continue
                    if window and (i - j >= window or (not causal and j - i >= window)):
                        continue
                    if doc_of is not None and doc_of[i] != doc_of[j]:
                        continue
                    acc = 0.0
                    for c in range(d):
                        acc += float(q[b, h, i, c]) * float(k[b, g, j, c])
                    val = scale * acc
                    if softcap:
                        val = softcap * math.tanh(val / softcap)
                    if alibi is not None:
                        val -= float(alibi[h]) * abs(i - j)
                    s.append((j, val))
                if not s:
                    lse[b, h, i] = -math.inf
                    continue
                mx = max(val for _, val in s)
                w = [(j, math.exp(val - mx)) for j, val in s]
                tot = sum(x for _, x in w)
                for c in range(dv):
                    o[b, h, i, c] = sum(x * float(v[b, g, j, c]) for j, x in w) / tot
                lse[b, h, i] = mx + math.log(tot)
    return o, lse

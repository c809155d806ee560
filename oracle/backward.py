"""Exact attention backward in float64: the gradients of the forward's plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages give.  The series keeps memory linear by not storing the N x N
matrix and recomputing it in the backward pass ("FlashAttention-4发布：原生支持
Blackwell…", section "从V1到V4", FlashAttention (2022) entry: tiling plus
recomputation); "Hardware-Aware FP4 FlashAttention-4", section "2. Causal
Backward Cuantizado", saves the log-sum-exp in the forward so that the backward
rebuilds the probabilities from it.  The pages print no formula, so this is the
chain rule applied to the forward's definition (oracle.exact), with P rebuilt
from the saved LSE:

    s_ij   = scale * q_i . k_j            (-inf where masked)
    P_ij   = exp(s_ij - LSE_i)            the forward's probabilities
    dV_j   = sum_i P_ij dO_i
    dP_ij  = dO_i . v_j
    D_i    = sum_j P_ij dP_ij = dO_i . O_i
    dS_ij  = P_ij (dP_ij - D_i)           gradient of the loss w.r.t. s_ij
    dQ_i   = scale * sum_j dS_ij k_j
    dK_j   = scale * sum_i dS_ij q_i

The masks are the forward's (oracle.exact.visible): causal, sliding window,
packed documents; a hidden key has s_ij = -inf, so P_ij = 0 and it gets no
gradient from that query.

The score modifications are the forward's too (oracle.exact.modify_scores:
soft-capping t = C tanh(s / C), then the ALiBi bias u = t - a_h |i - j|), and P
is built from the modified score u.  The softmax gives the gradient w.r.t. u,
dU = P (dP - D); the bias does not depend on q or k, and the chain rule through
the cap multiplies by dt/ds = 1 - tanh(s / C)^2:

    dS_ij  = dU_ij (1 - tanh(s_ij / C)^2)     (dS = dU without soft-capping)

With grouped-query attention the key/value head hk serves query heads
hk*g .. hk*g + g - 1 (g = Hq / Hkv), so dK and dV of hk are the sums of those
query heads' contributions.  A row whose keys are all masked contributes
nothing.  Inputs: float64 q [B, Hq, N, d], k, v [B, Hkv, N, d], dO like q; O
and LSE are the forward's (recomputed here from the definition unless given).
"""

import numpy as np

from .exact import apply_mask, attention, modify_scores, scores, visible


def backward_head(q, k, v, do, causal, scale, o=None, lse=None, window=0, docs=None,
                  softcap=0.0, alibi_slope=None):
    """Gradients for one (batch, query head) slice: q, do [N, d]; k, v [Nk, d].

    Returns (dq [N, d], dk [Nk, d], dv [Nk, d]) of that query head alone.
    """
    n = q.shape[0]
    rows = np.arange(n)
    raw = scores(q, k, scale)
    s = apply_mask(modify_scores(raw, rows, softcap, alibi_slope), rows, causal, window, docs)
    if lse is None or o is None:
        m = s.max(axis=1)
        m_safe = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m_safe[:, None])
        l = e.sum(axis=1)
        live = l > 0
        lse = np.where(live, m_safe + np.log(np.where(live, l, 1.0)), -np.inf)
        o = np.where(live[:, None], (e @ v) / np.where(live, l, 1.0)[:, None], 0.0)
    live = np.isfinite(lse)
    p = np.where(live[:, None], np.exp(s - np.where(live, lse, 0.0)[:, None]), 0.0)
    dv = p.T @ do
    dp = do @ v.T
    delta = np.sum(do * o, axis=1)
    ds = p * (dp - delta[:, None])
    if softcap:
        ds = ds * (1.0 - np.tanh(raw / softcap) ** 2)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, causal, scale, o=None, lse=None, window=0, docs=None,
                       softcap=0.0, alibi=None):
    """Gradients over [B, H, N, d] operands: returns (dq, dk, dv) in float64.

    o and lse, when given, are the forward's outputs [B, Hq, N, d] and [B, Hq, N];
    otherwise they are recomputed from the definition (with the same masks and
    modifications).  alibi: Hq slopes or None; softcap: C (0 = off).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if o is None or lse is None:
        o, lse = attention(q, k, v, causal, scale, window=window, docs=docs, softcap=softcap,
                           alibi=alibi)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            gq, gk, gv = backward_head(q[b, h], k[b, hk], v[b, hk], do[b, h], causal, scale,
                                       o[b, h], lse[b, h], window, docs, softcap,
                                       None if alibi is None else float(alibi[h]))
            dq[b, h] = gq
            dk[b, hk] += gk
            dv[b, hk] += gv
    return dq, dk, dv


def delta(o, do):
    """D_i = dO_i . O_i per row: [B, Hq, N].  Equal to sum_j P_ij dP_ij, because
    O_i = sum_j P_ij v_j and dP_ij = dO_i . v_j."""
    return np.sum(np.asarray(o, dtype=np.float64) * np.asarray(do, dtype=np.float64), axis=-1)


def backward_rows(q, k, v, do, causal, scale, o, lse, qrows, krows, window=0, docs=None,
                  softcap=0.0, alibi_slope=None):
    """The same gradients as backward_head, for listed rows only, at sizes where the N x N
    matrices do not fit: dQ of the query rows `qrows` and dK, dV of the key rows `krows`,
    for one (batch, query head) slice.  q, do [N, d]; k, v [Nk, d]; o [N, d] and lse [N]
    are the forward's outputs for every query row of the slice (D_i and P_ij need them).

    dQ_i needs row i of P and dP (all keys); dK_j and dV_j need column j of P and dP (all
    queries), so only those rows and columns of the score matrix are formed.  Returns
    (dq [len(qrows), d], dk [len(krows), d], dv [len(krows), d])."""
    qrows = np.asarray(qrows, dtype=np.int64)
    krows = np.asarray(krows, dtype=np.int64)
    n, nk = q.shape[0], k.shape[0]
    all_rows = np.arange(n)
    live = np.isfinite(lse)
    lse0 = np.where(live, lse, 0.0)
    dlt = np.sum(do * o, axis=1)                 # D_i for every query row

    def masked(raw, rows, cols):
        s = modify_scores(raw, rows, softcap, None)
        if alibi_slope is not None:
            s = s - alibi_slope * np.abs(rows[:, None] - cols[None, :])
        if not causal and not window and docs is None:
            return s
        return np.where(visible(rows, nk, causal, window, docs)[:, cols], s, -np.inf)

    # rows of the score matrix: dQ
    raw_r = scale * (q[qrows] @ k.T)
    cols_all = np.arange(nk)
    p_r = np.where(live[qrows, None],
                   np.exp(masked(raw_r, qrows, cols_all) - lse0[qrows, None]), 0.0)
    ds_r = p_r * (do[qrows] @ v.T - dlt[qrows, None])
    if softcap:
        ds_r = ds_r * (1.0 - np.tanh(raw_r / softcap) ** 2)
    dq = scale * (ds_r @ k)
    # columns of the score matrix: dK, dV
    raw_c = scale * (q @ k[krows].T)
    p_c = np.where(live[:, None],
                   np.exp(masked(raw_c, all_rows, krows) - lse0[:, None]), 0.0)
    dv = p_c.T @ do
    ds_c = p_c * (do @ v[krows].T - dlt[:, None])
    if softcap:
        ds_c = ds_c * (1.0 - np.tanh(raw_c / softcap) ** 2)
    dk = scale * (ds_c.T @ q)
    return dq, dk, dv

"""Skip-ratio model of the thresholded rescale: a diagnostic, not part of the parity
definition (the attention output does not depend on tau in exact arithmetic).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages give.  The online softmax moves its running maximum, and rescales the
output accumulator, only when the maximum changes by enough; the aigc.bar page
("FlashAttention-4发布…", section "FlashAttention-4：为Blackwell而生的性能猛兽", item 1)
says this skips up to 90 % of the rescales.  No threshold or grouping is printed.

The rule modelled (the reading the kernels take): rows go through the keys in groups of
`rows` consecutive query rows (one wavefront of the kernel) and tiles of `keys` keys.
For each group and each tile it visits, in log2 units t_ij = scale * q_i . k_j * log2(e):

    M_i   = max of t_ij over the tile's keys visible to row i   (-inf if none)
    fire  = any row i of the group has M_i > m_i + tau
    m_i   = max(m_i, M_i) for every row of the group when it fires, else unchanged

with m_i = -inf before the first tile.  A group visits the tiles holding at least one key
visible to one of its rows (causal: tiles starting at or below its last row).  The first
visited tile always fires and is not counted; the skip ratio is 1 - (fires after the first
tile) / (tiles visited after the first), summed over groups.  Rows past N (a ragged last
group) repeat row N - 1, as the kernel's clamped row loads do.

With integer_ref (the block-scaled forwards' rule, "Hardware-Aware FP4 FlashAttention-4",
section "1. Direct-P para Inferencia Directa": the reference the weights are taken against
is an integer), a firing group sets m_i = max(m_i, ceil(M_i)) instead.

Only the non-causal and causal masks are modelled.  Scores are float64 here and fp32 in
the kernel, so a decision can differ where M_i - m_i sits within rounding of tau.
"""

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


def tile_maxima(q, k, scale, causal, rows=32, keys=64, chunk=256):
    """M [n_groups * rows, n_tiles]: per-row maxima of t over each tile's visible keys
    (rows past N repeat row N - 1).  q [N, d], k [N, d] float64."""
    n = q.shape[0]
    n_groups = -(-n // rows)
    n_tiles = -(-k.shape[0] // keys)
    row_ids = np.minimum(np.arange(n_groups * rows), n - 1)
    out = np.empty((n_groups * rows, n_tiles))
    for r0 in range(0, n_groups * rows, chunk):
        ids = row_ids[r0:r0 + chunk]
        t = (scale * LOG2E) * (q[ids] @ k.T)
        if causal:
            t = np.where(np.arange(k.shape[0])[None, :] <= ids[:, None], t, -np.inf)
        pad = n_tiles * keys - k.shape[0]
        if pad:
            t = np.concatenate([t, np.full((t.shape[0], pad), -np.inf)], axis=1)
        out[r0:r0 + len(ids)] = t.reshape(len(ids), n_tiles, keys).max(axis=2)
    return out


def count_rescales(m_tiles, n, tau, causal, rows=32, keys=64, integer_ref=False):
    """(steps, fires) for the rule above, from tile_maxima's output."""
    n_groups = m_tiles.shape[0] // rows
    n_tiles = m_tiles.shape[1]
    mt = m_tiles.reshape(n_groups, rows, n_tiles)
    # tiles a group visits: [0, last) with last = tiles up to its last real row (causal)
    if causal:
        last_row = np.minimum((np.arange(n_groups) + 1) * rows, n) - 1
        visits = np.minimum(last_row // keys + 1, n_tiles)
    else:
        visits = np.full(n_groups, n_tiles)
    m = np.full((n_groups, rows), -np.inf)
    steps = fires = 0
    for j in range(n_tiles):
        live = visits > j
        if not live.any():
            break
        tile = mt[:, :, j]
        fire = np.any(tile > m + tau, axis=1) & live
        up = np.ceil(tile) if integer_ref else tile
        m = np.where(fire[:, None], np.maximum(m, up), m)
        if j > 0:
            steps += int(live.sum())
            fires += int(fire.sum())
    return steps, fires


def skip_counts(q, k, scale, tau, causal, rows=32, keys=64, integer_ref=False):
    """(steps, fires) of one head: q [N, d], k [N, d] float64."""
    return count_rescales(tile_maxima(q, k, scale, causal, rows, keys), q.shape[0], tau,
                          causal, rows, keys, integer_ref)


def skip_counts_brute(q, k, scale, tau, causal, rows=32, keys=64, integer_ref=False):
    """The same rule as scalar Python loops (tiny inputs only)."""
    n, nk = q.shape[0], k.shape[0]
    steps = fires = 0
    for g0 in range(0, n, rows):
        ids = [min(i, n - 1) for i in range(g0, g0 + rows)]
        m = [-math.inf] * rows
        first = True
        for t0 in range(0, nk, keys):
            if causal and t0 > min(g0 + rows, n) - 1:
                break
            tile_m = []
            for i in ids:
                best = -math.inf
                for j in range(t0, min(t0 + keys, nk)):
                    if causal and j > i:
                        continue
                    s = scale * sum(float(a) * float(b) for a, b in zip(q[i], k[j])) * LOG2E
                    best = max(best, s)
                tile_m.append(best)
            fire = any(tile_m[r] > m[r] + tau for r in range(rows))
            if fire:
                m = [max(m[r], math.ceil(tile_m[r]) if integer_ref and tile_m[r] > -math.inf
                         else tile_m[r]) for r in range(rows)]
            if not first:
                steps += 1
                fires += int(fire)
            first = False
    return steps, fires

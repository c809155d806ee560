"""The skip-ratio model (oracle.skipsim) against scalar loops and closed forms."""

import numpy as np
import pytest

from oracle import skipsim


def _qk(seed, n, d, sigma):
    rng = np.random.default_rng(seed)
    return sigma * rng.standard_normal((n, d)), sigma * rng.standard_normal((n, d))


@pytest.mark.parametrize("n,causal,tau", [(70, False, 0.0), (70, True, 0.0), (96, False, 1.0),
                                          (130, True, 2.0), (33, True, 0.5)])
@pytest.mark.parametrize("integer_ref", [False, True])
def test_matches_scalar_loops(n, causal, tau, integer_ref):
    q, k = _qk(n, n, 4, 2.0)
    got = skipsim.skip_counts(q, k, 0.7, tau, causal, rows=8, keys=16, integer_ref=integer_ref)
    assert got == skipsim.skip_counts_brute(q, k, 0.7, tau, causal, rows=8, keys=16,
                                            integer_ref=integer_ref)


def test_integer_reference_fires_less_or_equal():
    """Raising the reference to the ceiling of the tile maximum leaves more headroom, so the
    integer rule never fires more often than the plain one on the same scores."""
    q, k = _qk(4, 700, 8, 3.0)
    for tau in (0.0, 2.0, 8.0):
        plain = skipsim.skip_counts(q, k, 0.3, tau, False)[1]
        integer = skipsim.skip_counts(q, k, 0.3, tau, False, integer_ref=True)[1]
        assert integer <= plain


def test_step_count_closed_form():
    """Non-causal: every group visits every tile; causal: group g visits
    ceil(last row + 1 / keys) tiles."""
    q, k = _qk(1, 256, 4, 1.0)
    steps, _ = skipsim.skip_counts(q, k, 0.5, 8.0, False, rows=32, keys=64)
    assert steps == (256 // 32) * (256 // 64 - 1)
    steps, _ = skipsim.skip_counts(q, k, 0.5, 8.0, True, rows=32, keys=64)
    assert steps == sum(((g + 1) * 32 - 1) // 64 for g in range(8))


def test_monotone_scores():
    """Keys whose scores rise along the sequence move the maximum on every tile (tau = 0:
    every step fires); falling scores never move it after the first tile."""
    n = 128
    q = np.ones((n, 1))
    k_up = np.arange(n, dtype=np.float64)[:, None]
    steps, fires = skipsim.skip_counts(q, k_up, 1.0, 0.0, False, rows=32, keys=16)
    assert fires == steps > 0
    steps, fires = skipsim.skip_counts(q, -k_up, 1.0, 0.0, False, rows=32, keys=16)
    assert fires == 0 and steps > 0
    # a threshold above the total rise never fires
    steps, fires = skipsim.skip_counts(q, k_up, 1.0, 1000.0, False, rows=32, keys=16)
    assert fires == 0


def test_larger_tau_skips_more():
    q, k = _qk(3, 512, 16, 3.0)
    f = [skipsim.skip_counts(q, k, 0.25, tau, False)[1] for tau in (0.0, 2.0, 8.0)]
    assert f[0] >= f[1] >= f[2]

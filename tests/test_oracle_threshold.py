"""Pins of the threshold-acceptance oracle ("Accélérer Sonar par la Spéculation", section
"Décodage spéculatif": the longest candidate prefix whose probability is above a threshold is
kept, and the target gives one more token).

The pins do not re-type the oracle's running log-score. They check it against:
  * the limits tau = 0 (every prefix kept: AL = L + 1, the extra token a plain draw from p_L)
    and tau >= 1 (no prefix kept: AL = 1, the extra token a plain draw from p_0), with the draw
    computed by numpy.searchsorted over scipy's softmax;
  * brute force on small cases: the score of every prefix as a product of scipy softmax
    probabilities, the longest prefix above tau found by enumerating all prefix lengths;
  * monotonicity in tau and the greedy rows of the standard oracle.
"""
import numpy as np
import pytest
import scipy.special

from oracle import verify, verify_threshold, verify_threshold_workload, verify_workload
from workloads import make


def _plain_draw(row, T, u):
    p = scipy.special.softmax(row.astype(np.float64) / T)
    return int(np.searchsorted(np.cumsum(p), u * p.sum(), side="right"))


@pytest.mark.parametrize("cfg,kw", [("c3", dict(B=24, V=3000)), ("c5", dict(B=32, V=2000))])
def test_threshold_zero_keeps_every_prefix(cfg, kw):
    w = make(cfg, 1, **kw)
    r = verify_threshold_workload(w, 0.0)
    t = w.target_f32()
    for b in range(w.B):
        L = w.lens[b]
        assert r.accept_len[b] == L + 1
        assert np.array_equal(r.tokens[b, :L], w.tokens[b, :L])
        if not r.flagged[b]:
            assert r.tokens[b, L] == _plain_draw(t[b, L], w.temperature[b], w.uniforms[b, w.D])


@pytest.mark.parametrize("tau", [1.0, 3.0])
def test_threshold_one_keeps_nothing(tau):
    w = make("c3", 2, B=24, V=3000)
    r = verify_threshold_workload(w, tau)
    t = w.target_f32()
    assert np.all(r.accept_len == 1)
    for b in range(w.B):
        if not r.flagged[b]:
            assert r.tokens[b, 0] == _plain_draw(t[b, 0], w.temperature[b], w.uniforms[b, w.D])


@pytest.mark.parametrize("tau", [0.3, 0.05, 1e-3])
def test_brute_force_longest_prefix(tau):
    rng = np.random.default_rng(int(1 / tau))
    B, D, V = 300, 4, 6
    tgt = (rng.standard_normal((B, D + 1, V)) * 1.5).astype(np.float32)
    toks = rng.integers(0, V, (B, D)).astype(np.int32)
    lens = rng.integers(0, D + 1, B).astype(np.int32)
    u = rng.random((B, D + 1), dtype=np.float32)
    T = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), B)
    r = verify_threshold(tgt, toks, lens, u, T, tau)
    checked = 0
    for b in range(B):
        if r.flagged[b]:
            continue
        L = lens[b]
        p = [scipy.special.softmax(tgt[b, i].astype(np.float64) / T[b]) for i in range(D + 1)]
        scores = [np.prod([p[i][toks[b, i]] for i in range(k)]) for k in range(L + 1)]
        kept = max(k for k in range(L + 1) if k == 0 or scores[k] > tau)
        assert r.accept_len[b] == kept + 1
        assert r.tokens[b, kept] == _plain_draw(tgt[b, kept], T[b], u[b, D])
        checked += 1
    assert checked > 0.95 * B


def test_accept_length_falls_as_tau_rises():
    w = make("c5", 3, B=48, V=2000)
    prev = None
    for tau in (0.0, 1e-6, 1e-3, 0.02, 0.2, 0.9, 1.0):
        al = verify_threshold_workload(w, tau).accept_len
        if prev is not None:
            assert np.all(al <= prev)
        prev = al
    assert np.all(prev == 1)


def test_greedy_rows_follow_the_standard_rule():
    w = make("c4", 4, B=40, V=3000)
    g = w.temperature == 0
    ref = verify_workload(w)
    for tau in (0.0, 0.01, 0.5):
        r = verify_threshold_workload(w, tau)
        assert np.array_equal(r.accept_len[g], ref.accept_len[g])
        assert np.array_equal(r.tokens[g], ref.tokens[g])


def test_invalid_rows_are_marked():
    w = make("c3", 5, B=6, V=500)
    w.tokens[0, 1] = w.V
    w.temperature[1] = -1.0
    r = verify_threshold_workload(w, 0.01)
    assert r.accept_len[0] == 0 and r.accept_len[1] == 0
    assert np.all(r.tokens[:2] == -1) and np.all(r.accept_len[2:] >= 1)


def test_flag_rate_estimator_is_small_on_full_headline_config():
    """The expected number of flagged decisions of threshold acceptance (prefix tests through
    the draft tokens' distribution, plus the final draw) is below 1e-4 per row at full size."""
    from workloads import make
    for tau in (1e-3, 0.05):
        w = make("c3", 0)
        r = verify_threshold_workload(w, tau)
        assert r.flag_measure.mean() < 1e-4, (tau, r.flag_measure.mean())

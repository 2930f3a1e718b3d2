"""Accuracy and brute-force pins of the oracle's arithmetic.

  * mpmath at 50 digits recomputes p(x), q(x), the ratio and the inverse-CDF bins on tiny
    vocabularies: the oracle's fp64 values agree to 1e-12, and every decision the oracle does
    not flag agrees with the 50-digit decision.
  * Brute force: sweeping the final uniform over a fine grid, the drawn token is monotone in u
    and each token's share of [0, 1) equals its normalised weight (bonus draw from p, and
    residual draw max(0, p - q) after a forced rejection); zero-weight tokens never appear.
"""
import mpmath
import numpy as np
import pytest
import scipy.special

from oracle import verify

mpmath.mp.dps = 50


def _mp_softmax(row, T):
    z = [mpmath.mpf(float(v)) / mpmath.mpf(float(T)) for v in row]
    m = max(z)
    e = [mpmath.e ** (zi - m) for zi in z]
    s = mpmath.fsum(e)
    return [ei / s for ei in e]


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_fp64_agrees_with_50_digit_arithmetic(T):
    rng = np.random.default_rng(21)
    B, D, V = 60, 2, 6
    tgt = (rng.standard_normal((B, D + 1, V)) * 4).astype(np.float32)
    drf = (tgt[:, :D] + rng.standard_normal((B, D, V)) * 1.5).astype(np.float32)
    toks = rng.integers(0, V, (B, D)).astype(np.int32)
    u = rng.random((B, D + 1), dtype=np.float32)
    temp = np.full(B, T, np.float32)
    r = verify(tgt, drf, toks, None, u, temp)
    T = float(temp[0])                           # the float32 temperature the call receives
    for b in range(B):
        al_mp = None
        out = []
        for i in range(D):
            p = _mp_softmax(tgt[b, i], T)
            q = _mp_softmax(drf[b, i], T)
            x = int(toks[b, i])
            assert abs(float(mpmath.log(p[x])) - r.logp_x[b, i]) < 1e-12 * max(1, abs(r.logp_x[b, i]))
            assert abs(float(mpmath.log(q[x])) - r.logq_x[b, i]) < 1e-12 * max(1, abs(r.logq_x[b, i]))
            ratio = p[x] / q[x]
            if mpmath.mpf(float(u[b, i])) < min(mpmath.mpf(1), ratio):
                out.append(x)
                continue
            w = [max(mpmath.mpf(0), pi - qi) for pi, qi in zip(p, q)]
            al_mp = i + 1
            break
        if al_mp is None:
            w = _mp_softmax(tgt[b, D], T)
            al_mp = D + 1
        Z = mpmath.fsum(w)
        t = mpmath.mpf(float(u[b, D])) * Z
        F = mpmath.mpf(0)
        for k, wk in enumerate(w):
            F += wk
            if F > t:
                break
        out.append(k)
        if not r.flagged[b]:
            assert r.accept_len[b] == al_mp
            assert list(r.tokens[b, :al_mp]) == out


def _sweep_final(tgt, drf, toks, lens, uacc, T, n=20001):
    grid = (np.arange(n, dtype=np.float64) / n).astype(np.float32)
    B = n
    target = np.broadcast_to(tgt, (B,) + tgt.shape)
    draft = np.broadcast_to(drf, (B,) + drf.shape)
    u = np.empty((B, tgt.shape[0]), np.float32)
    u[:, :-1] = uacc
    u[:, -1] = grid
    r = verify(target, draft, np.broadcast_to(toks, (B,) + toks.shape),
               np.full(B, lens, np.int32), u, np.full(B, T, np.float32))
    return grid, r


def test_bonus_draw_brute_force_bins():
    rng = np.random.default_rng(5)
    V, T = 8, 0.9
    tgt = (rng.standard_normal((1, V)) * 2).astype(np.float32)
    grid, r = _sweep_final(tgt, np.zeros((0, V), np.float32), np.zeros(0, np.int32), 0,
                           np.zeros(0, np.float32), T)
    tok = r.tokens[:, 0]
    assert np.all(np.diff(tok) >= 0)
    p = scipy.special.softmax(tgt[0].astype(np.float64) / T)
    share = np.bincount(tok, minlength=V) / len(grid)
    assert np.allclose(share, p, atol=2.0 / len(grid))


def test_residual_draw_brute_force_bins():
    rng = np.random.default_rng(8)
    V, T = 8, 1.0
    tgt = (rng.standard_normal((2, V)) * 2).astype(np.float32)
    drf = (tgt[:1] + rng.standard_normal((1, V)) * 1.5).astype(np.float32)
    p = scipy.special.softmax(tgt[0].astype(np.float64) / T)
    q = scipy.special.softmax(drf[0].astype(np.float64) / T)
    x = int(np.argmax(q / p))                    # ratio p/q < 1 here, so u close to 1 rejects
    assert p[x] / q[x] < 0.999
    grid, r = _sweep_final(tgt, drf, np.array([x], np.int32), 1,
                           np.array([0.9999], np.float32), T)
    assert np.all(r.accept_len == 1) and np.all(r.final_mode == 2)
    tok = r.tokens[:, 0]
    assert np.all(np.diff(tok) >= 0)
    res = np.maximum(p - q, 0)
    res /= res.sum()
    share = np.bincount(tok, minlength=V) / len(grid)
    assert np.all(share[res == 0] == 0)
    assert np.allclose(share, res, atol=2.0 / len(grid))

"""Statistical pins of the fp64 oracle.

  * Lossless: each emitted token is distributed as the target alone would sample it
    ("Speculative Speculative Decoding", the remark after the three-step rule; "NVIDIA: öt
    irányelv ...", section "Mit csinál a spekulatív dekódolás?"). Here the synthetic p_j do not
    depend on earlier tokens, so the token at position j, given that position j is emitted,
    must follow p_j. V=8, D=2, 10^6 draws, chi-square per position.
  * Residual: given a rejection at position 0 the emitted token follows
    norm(max(0, p_0 - q_0)) (step 3 of the same rule).
  * Acceptance length: with x_i ~ q_i, position i accepts with probability
    alpha_i = sum_x min(p_i(x), q_i(x)), so P(AL = k) = prod_{i<k-1} alpha_i * (1 - alpha_{k-1})
    and P(AL = L + 1) = prod_i alpha_i (derived from the rule, not printed on the pages).
  * Negative controls: the rule exactly as the extracted text prints it ("otherwise reject with
    probability p/q") and resampling from p instead of the residual must both fail.
"""
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle import oracle as oracle_mod

V, D = 8, 2
N_DRAWS = 1_000_000


def _dists(seed=123):
    rng = np.random.default_rng(seed)
    tgt = (rng.standard_normal((D + 1, V)) * 1.3).astype(np.float32)
    drf = (tgt[:D] + rng.standard_normal((D, V)) * 1.1).astype(np.float32)
    return tgt, drf


def _batch(n, seed, tgt, drf, T=1.0):
    rng = np.random.default_rng(seed)
    q = scipy.special.softmax(drf.astype(np.float64) / T, axis=-1)
    toks = np.stack([rng.choice(V, size=n, p=q[i]) for i in range(D)], axis=1).astype(np.int32)
    u = rng.random((n, D + 1), dtype=np.float32)
    target = np.broadcast_to(tgt, (n, D + 1, V))
    draft = np.broadcast_to(drf, (n, D, V))
    return target, draft, toks, u, np.full(n, T, np.float32)


def _run_chunk(args):
    n, seed, variant = args
    tgt, drf = _dists()
    if variant == "literal_reject":
        # "otherwise reject with probability p/q": keep the draft with probability 1 - p/q
        oracle_mod.accepts = lambda u, r: (r >= 1.0) or (u < 1.0 - r)
    elif variant == "resample_from_p":
        oracle_mod.residual_weights = lambda p, q: p
    target, draft, toks, u, temp = _batch(n, seed, tgt, drf)
    res = oracle.verify(target, draft, toks, None, u, temp)
    return res.accept_len, res.tokens


def _draw(total, variant=None, workers=8):
    chunk = (total + workers - 1) // workers
    jobs = [(min(chunk, total - i * chunk), 1000 + i, variant) for i in range(workers)]
    with ProcessPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(_run_chunk, jobs))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _per_position_pvalues(al, toks, tgt, T=1.0):
    p = scipy.special.softmax(tgt.astype(np.float64) / T, axis=-1)
    pv = []
    for j in range(D + 1):
        sel = al > j
        counts = np.bincount(toks[sel, j], minlength=V)
        pv.append(scipy.stats.chisquare(counts, sel.sum() * p[j]).pvalue)
    return pv


@pytest.fixture(scope="module")
def draws():
    return _draw(N_DRAWS)


def test_lossless_chi_square(draws):
    al, toks = draws
    tgt, _ = _dists()
    pv = _per_position_pvalues(al, toks, tgt)
    assert min(pv) > 1e-3, pv


def test_acceptance_length_histogram_closed_form(draws):
    al, _ = draws
    tgt, drf = _dists()
    p = scipy.special.softmax(tgt.astype(np.float64), axis=-1)
    q = scipy.special.softmax(drf.astype(np.float64), axis=-1)
    alpha = np.minimum(p[:D], q).sum(axis=1)
    probs = [1 - alpha[0], alpha[0] * (1 - alpha[1]), alpha[0] * alpha[1]]
    counts = np.bincount(al, minlength=D + 2)[1:]
    assert scipy.stats.chisquare(counts, len(al) * np.array(probs)).pvalue > 1e-3


def test_residual_after_rejection_at_first_position(draws):
    al, toks = draws
    tgt, drf = _dists()
    p = scipy.special.softmax(tgt.astype(np.float64), axis=-1)
    q = scipy.special.softmax(drf.astype(np.float64), axis=-1)
    res = np.maximum(p[0] - q[0], 0)
    res /= res.sum()
    sel = al == 1
    counts = np.bincount(toks[sel, 0], minlength=V)
    nz = res > 0
    assert np.all(counts[~nz] == 0)
    assert scipy.stats.chisquare(counts[nz], sel.sum() * res[nz]).pvalue > 1e-3


@pytest.mark.parametrize("variant", ["literal_reject", "resample_from_p"])
def test_negative_controls_fail(variant):
    al, toks = _draw(200_000, variant=variant)
    tgt, _ = _dists()
    pv = _per_position_pvalues(al, toks, tgt)
    assert min(pv) < 1e-6, pv

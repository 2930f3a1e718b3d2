"""Pins of the Saguaro reshaping oracle ("Speculative Speculative Decoding - асинхронизируй
это", saguaro sampling: the draft's top-5 tokens get lower probabilities when the draft is
generated, so that the residual concentrates on them).

  * c = 1 changes nothing.
  * The reshaped tokens are the top k by brute force (Python's sorted, ties to the lowest index).
  * In probability space the reshaped row is q with its top k scaled by c and renormalised
    (scipy's softmax), the definition restated.
  * Losslessness: drafts sampled from the reshaped q' and verified against the reshaped logits
    emit tokens distributed as p (chi-square, V=8, D=2); verified against the original logits
    instead, they do not (negative control).
  * The residual mass max(0, p - q') on the top k is at least that of max(0, p - q).
"""
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle.saguaro import reshape_draft, top_k_indices
from workloads import make


def test_factor_one_changes_nothing():
    for cfg, kw in (("c3", dict(B=6, V=3000)), ("c2", dict(B=4, V=2000))):
        w = make(cfg, 1, **kw)
        r = reshape_draft(w.draft, w.dtype, w.lens, w.temperature, 1.0)
        assert np.array_equal(r.view(np.uint8), w.draft.view(np.uint8))


def test_top_k_is_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for _ in range(200):
        row = rng.integers(-3, 4, rng.integers(1, 40)).astype(np.float32)   # many ties
        k = int(rng.integers(1, 9))
        want = [i for _, i in sorted((-float(v), i) for i, v in enumerate(row))][:k]
        assert top_k_indices(row, k).tolist() == want


@pytest.mark.parametrize("factor,k", [(0.5, 5), (0.05, 3), (0.9, 16)])
def test_reshaped_row_is_scaled_and_renormalised_q(factor, k):
    rng = np.random.default_rng(3)
    B, D, V = 5, 3, 200
    draft = (rng.standard_normal((B, D, V)) * 2).astype(np.float32)
    T = np.array([1.0, 0.7, 2.0, 0.3, 1.5], np.float32)
    lens = np.array([3, 2, 0, 3, 1], np.int32)
    r = reshape_draft(draft, "f32", lens, T, factor, k)
    for b in range(B):
        for i in range(D):
            q = scipy.special.softmax(draft[b, i].astype(np.float64) / T[b])
            if i >= lens[b]:
                assert np.array_equal(r[b, i], draft[b, i])
                continue
            top = np.argsort(-q, kind="stable")[:k]
            want = q.copy()
            want[top] *= factor
            want /= want.sum()
            got = scipy.special.softmax(r[b, i].astype(np.float64) / T[b])
            assert np.allclose(got, want, rtol=2e-6, atol=1e-12)
            changed = np.nonzero(r[b, i] != draft[b, i])[0]
            assert set(changed.tolist()) <= set(top.tolist())


def test_greedy_and_invalid_sequences_are_untouched():
    w = make("c4", 2, B=30, V=500)
    w.lens[3] = w.D + 2
    r = reshape_draft(w.draft, w.dtype, w.lens, w.temperature, 0.3)
    for b in range(w.B):
        if w.temperature[b] == 0 or b == 3:
            assert np.array_equal(r[b], w.draft[b])


V, D, N = 8, 2, 600_000
FACTOR = 0.2


def _chunk(args):
    n, seed, against_original = args
    rng = np.random.default_rng(seed)
    r0 = np.random.default_rng(7)
    tgt = (r0.standard_normal((D + 1, V)) * 1.3).astype(np.float32)
    drf = (tgt[:D] + r0.standard_normal((D, V)) * 0.6).astype(np.float32)
    shaped = reshape_draft(drf[None], "f32", None, np.ones(1, np.float32), FACTOR)[0]
    q = scipy.special.softmax(shaped.astype(np.float64), axis=-1)
    toks = np.stack([rng.choice(V, size=n, p=q[i]) for i in range(D)], axis=1).astype(np.int32)
    u = rng.random((n, D + 1), dtype=np.float32)
    used = drf if against_original else shaped
    res = oracle.verify(np.broadcast_to(tgt, (n, D + 1, V)), np.broadcast_to(used, (n, D, V)),
                        toks, None, u, np.ones(n, np.float32))
    return res.accept_len, res.tokens, tgt


def _pvalues(against_original):
    jobs = [(N // 8, 500 + i, against_original) for i in range(8)]
    with ProcessPoolExecutor(max_workers=8) as ex:
        parts = list(ex.map(_chunk, jobs))
    al = np.concatenate([p[0] for p in parts])
    toks = np.concatenate([p[1] for p in parts])
    p = scipy.special.softmax(parts[0][2].astype(np.float64), axis=-1)
    pv = []
    for j in range(D + 1):
        sel = al > j
        counts = np.bincount(toks[sel, j], minlength=V)
        pv.append(scipy.stats.chisquare(counts, sel.sum() * p[j]).pvalue)
    return pv


def test_reshaped_drafts_stay_lossless():
    assert min(_pvalues(False)) > 1e-3


def test_verifying_against_the_unreshaped_draft_is_not_lossless():
    assert min(_pvalues(True)) < 1e-6


def test_residual_concentrates_on_the_top_k():
    rng = np.random.default_rng(4)
    for _ in range(50):
        t = rng.standard_normal(300) * 2
        d = (t + rng.standard_normal(300)).astype(np.float32)
        p = scipy.special.softmax(t)
        q = scipy.special.softmax(d.astype(np.float64))
        shaped = reshape_draft(d[None, None], "f32", None, np.ones(1, np.float32), 0.3)[0, 0]
        q2 = scipy.special.softmax(shaped.astype(np.float64))
        top = top_k_indices(d, 5)
        assert np.maximum(0, p - q2)[top].sum() >= np.maximum(0, p - q)[top].sum() - 1e-12

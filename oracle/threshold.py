"""Plain fp64 CPU oracle of threshold (relaxed) acceptance.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs this file: only
the tests and the benchmark's CPU-baseline leg use it. It shares no code with the HIP library.

Source: "Accélérer Sonar par la Spéculation" (Perplexity), section "Décodage spéculatif": every
prefix of the draft candidates is scored with a probability and the longest one above an
acceptance threshold is kept; the target then gives one more token for free, sampled from its
logits at the first position not kept ("Génération cible": the logits at the mismatched position
or at the end of the tail are sampled).

Readings adopted (the page gives neither the score nor the threshold):
  * The score of the prefix x_0..x_{k-1} is the probability the target gives it,
    prod_{i<k} p_i(x_i), with p_i = softmax(target_i / T). The draft distribution is not used.
  * A prefix is kept while its score is strictly above tau. Scores only fall as the prefix grows
    (each factor is at most 1), so the longest prefix above tau ends just before the first
    prefix whose score is at most tau: with j that first position (or L if none), AL = j + 1.
  * The extra token is drawn from p_j (plain target sample, no residual) by the same inverse CDF
    and final uniform u[b][D] as the standard rule.
  * T = 0: the score is 1 while the drafts equal the target argmax and 0 after, so for any tau in
    [0, 1) the rule is greedy argmax matching; greedy sequences follow it unchanged.
  * Flags: a prefix test is flagged when its log-score lies within 1e-5 * k of ln tau (k terms,
    each an fp32 log-probability on the GPU with error below 1e-5); the final draw is flagged as
    in the standard rule.
  * Window measure of a prefix test (the expected number of flags, as for the standard rule's
    accept tests): the draft token x_i is a draw from q_i = softmax(draft_i / T), independent of
    the earlier positions, so given the score s_{i-1} of the prefix before it, test i is flagged
    with probability sum_x q_i(x) [|s_{i-1} + log p_i(x) - ln tau| < 1e-5 (i+1)]. Summed over
    the tests performed it estimates the expected number of flagged tests (tower property). It
    needs the draft logits the tokens were drawn from; without them each flagged test counts 1.
"""
from __future__ import annotations

import math

import numpy as np

from .oracle import (FLAG_TOL, Result, final_window_measure, inverse_cdf, row_is_valid,
                     softmax, tempered_log_softmax)


def prefix_window_measure(lp: np.ndarray, q: np.ndarray, prev: float, log_tau: float,
                          win: float) -> float:
    """Probability that test i is flagged given the prefix score `prev` before it: the q-mass of
    the tokens x whose prefix score prev + lp[x] lies within `win` of ln tau."""
    return float(np.sum(q[np.abs(prev + lp - log_tau) < win]))


def verify_threshold(target: np.ndarray, tokens: np.ndarray, lens, uniforms: np.ndarray,
                     temperature: np.ndarray, tau: float, draft: np.ndarray | None = None) -> Result:
    """Threshold acceptance of a batch. target [B][D+1][V] (float32 values), tokens [B][D],
    lens [B] or None (all D), uniforms [B][D+1], temperature [B], tau >= 0. draft [B][D][V]
    (optional, never used by the rule): the logits the draft tokens were drawn from, for the
    window measure of the prefix tests."""
    B, D1, V = target.shape
    D = D1 - 1
    if lens is None:
        lens = np.full(B, D, dtype=np.int32)
    log_tau = math.log(tau) if tau > 0 else -math.inf
    nan = np.nan
    res = Result(
        accept_len=np.zeros(B, np.int32), tokens=np.full((B, D + 1), -1, np.int32),
        flagged=np.zeros(B, bool), flag_measure=np.zeros(B, np.float64),
        final_row=np.full(B, -1, np.int32), final_mode=np.zeros(B, np.int8),
        logp_x=np.full((B, D), nan), logq_x=np.full((B, D), nan),
        row_max_t=np.full((B, D + 1), nan), row_logsum_t=np.full((B, D + 1), nan),
        row_max_d=np.full((B, D), nan), row_logsum_d=np.full((B, D), nan),
        greedy_argmax=np.full((B, D + 1), -1, np.int64))
    for b in range(B):
        L = int(lens[b])
        T = float(temperature[b])
        if not row_is_valid(L, D, T, tokens[b], V):
            continue
        x = tokens[b]
        out = res.tokens[b]
        if T == 0.0:
            g = [int(np.argmax(target[b, i])) for i in range(L + 1)]
            res.greedy_argmax[b, :L + 1] = g
            j = 0
            while j < L and x[j] == g[j]:
                out[j] = x[j]
                j += 1
            out[j] = g[j]
            res.accept_len[b] = j + 1
            res.final_row[b] = j
            res.final_mode[b] = 1
            continue
        score = 0.0                       # log of the prefix's target probability
        j = L
        for i in range(L):
            lp, _, _ = tempered_log_softmax(target[b, i], T)
            res.logp_x[b, i] = lp[x[i]]
            win = FLAG_TOL * (i + 1)
            if draft is not None:
                res.flag_measure[b] += prefix_window_measure(lp, softmax(draft[b, i], T),
                                                             score, log_tau, win)
            score += lp[x[i]]
            if abs(score - log_tau) < win:
                res.flagged[b] = True
                if draft is None:
                    res.flag_measure[b] += 1.0
            if not score > log_tau:
                j = i
                break
            out[i] = x[i]
        w = softmax(target[b, j], T)
        k, fl, _, _, _ = inverse_cdf(w, float(uniforms[b, D]))
        out[j] = k
        res.flagged[b] |= fl
        res.flag_measure[b] += final_window_measure(w)
        res.accept_len[b] = j + 1
        res.final_row[b] = j
        res.final_mode[b] = 3
    return res


def verify_threshold_workload(w, tau: float) -> Result:
    """The workload's draft logits are passed for the window measure only."""
    return verify_threshold(w.target_f32(), w.tokens, w.lens if w.lens_given else None,
                            w.uniforms, w.temperature, tau, draft=w.draft_f32())

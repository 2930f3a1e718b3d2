"""Plain fp64 CPU oracle for the speculative-decoding verification sampler.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs this file: only
the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no code with
the HIP library and does not import it.

Sources (web pages, cited by title and section):
  [SSD]  "Speculative Speculative Decoding - асинхронизируй это" (x0ct.com), the recap of
         standard speculative decoding: the three-step accept / reject / residual rule and the
         lossless remark that follows it.
  [PPLX] "Accélérer Sonar par la Spéculation" (Perplexity), sections "Décodage spéculatif"
         (n drafts give up to n+1 tokens; the target's logits at the mismatch or at the end of
         the tail are sampled for one more token) and "Cible-Brouillon" (acceptance compares
         the full draft and target distributions; the draft takes the top token).
  [NV]   "NVIDIA: öt irányelv ... spekulatív dekódolás" (aihirek.info), section
         "Mit csinál a spekulatív dekódolás?" (tokens are accepted in order up to the first
         mismatch; AL lies in [1, 1 + D]; output equals conventional decoding).

What it computes, per sequence b with draft length L = L_b, temperature T = T_b, draft tokens
x_0..x_{L-1} and uniforms u[b][0..D]:

  * T == 0 (greedy): g_i = argmax of the raw target logits of position i (lowest index on ties).
    Draft token x_i is kept while x_i == g_i; at the first mismatch j the target's g_j is
    emitted and AL = j + 1; if all L match, g_L is emitted as the bonus and AL = L + 1.
  * T > 0 (sampled): p_i = softmax(target_i / T), q_i = softmax(draft_i / T) in fp64.
    Position i accepts x_i iff u[b][i] < min(1, p_i(x_i) / q_i(x_i)) ([SSD] rule, read as
    "accept with probability p/q"; the extracted text says "reject", which contradicts its
    own first step and the lossless claim). The scan stops at the first rejection j; the
    token emitted there is drawn from norm(max(0, p_j - q_j)) over the whole vocabulary. If
    all L drafts are accepted, the bonus token is drawn from p_L. Both draws use the single
    final uniform u_f = u[b][D] by inverse CDF in ascending token id: the smallest k with
    F_k > u_f * Z, F = cumulative sum of the weights, Z = F_{V-1}.
  * AL in [1, L + 1]; out_tokens[b][0..AL-2] are the accepted drafts, [AL-1] the final token,
    the rest -1. A row whose inputs are invalid (L outside [0, D], T negative / NaN /
    infinite, a draft token outside [0, V) at a position < L) gets AL = 0 and all tokens -1.

Boundary flags (decisions that rounding may legitimately flip): an accept test is flagged when
|u - r| < 1e-5 (r = p(x)/q(x), unclamped); a sampled final draw is flagged when t = u_f * Z lies
closer to either edge of the chosen token's bin [F_{k-1}, F_k) than max(1e-5 * w_k, ABS_WINDOW),
with the weights w in probability units (p, q and p - q normalised, Z <= 1).

The absolute part ABS_WINDOW = 1e-12 comes from an error bound, not from the data. Any fp64
evaluation of the weights carries a relative error of at most EVAL_REL = 1e-13 on each
probability (an fp64 exponential, its argument and the normalising division, at the
temperatures used). A residual weight max(0, p_v - q_v) is then off by at most
EVAL_REL * (p_v + q_v), so every prefix sum F_k and the total Z are off by at most
EVAL_REL * sum_v (p_v + q_v) = 2 * EVAL_REL = 2e-13 (bonus draws: EVAL_REL * F_k, less). Two
such evaluations (this oracle and any other) can disagree on t - F_{k-1} or F_k - t by twice
that, 4e-13; ABS_WINDOW keeps a factor 2.5 above it. A residual draw whose whole mass Z is below
ABS_WINDOW is therefore always flagged: its weights are differences of nearly equal
probabilities that the rounding decides. A residual of exactly zero mass (only possible through
rounding) falls back to a draw from p_j and is flagged too.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

FLAG_TOL = 1e-5
EVAL_REL = 1e-13       # relative error bound of an fp64 evaluation of one probability
ABS_WINDOW = 1e-12     # absolute final-draw window, probability units (module docstring)


@dataclasses.dataclass
class Result:
    accept_len: np.ndarray     # [B] int32
    tokens: np.ndarray         # [B][D+1] int32
    flagged: np.ndarray        # [B] bool: some decision of the row lies within the window
    flag_measure: np.ndarray   # [B] float64: expected number of flagged decisions given the
                               #   performed tests (window measure summed over them)
    final_row: np.ndarray      # [B] int32: position whose distribution the final token came from
    final_mode: np.ndarray     # [B] int8: 0 invalid, 1 greedy, 2 residual, 3 bonus
    logp_x: np.ndarray         # [B][D] float64: log p_i(x_i) (nan where not computed)
    logq_x: np.ndarray         # [B][D] float64: log q_i(x_i)
    row_max_t: np.ndarray      # [B][D+1] float64: max_v target/T  (nan where not computed)
    row_logsum_t: np.ndarray   # [B][D+1] float64: ln sum_v exp(target/T - max)
    row_max_d: np.ndarray      # [B][D]
    row_logsum_d: np.ndarray   # [B][D]
    greedy_argmax: np.ndarray  # [B][D+1] int64: target argmax per position (-1 if unused)


# --------------------------------------------------------------------------------------------
# building blocks, each a direct statement of one definition

def tempered_log_softmax(logits: np.ndarray, T: float):
    """log softmax(logits / T) in fp64. Returns (log-probabilities, max of z, ln of the sum)."""
    z = logits.astype(np.float64) / T
    m = np.max(z)
    log_s = math.log(np.sum(np.exp(z - m)))
    return z - m - log_s, m, log_s


def softmax(logits: np.ndarray, T: float) -> np.ndarray:
    """softmax(logits / T) in fp64, as exp(z - max z) / sum."""
    z = logits.astype(np.float64) / T
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def accepts(u: float, ratio: float) -> bool:
    """[SSD] step 1-2: keep the draft when q <= p; otherwise keep it with probability p/q.
    With a uniform u in [0, 1) both cases are the single test u < min(1, p/q)."""
    return u < min(1.0, ratio)


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """[SSD] step 3: unnormalised residual max(0, p - q) over the whole vocabulary."""
    return np.maximum(0.0, p - q)


def final_window(wk: float) -> float:
    """Half-width of the flagged window at each edge of a bin of weight wk (probability units):
    1e-5 of the bin, but never below the absolute rounding bound ABS_WINDOW."""
    return max(FLAG_TOL * wk, ABS_WINDOW)


def inverse_cdf(w: np.ndarray, u: float):
    """Draw a token from weights w >= 0 (probability units) with one uniform u in [0, 1): the
    smallest k with F_k > u * Z, where F is the running sum in ascending token id and Z = F[-1].
    If no k qualifies (only possible through rounding) the last token with positive weight is
    taken. Returns (token, flagged, F_{k-1}, F_k, Z)."""
    F = np.cumsum(w)
    Z = F[-1]
    t = u * Z
    hits = np.nonzero(F > t)[0]
    if hits.size:
        k = int(hits[0])
    else:
        k = int(np.nonzero(w > 0)[0][-1])
    lo = F[k - 1] if k > 0 else 0.0
    hi = F[k]
    win = final_window(float(w[k]))
    flagged = bool((t - lo) < win or (hi - t) < win)
    return k, flagged, lo, hi, Z


def final_window_measure(w: np.ndarray) -> float:
    """Lebesgue measure of the uniforms u in [0, 1) whose draw from w is flagged: in t = u Z the
    flagged part of bin k is its first and last final_window(w_k), or the whole bin when it is
    narrower than both together; divided by Z."""
    wp = w[w > 0]
    Z = float(np.sum(w))
    win = np.maximum(FLAG_TOL * wp, ABS_WINDOW)
    return float(min(1.0, np.sum(np.minimum(wp, 2.0 * win)) / Z))


def accept_window_measure(ratio: float) -> float:
    """Lebesgue measure of {u in [0,1) : |u - r| < 1e-5}: the chance that a test with this
    ratio is flagged. Summed over the tests actually performed it estimates the expected
    number of flagged accept decisions."""
    return max(0.0, min(1.0, ratio + FLAG_TOL) - max(0.0, ratio - FLAG_TOL))


# --------------------------------------------------------------------------------------------

def row_is_valid(L: int, D: int, T: float, tokens_b: np.ndarray, V: int) -> bool:
    if not (0 <= L <= D):
        return False
    if not (math.isfinite(T) and T >= 0.0):
        return False
    x = tokens_b[:L]
    return bool(np.all((x >= 0) & (x < V)))


def verify(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray,
           lens: np.ndarray | None, uniforms: np.ndarray,
           temperature: np.ndarray) -> Result:
    """Verify a batch. target [B][D+1][V], draft [B][D][V] (float32 values; bf16 inputs are
    passed decoded), tokens [B][D] int, lens [B] or None (all D), uniforms [B][D+1] float32,
    temperature [B] float32."""
    B, D1, V = target.shape
    D = D1 - 1
    assert draft.shape == (B, D, V) and tokens.shape == (B, D)
    assert uniforms.shape == (B, D + 1) and temperature.shape == (B,)
    if lens is None:
        lens = np.full(B, D, dtype=np.int32)

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

        if T == 0.0:                                   # greedy: exact argmax match
            for i in range(L + 1):
                res.greedy_argmax[b, i] = int(np.argmax(target[b, i]))
            j = 0
            while j < L and x[j] == res.greedy_argmax[b, j]:
                out[j] = x[j]
                j += 1
            out[j] = res.greedy_argmax[b, j]
            res.accept_len[b] = j + 1
            res.final_row[b] = j
            res.final_mode[b] = 1
            continue

        u_final = float(uniforms[b, D])
        rejected_at = -1
        for i in range(L):
            lp, mt, lst = tempered_log_softmax(target[b, i], T)
            lq, md, lsd = tempered_log_softmax(draft[b, i], T)
            res.row_max_t[b, i], res.row_logsum_t[b, i] = mt, lst
            res.row_max_d[b, i], res.row_logsum_d[b, i] = md, lsd
            res.logp_x[b, i], res.logq_x[b, i] = lp[x[i]], lq[x[i]]
            # p/q = exp(log p - log q); beyond the double range it is +inf (an acceptance)
            d = lp[x[i]] - lq[x[i]]
            ratio = math.exp(d) if d < 709.0 else math.inf
            u = float(uniforms[b, i])
            if abs(u - ratio) < FLAG_TOL:
                res.flagged[b] = True
            res.flag_measure[b] += accept_window_measure(ratio)
            if accepts(u, ratio):
                out[i] = x[i]
                continue
            rejected_at = i
            break

        if rejected_at >= 0:
            j = rejected_at
            w = residual_weights(softmax(target[b, j], T), softmax(draft[b, j], T))
            res.final_mode[b] = 2
        else:
            j = L
            _, mt, lst = tempered_log_softmax(target[b, j], T)
            res.row_max_t[b, j], res.row_logsum_t[b, j] = mt, lst
            w = softmax(target[b, j], T)
            res.final_mode[b] = 3
        if not np.any(w > 0):                 # residual of zero mass: rounding only
            w = softmax(target[b, j], T)
            res.flagged[b] = True
            res.flag_measure[b] += 1.0
        else:
            res.flag_measure[b] += final_window_measure(w)
        k, fl, _, _, _ = inverse_cdf(w, u_final)
        out[j] = k
        res.flagged[b] |= fl
        res.accept_len[b] = j + 1
        res.final_row[b] = j
    return res


def verify_workload(w) -> Result:
    """Convenience wrapper for a workloads.Workload."""
    return verify(w.target_f32(), w.draft_f32(), w.tokens,
                  w.lens if w.lens_given else None, w.uniforms, w.temperature)

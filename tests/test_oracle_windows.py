"""Pins of the oracle's excusal windows and of the Saguaro oracle's bf16 rounding.

Every GPU parity claim excuses the rows the oracle flags, so the flags themselves are pinned
here against values computed apart from the oracle (mpmath at 50 digits on the same fp32
inputs, torch's own float32 -> bfloat16 conversion):

  * accept tests: a uniform planted 0.7e-5 from p(x)/q(x) is flagged, one planted 2e-5 away is
    not (below, above, and around r = 1 where min(1, r) clips);
  * the accept-window measure equals the flagged fraction of a fine grid of uniforms;
  * final draws: u * Z planted 0.7e-5 * w_k inside either edge of the chosen bin is flagged,
    2e-5 * w_k inside is not (bonus and residual draws);
  * the absolute floor of the final window: on a residual of mass about 1e-9, u * Z planted
    0.5e-12 from an edge is flagged and 3e-12 away is not;
  * the final-window measure equals the flagged fraction of a fine grid of uniforms;
  * threshold acceptance: a prefix score planted 0.7e-5 from ln tau is flagged, 2e-5 away is
    not, and the prefix-test window measure equals the flag rate over the draft token's
    distribution, enumerated token by token;
  * the bf16 rounding of reshaped Saguaro logits (and the generator's) equals torch's
    float32 -> bfloat16 conversion, exact ties and the largest finite values included.

Each pin is a function of the oracle entry points, so that test_oracle_mutations.py can run it
against copies with a widened, narrowed or missing window, or a truncating rounding.
"""
import mpmath
import numpy as np
import scipy.special
import torch

import oracle
from oracle import saguaro
from workloads import gen

mpmath.mp.dps = 50

T1 = np.ones(1, np.float32)


def _mp_softmax(row, T=1.0):
    """50-digit softmax of the fp32 values of row (the values the oracle receives)."""
    z = [mpmath.mpf(float(np.float32(v))) / mpmath.mpf(float(T)) for v in row]
    m = max(z)
    e = [mpmath.e ** (zi - m) for zi in z]
    s = mpmath.fsum(e)
    return [ei / s for ei in e]


def _batch(rows, B):
    return np.ascontiguousarray(np.broadcast_to(np.asarray(rows, np.float32), (B,) + np.shape(rows)))


# ------------------------------------------------------------------ accept tests

# (target row 0, draft row 0, draft token): the residual max(0, p0 - q0) has one positive
# token, so a rejection draws it with certainty; target row 1 is one-hot to fp64 precision,
# so a bonus draw at u = 0.5 is far from every edge. Only the accept test can be flagged.
ACCEPT_CASES = [
    ([0.0, -0.5, -1.2], [-0.3, 0.2, -0.5], 1),          # r about 0.67
    ([0.0, 0.0, -1.0], [0.0, 9.47e-6, -1.0], 0),        # r about 1 + 4e-6 (min(1, r) = 1)
    ([0.0, 0.0, -1.0], [0.0, -9.47e-6, -1.0], 0),       # r about 1 - 4e-6
    ([0.0, -12.0, -1.0], [-1.0, 0.3, -1.0], 1),         # r about 4e-6
]
BONUS_ROW = [0.0, -60.0, -60.0]


def _mp_ratio(t0, d0, x):
    return _mp_softmax(t0)[x] / _mp_softmax(d0)[x]


def _run_accept(verify, t0, d0, x, us):
    B = len(us)
    u = np.zeros((B, 2), np.float32)
    u[:, 0] = us
    u[:, 1] = 0.5
    return verify(_batch([t0, BONUS_ROW], B), _batch([d0], B), np.full((B, 1), x, np.int32),
                  None, u, np.ones(B, np.float32))


def pin_accept_window(verify):
    """Uniforms planted at distances 0.7e-5 (flagged) and 2e-5 (not flagged) from r."""
    for t0, d0, x in ACCEPT_CASES:
        r = _mp_ratio(t0, d0, x)
        us = []
        for d in (-2e-5, -0.7e-5, 0.7e-5, 2e-5):
            v = float(r + d)
            if 0.0 <= v < 1.0:
                us.append(np.float32(v))
        res = _run_accept(verify, t0, d0, x, np.array(us, np.float32))
        for i, v in enumerate(us):
            want = abs(mpmath.mpf(float(v)) - r) < mpmath.mpf("1e-5")
            if bool(res.flagged[i]) != bool(want):
                return False
    return True


def _fp32_grid(lo, hi, n):
    g = np.unique(np.linspace(max(lo, 0.0), min(hi, 1.0), n).astype(np.float32))
    return g[(g >= 0) & (g < 1)]


def pin_accept_measure(verify, measure):
    """The flagged fraction of [0, 1) under a fine grid of fp32 uniforms around r (nothing is
    flagged on a coarse grid elsewhere) equals accept_window_measure(r)."""
    for t0, d0, x in ACCEPT_CASES:
        r = float(_mp_ratio(t0, d0, x))
        fine = _fp32_grid(r - 4e-5, r + 4e-5, 2001)
        res = _run_accept(verify, t0, d0, x, fine)
        f = res.flagged.astype(np.float64)
        # Riemann sum over the fp32 grid, each point standing for the gap after it (the last
        # one up to 1 when the grid reaches the largest fp32 below 1); the window lies inside
        # the grid, so its end points are unflagged unless the grid stops at 0 or 1
        top = 1.0 if fine[-1] == np.float32(1.0 - 2**-24) else float(fine[-1]) + 1e-8
        edges = np.append(fine.astype(np.float64), top)
        got = float(np.sum(f * np.diff(edges)))
        if (f[0] and fine[0] > 0) or (f[-1] and top < 1.0):
            return False
        coarse = np.arange(0.0005, 1.0, 0.001, dtype=np.float32)
        coarse = coarse[np.abs(coarse.astype(np.float64) - r) > 5e-5]
        if _run_accept(verify, t0, d0, x, coarse).flagged.any():
            return False
        if abs(got - measure(r)) > 2 * float(np.max(np.diff(edges))):
            return False
    return True


# ------------------------------------------------------------------ final draws

RES_T0 = [0.5, 0.0, 0.4, -1.0]        # p > q at tokens 0 and 2
RES_D0 = [0.0, 0.6, 0.0, -0.5]
BON_T1 = [0.3, -0.2, 0.1, -2.0]


def _final_case(kind):
    """(target [2][V], draft [1][V], token, u0, exact weights w, Z): a residual draw at
    position 0 (u0 = 0.9999 > r), or a bonus draw from target row 1 (u0 = 0 < r)."""
    if kind == "residual":
        p, q = _mp_softmax(RES_T0), _mp_softmax(RES_D0)
        w = [max(mpmath.mpf(0), a - b) for a, b in zip(p, q)]
        assert w[0] > 0 and w[2] > 0 and w[1] == 0 and w[3] == 0
        assert float(p[1] / q[1]) < 0.99
        return [RES_T0, BON_T1], [RES_D0], 1, 0.9999, w
    w = _mp_softmax(BON_T1)
    return [RES_T0, BON_T1], [RES_D0], 1, 0.0, w


def _run_final(verify, target, draft, x, u0, ufs):
    B = len(ufs)
    u = np.zeros((B, 2), np.float32)
    u[:, 0] = u0
    u[:, 1] = ufs
    return verify(_batch(target, B), _batch(draft, B), np.full((B, 1), x, np.int32), None, u,
                  np.ones(B, np.float32))


def _expected_flag(w, uf, abs_window=1e-12):
    """Chosen bin and flag of the exact weights at the fp32 uniform uf (50-digit arithmetic)."""
    Z = mpmath.fsum(w)
    t = mpmath.mpf(float(uf)) * Z
    F = mpmath.mpf(0)
    for k, wk in enumerate(w):
        lo, F = F, F + wk
        if F > t:
            win = max(mpmath.mpf("1e-5") * wk, mpmath.mpf(abs_window))
            return k, bool(t - lo < win or F - t < win)
    raise AssertionError("u * Z beyond the last bin")


def pin_final_window(verify):
    """u * Z planted 0.7e-5 * w_k (flagged) and 2e-5 * w_k (not) inside the lower and upper
    edges of a positive bin, for residual and bonus draws."""
    for kind in ("residual", "bonus"):
        target, draft, x, u0, w = _final_case(kind)
        Z = mpmath.fsum(w)
        F = np.cumsum([mpmath.mpf(0)] + list(w))
        ufs, want = [], []
        for k in (0, 2):
            lo, hi, wk = F[k], F[k + 1], w[k]
            for d in (0.7e-5, 2e-5):
                for t in (lo + d * wk, hi - d * wk):
                    uf = np.float32(float(t / Z))
                    kk, fl = _expected_flag(w, uf)
                    assert kk == k
                    ufs.append(uf)
                    want.append(fl)
        assert any(want) and not all(want)
        res = _run_final(verify, target, draft, x, u0, np.array(ufs, np.float32))
        if kind == "residual" and not np.all(res.final_mode == 2):
            return False
        if kind == "bonus" and not np.all(res.final_mode == 3):
            return False
        if not np.array_equal(res.flagged, np.array(want)):
            return False
    return True


# residual of mass about 1e-9: p and q agree to 4e-9 on tokens 0 and 1
TINY_T0 = [0.0, -4e-9, -50.0]
TINY_D0 = [0.0, 0.0, -40.0]


def _tiny_case():
    p, q = _mp_softmax(TINY_T0), _mp_softmax(TINY_D0)
    w = [max(mpmath.mpf(0), a - b) for a, b in zip(p, q)]
    assert w[1] == 0 and w[2] == 0 and 5e-10 < w[0] < 2e-9
    return w


def pin_absolute_window(verify):
    """On the residual of mass about 1e-9 (one positive token, bin [0, Z)): u * Z planted 0.5e-12
    from either edge is flagged, 3e-12 away is not (1e-5 * w_k is only 1e-14 there)."""
    w = _tiny_case()
    Z = w[0]
    ufs, want = [], []
    for t in (mpmath.mpf("0.5e-12"), mpmath.mpf("3e-12"), Z - mpmath.mpf("0.5e-12"),
              Z - mpmath.mpf("3e-12")):
        uf = np.float32(float(t / Z))
        ufs.append(uf)
        want.append(_expected_flag(w, uf)[1])
    if want != [True, False, True, False]:
        raise AssertionError(want)
    res = _run_final(verify, [TINY_T0, BONUS_ROW], [TINY_D0], 2, 0.5, np.array(ufs, np.float32))
    return bool(np.all(res.final_mode == 2) and np.array_equal(res.flagged, np.array(want)))


def pin_final_measure(inverse_cdf, measure):
    """The flagged fraction of [0, 1) over a fine grid of uniforms near every bin edge (and none
    on a coarse grid elsewhere) equals final_window_measure(w), for a residual, a bonus and the
    tiny residual (weights as the oracle computes them: fp64 softmax and max(0, p - q))."""
    cases = [oracle.residual_weights(oracle.softmax(np.float32(RES_T0), 1.0),
                                     oracle.softmax(np.float32(RES_D0), 1.0)),
             oracle.softmax(np.float32(BON_T1), 1.0),
             oracle.residual_weights(oracle.softmax(np.float32(TINY_T0), 1.0),
                                     oracle.softmax(np.float32(TINY_D0), 1.0))]
    for w in cases:
        Z = float(np.sum(w))
        edges = np.unique(np.concatenate([[0.0], np.cumsum(w) / Z]))
        half = 4e-5 if Z > 1e-6 else 4e-3
        got = 0.0
        covered = []
        for e in edges:
            a, b = max(0.0, e - half), min(1.0, e + half)
            n = 20001
            g = np.linspace(a, b, n, endpoint=False)
            step = (b - a) / n
            fl = np.array([inverse_cdf(w, float(u))[1] for u in g])
            if (a > 0 and fl[0]) or (b < 1 and fl[-1]):
                return False                 # the grid must contain the whole window
            got += float(np.sum(fl)) * step
            covered.append((a, b))
        coarse = [u for u in np.arange(5e-4, 1.0, 1e-3)
                  if all(not (a <= u < b) for a, b in covered)]
        if any(inverse_cdf(w, float(u))[1] for u in coarse):
            return False
        want = measure(w)
        if abs(got - want) > 1e-3 * want + 1e-9:
            return False
    return True


# ------------------------------------------------------------------ threshold acceptance

THR_T = [0.3, -0.2, 0.1, -2.0]        # target rows 0 and 1 (equal: the extra token's row does
THR_D = [0.2, 0.1, -0.3, -1.0]        # not depend on where the prefix stops)


def _thr_center_uniform():
    """A final uniform at the centre of the widest bin of p (never flagged)."""
    p = [float(v) for v in _mp_softmax(THR_T)]
    F = np.concatenate([[0.0], np.cumsum(p)])
    k = int(np.argmax(p))
    return np.float32((F[k] + F[k + 1]) / 2)


def _run_thr(vt, x0s, tau):
    B = len(x0s)
    u = np.zeros((B, 2), np.float32)
    u[:, 1] = _thr_center_uniform()
    return vt(_batch([THR_T, THR_T], B), np.array(x0s, np.int32).reshape(B, 1), None, u,
              np.ones(B, np.float32), tau, draft=_batch([THR_D], B))


def pin_threshold_window(vt):
    """ln tau planted 0.7e-5 (flagged) and 2e-5 (not flagged) from the score log p_0(x_0)."""
    lp = mpmath.log(_mp_softmax(THR_T)[2])
    for d in (-2e-5, -0.7e-5, 0.7e-5, 2e-5):
        tau = float(mpmath.e ** (lp + d))
        res = _run_thr(vt, [2], tau)
        want = abs(mpmath.log(mpmath.mpf(tau)) - lp) < mpmath.mpf("1e-5")
        if bool(res.flagged[0]) != bool(want):
            return False
        if res.accept_len[0] != (2 if d < 0 else 1):
            return False
    return True


def pin_threshold_measure(vt):
    """With ln tau planted 0.3e-5 above log p_0(2), test 0 is flagged exactly when the draft
    token is 2: enumerating x_0 over the vocabulary, the q-weighted flag rate (scipy's softmax of
    the draft row) equals the prefix part of the oracle's window measure, for every x_0."""
    lp = _mp_softmax(THR_T)
    tau = float(mpmath.e ** (mpmath.log(lp[2]) + mpmath.mpf("0.3e-5")))
    V = len(THR_T)
    res = _run_thr(vt, list(range(V)), tau)
    q = scipy.special.softmax(np.float32(THR_D).astype(np.float64))
    rate = float(np.sum(q * res.flagged))
    final = np.array([oracle.final_window_measure(oracle.softmax(np.float32(THR_T), 1.0))] * V)
    prefix = res.flag_measure - final
    return bool(abs(rate - q[2]) < 1e-15 and np.all(np.abs(prefix - rate) < 1e-12))


# ------------------------------------------------------------------ bf16 rounding

def _torch_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _rounding_inputs():
    rng = np.random.default_rng(31)
    vals = [(rng.standard_normal(20000) * 30).astype(np.float32)]
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]                 # finite patterns only
    vals.append(bits.view(np.float32))
    hi = rng.integers(0, 2**16, 4000, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]
    ties = ((hi << 16) | 0x8000).astype(np.uint32)                  # exactly half an ulp
    near = np.concatenate([(hi << 16) | 0x7FFF, (hi << 16) | 0x8001]).astype(np.uint32)
    edge = np.array([0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000, 0xFF7F7FFF, 0x7F7E8000, 0x00008000,
                     0x00018000, 0x80008000, 0x3F808000, 0x3F818000], np.uint32)
    for b in (ties, near, edge):
        vals.append(b.view(np.float32))
    return np.concatenate(vals)


def pin_bf16_rounding(rne):
    x = _rounding_inputs()
    return bool(np.array_equal(rne(x), _torch_bf16_bits(x)))


# ------------------------------------------------------------------ the pins on the oracle

def test_accept_window_is_pinned():
    assert pin_accept_window(oracle.verify)


def test_accept_measure_matches_the_flagged_fraction():
    assert pin_accept_measure(oracle.verify, oracle.accept_window_measure)


def test_final_window_is_pinned():
    assert pin_final_window(oracle.verify)


def test_absolute_final_window_is_pinned():
    assert pin_absolute_window(oracle.verify)


def test_final_measure_matches_the_flagged_fraction():
    assert pin_final_measure(oracle.inverse_cdf, oracle.final_window_measure)


def test_threshold_window_is_pinned():
    assert pin_threshold_window(oracle.verify_threshold)


def test_threshold_measure_matches_the_flag_rate():
    assert pin_threshold_measure(oracle.verify_threshold)


def test_saguaro_bf16_rounding_matches_torch():
    assert pin_bf16_rounding(saguaro._bf16_rne)


def test_generator_bf16_rounding_matches_torch():
    assert pin_bf16_rounding(gen.bf16_round)

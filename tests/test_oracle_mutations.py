"""The oracle pins catch plausible mistakes.

Each pin below is a check of an oracle against something other than itself (a library routine,
brute force, or the definition restated another way). Each is run against the real oracle, where
it must pass, and against copies of the oracle with one planted mistake (a dropped temperature, a
wrong sign, an index off by one, a shifted position), where it must fail. The mistakes are planted
in the CPU oracles only.
"""
import importlib
import inspect
import textwrap

import numpy as np
import pytest
import scipy.special

import oracle
# the modules (the package exports functions of the same names)
advance_mod = importlib.import_module("oracle.advance")
oracle_mod = importlib.import_module("oracle.oracle")
threshold_mod = importlib.import_module("oracle.threshold")


def _sp_softmax(row, T):
    return scipy.special.softmax(np.asarray(row, np.float64) / T)


def _plain_draw(p, u):
    return int(np.searchsorted(np.cumsum(p), u * p.sum(), side="right"))


# ---------------------------------------------------------------- pins of the sampler oracle

def pin_no_draft_draw(verify):
    """L = 0 at T = 0.7: the token is searchsorted over scipy's softmax of target row 0, with the
    final uniform u[b][D]."""
    rng = np.random.default_rng(5)
    B, D, V = 200, 3, 12
    tgt = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    drf = (rng.standard_normal((B, D, V)) * 2).astype(np.float32)
    toks = rng.integers(0, V, (B, D)).astype(np.int32)
    u = rng.random((B, D + 1), dtype=np.float32)
    T = np.full(B, 0.7, np.float32)
    r = verify(tgt, drf, toks, np.zeros(B, np.int32), u, T)
    ok = ~r.flagged
    want = np.array([_plain_draw(_sp_softmax(tgt[b, 0], 0.7), u[b, D]) for b in range(B)])
    return bool(np.all(r.accept_len == 1) and np.array_equal(r.tokens[ok, 0], want[ok]))


def pin_residual_draw(verify):
    """A forced rejection at position 0 (the draft token has q far above p, u near 1): the token
    is searchsorted over scipy's max(0, p - q)."""
    rng = np.random.default_rng(6)
    B, D, V = 200, 1, 10
    tgt = (rng.standard_normal((B, D + 1, V)) * 1.5).astype(np.float32)
    drf = tgt[:, :D].copy()
    toks = rng.integers(0, V, (B, D)).astype(np.int32)
    for b in range(B):                      # make the draft token far more likely under q
        drf[b, 0, toks[b, 0]] += 6.0
    u = rng.random((B, D + 1), dtype=np.float32)
    u[:, 0] = 0.999
    r = verify(tgt, drf, toks, None, u, np.ones(B, np.float32))
    ok = ~r.flagged
    good = 0
    for b in np.nonzero(ok)[0]:
        if r.accept_len[b] != 1:
            return False
        w = np.maximum(0.0, _sp_softmax(tgt[b, 0], 1.0) - _sp_softmax(drf[b, 0], 1.0))
        if r.tokens[b, 0] != _plain_draw(w, u[b, D]):
            return False
        good += 1
    return good > 0.9 * B


def pin_scaling(verify):
    """Scaling logits and temperature by the same power of two changes no output."""
    rng = np.random.default_rng(7)
    B, D, V = 100, 3, 16
    tgt = (rng.standard_normal((B, D + 1, V)) * 2).astype(np.float32)
    drf = (tgt[:, :D] + rng.standard_normal((B, D, V))).astype(np.float32)
    toks = rng.integers(0, V, (B, D)).astype(np.int32)
    u = rng.random((B, D + 1), dtype=np.float32)
    T = np.full(B, 0.5, np.float32)
    a = verify(tgt, drf, toks, None, u, T)
    b = verify(tgt * 4, drf * 4, toks, None, u, T * 4)
    ok = ~(a.flagged | b.flagged)
    return bool(np.array_equal(a.accept_len[ok], b.accept_len[ok]) and
                np.array_equal(a.tokens[ok], b.tokens[ok]))


SAMPLER_PINS = [pin_no_draft_draw, pin_residual_draw, pin_scaling]


def test_sampler_pins_pass_on_the_oracle():
    for pin in SAMPLER_PINS:
        assert pin(oracle.verify), pin.__name__


@pytest.mark.parametrize("mutation", ["temperature_dropped", "residual_sign", "draw_off_by_one",
                                      "ratio_inverted"])
def test_sampler_mutations_are_caught(monkeypatch, mutation):
    if mutation == "temperature_dropped":
        real_sm, real_lsm = oracle_mod.softmax, oracle_mod.tempered_log_softmax
        monkeypatch.setattr(oracle_mod, "softmax", lambda x, T: real_sm(x, 1.0))
        monkeypatch.setattr(oracle_mod, "tempered_log_softmax", lambda x, T: real_lsm(x, 1.0))
    elif mutation == "residual_sign":
        monkeypatch.setattr(oracle_mod, "residual_weights", lambda p, q: np.maximum(0.0, q - p))
    elif mutation == "draw_off_by_one":
        real = oracle_mod.inverse_cdf

        def shifted(w, u):
            k, fl, lo, hi, Z = real(w, u)
            return min(k + 1, len(w) - 1), fl, lo, hi, Z
        monkeypatch.setattr(oracle_mod, "inverse_cdf", shifted)
    elif mutation == "ratio_inverted":
        monkeypatch.setattr(oracle_mod, "accepts",
                            lambda u, r: u < min(1.0, 1.0 / r if r > 0 else np.inf))
    caught = [not pin(oracle.verify) for pin in SAMPLER_PINS]
    if mutation == "ratio_inverted":          # only the accept tests change: statistical pins
        # (test_oracle_stats) cover it; here, the forced rejection must turn into acceptance
        assert not pin_residual_draw(oracle.verify)
    else:
        assert any(caught), mutation


# ---------------------------------------------------------------- threshold acceptance

def pin_threshold_bruteforce(vt):
    rng = np.random.default_rng(8)
    B, D, V = 200, 3, 6
    tgt = (rng.standard_normal((B, D + 1, V)) * 1.5).astype(np.float32)
    toks = rng.integers(0, V, (B, D)).astype(np.int32)
    lens = rng.integers(0, D + 1, B).astype(np.int32)
    u = rng.random((B, D + 1), dtype=np.float32)
    T = rng.choice(np.array([0.5, 2.0], np.float32), B)
    tau = 0.02
    r = vt(tgt, toks, lens, u, T, tau)
    for b in np.nonzero(~r.flagged)[0]:
        L = lens[b]
        p = [_sp_softmax(tgt[b, i], T[b]) for i in range(D + 1)]
        scores = [np.prod([p[i][toks[b, i]] for i in range(k)]) for k in range(L + 1)]
        kept = max(k for k in range(L + 1) if k == 0 or scores[k] > tau)
        if r.accept_len[b] != kept + 1 or r.tokens[b, kept] != _plain_draw(p[kept], u[b, D]):
            return False
    return True


def test_threshold_pin_passes_on_the_oracle():
    assert pin_threshold_bruteforce(oracle.verify_threshold)


@pytest.mark.parametrize("mutation", ["temperature_dropped", "position_shift", "draw_row_shift"])
def test_threshold_mutations_are_caught(monkeypatch, mutation):
    if mutation == "temperature_dropped":
        real = threshold_mod.tempered_log_softmax
        monkeypatch.setattr(threshold_mod, "tempered_log_softmax", lambda x, T: real(x, 1.0))
    elif mutation == "position_shift":
        # each prefix scored with the next token's log-probability
        real = threshold_mod.tempered_log_softmax

        def rolled(x, T):
            lp, m, s = real(x, T)
            return np.roll(lp, 1), m, s
        monkeypatch.setattr(threshold_mod, "tempered_log_softmax", rolled)
    elif mutation == "draw_row_shift":
        real = threshold_mod.softmax
        monkeypatch.setattr(threshold_mod, "softmax", lambda x, T: real(np.roll(x, 1), T))
    assert not pin_threshold_bruteforce(oracle.verify_threshold), mutation


# ---------------------------------------------------------------- epilogue

def pin_advance_suffix(adv):
    """After several steps each window equals the last W tokens of the whole token stream and
    each length its start plus every AL (AL up to D + 1)."""
    rng = np.random.default_rng(9)
    B, D, W = 16, 4, 6
    ids = rng.integers(0, 1000, (B, W)).astype(np.int32)
    lens = rng.integers(0, 50, B).astype(np.int32)
    stream = [list(ids[b]) for b in range(B)]
    total = lens.astype(np.int64).copy()
    for _ in range(6):
        al = rng.integers(1, D + 2, B).astype(np.int32)
        toks = np.full((B, D + 1), -1, np.int32)
        for b in range(B):
            toks[b, :al[b]] = rng.integers(0, 1000, al[b])
            stream[b].extend(toks[b, :al[b]].tolist())
        total += al
        ids, lens = adv(al, toks, D, ids, lens)
        if any(ids[b].tolist() != stream[b][-W:] for b in range(B)):
            return False
        if not np.array_equal(lens, total):
            return False
    return True


def _mutant_advance(old, new):
    """A copy of the epilogue oracle with one statement changed."""
    src = textwrap.dedent(inspect.getsource(advance_mod.advance))
    assert old in src, old
    ns = {"np": np, "INT32_MAX": advance_mod.INT32_MAX}
    exec(src.replace(old, new), ns)
    return ns["advance"]


def test_advance_pin_passes_on_the_oracle():
    assert pin_advance_suffix(oracle.advance)


@pytest.mark.parametrize("old,new", [
    ("src = j + a", "src = j + a - 1"),
    ("lens[b] += a", "lens[b] += a - 1"),
    ("if a < 1 or a > D + 1:", "if a < 1 or a > D:"),
    ("tokens[b, src - W]", "tokens[b, a - 1 - (src - W)]"),          # emitted tokens reversed
])
def test_advance_mutations_are_caught(old, new):
    assert not pin_advance_suffix(_mutant_advance(old, new)), new


# ---------------------------------------------------------------- Saguaro reshaping

saguaro_mod = importlib.import_module("oracle.saguaro")


def pin_saguaro(reshape, top_k):
    """Tie-heavy rows: the changed tokens are the brute-force top k; in probability space the
    row becomes q with its top k scaled by c and renormalised."""
    rng = np.random.default_rng(10)
    B, D, V, k, c = 4, 2, 60, 5, 0.4
    draft = rng.integers(-3, 4, (B, D, V)).astype(np.float32)
    T = np.array([1.0, 0.5, 2.0, 1.5], np.float32)
    out = reshape(draft, "f32", None, T, c, k)
    for b in range(B):
        for i in range(D):
            row = draft[b, i]
            want = [j for _, j in sorted((-float(v), j) for j, v in enumerate(row))][:k]
            if sorted(top_k(row, k).tolist()) != sorted(want):
                return False
            q = scipy.special.softmax(row.astype(np.float64) / T[b])
            q[want] *= c
            q /= q.sum()
            got = scipy.special.softmax(out[b, i].astype(np.float64) / T[b])
            if not np.allclose(got, q, rtol=2e-6, atol=1e-12):
                return False
    return True


def test_saguaro_pin_passes_on_the_oracle():
    assert pin_saguaro(saguaro_mod.reshape_draft, saguaro_mod.top_k_indices)


def _mutant_saguaro(old, new):
    src = inspect.getsource(saguaro_mod)
    assert old in src, old
    ns = {"__name__": "saguaro_mutant"}
    exec(src.replace(old, new), ns)
    return ns["reshape_draft"], ns["top_k_indices"]


@pytest.mark.parametrize("old,new", [
    ("order = np.lexsort((idx, -row.astype(np.float64)))",
     "order = np.lexsort((-idx, -row.astype(np.float64)))"),               # ties to the highest
    ("new = (vals[sel] + delta)", "new = (vals[sel] - delta)"),            # shift sign
    ("delta = np.float32(np.float32(temperature[b]) * lnf)", "delta = lnf"),  # temperature dropped
])
def test_saguaro_mutations_are_caught(old, new):
    assert not pin_saguaro(*_mutant_saguaro(old, new)), new


# ---------------------------------------------------------------- excusal windows and rounding

from tests import test_oracle_windows as PW  # noqa: E402


def _mutant_module(mod, old, new):
    """A copy of an oracle module with one statement changed (relative imports resolve against
    the real package)."""
    src = inspect.getsource(mod)
    assert old in src, old
    ns = {"__name__": mod.__name__, "__package__": "oracle"}
    exec(src.replace(old, new), ns)
    return ns


def _window_pins(ns):
    return {
        "accept": lambda: PW.pin_accept_window(ns["verify"]),
        "accept_measure": lambda: PW.pin_accept_measure(ns["verify"], ns["accept_window_measure"]),
        "final": lambda: PW.pin_final_window(ns["verify"]),
        "absolute": lambda: PW.pin_absolute_window(ns["verify"]),
        "final_measure": lambda: PW.pin_final_measure(ns["inverse_cdf"],
                                                      ns["final_window_measure"]),
    }


@pytest.mark.parametrize("old,new,catcher", [
    ("if abs(u - ratio) < FLAG_TOL:", "if abs(u - ratio) < 10 * FLAG_TOL:", "accept"),
    ("if abs(u - ratio) < FLAG_TOL:", "if abs(u - ratio) < 0.5 * FLAG_TOL:", "accept"),
    ("if abs(u - ratio) < FLAG_TOL:", "if abs(u - ratio) < 10 * FLAG_TOL:", "accept_measure"),
    ("min(1.0, ratio + FLAG_TOL) - max(0.0, ratio - FLAG_TOL)",
     "min(1.0, ratio + 2 * FLAG_TOL) - max(0.0, ratio - 2 * FLAG_TOL)", "accept_measure"),
    ("return max(FLAG_TOL * wk, ABS_WINDOW)", "return max(10 * FLAG_TOL * wk, ABS_WINDOW)",
     "final"),
    ("return max(FLAG_TOL * wk, ABS_WINDOW)", "return max(0.5 * FLAG_TOL * wk, ABS_WINDOW)",
     "final"),
    ("return max(FLAG_TOL * wk, ABS_WINDOW)", "return FLAG_TOL * wk", "absolute"),
    ("ABS_WINDOW = 1e-12", "ABS_WINDOW = 1e-11", "absolute"),
    ("return max(FLAG_TOL * wk, ABS_WINDOW)", "return max(10 * FLAG_TOL * wk, ABS_WINDOW)",
     "final_measure"),
    ("return float(min(1.0, np.sum(np.minimum(wp, 2.0 * win)) / Z))", "return 2.0 * FLAG_TOL",
     "final_measure"),
])
def test_window_mutations_are_caught(old, new, catcher):
    ns = _mutant_module(oracle_mod, old, new)
    assert _window_pins(importlib.import_module("oracle.oracle").__dict__)[catcher]()
    assert not _window_pins(ns)[catcher](), new


@pytest.mark.parametrize("old,new,catcher", [
    ("win = FLAG_TOL * (i + 1)", "win = 10 * FLAG_TOL * (i + 1)", PW.pin_threshold_window),
    ("win = FLAG_TOL * (i + 1)", "win = 0.5 * FLAG_TOL * (i + 1)", PW.pin_threshold_window),
    ("score, log_tau, win)", "score + lp[x[i]], log_tau, win)", PW.pin_threshold_measure),
])
def test_threshold_window_mutations_are_caught(old, new, catcher):
    ns = _mutant_module(threshold_mod, old, new)
    assert catcher(oracle.verify_threshold)
    assert not catcher(ns["verify_threshold"]), new


@pytest.mark.parametrize("old,new", [
    ("return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)",
     "return (u >> np.uint32(16)).astype(np.uint16)"),                      # truncation
    ("return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)",
     "return ((u + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)"),   # ties away
])
def test_bf16_rounding_mutations_are_caught(old, new):
    ns = _mutant_module(saguaro_mod, old, new)
    assert PW.pin_bf16_rounding(saguaro_mod._bf16_rne)
    assert not PW.pin_bf16_rounding(ns["_bf16_rne"]), new

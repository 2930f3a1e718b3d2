"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

  * AL lies in [1, 1 + L] ("NVIDIA: öt irányelv ...", section "Mit csinál a spekulatív
    dekódolás?").
  * A draft equal to the target is always accepted (q <= p accepts, step 1 of the rule in
    "Speculative Speculative Decoding", SD recap), so AL = L + 1.
  * Temperature 0 reproduces greedy autoregressive decoding of the target (NVIDIA page, same
    section: the output equals conventional decoding).
  * With no drafts (L = 0) the call is a plain inverse-CDF draw from p_0: checked against
    numpy.searchsorted over scipy's softmax.
  * Scaling logits and temperature by the same power of two changes nothing.
"""
import numpy as np
import pytest
import scipy.special

from oracle import verify, verify_workload
from workloads import make

SMALL = dict(c1={}, c2=dict(V=3000), c3=dict(B=12, V=4000), c4=dict(B=40, V=4000),
             c5=dict(B=48, V=4000), mtp=dict(B=64, V=4000))


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_accept_length_range_and_token_layout(cfg):
    for seed in range(3):
        w = make(cfg, seed, **SMALL[cfg])
        r = verify_workload(w)
        L = w.lens
        assert np.all(r.accept_len >= 1) and np.all(r.accept_len <= L + 1)
        for b in range(w.B):
            al = r.accept_len[b]
            assert np.array_equal(r.tokens[b, :al - 1], w.tokens[b, :al - 1])
            assert 0 <= r.tokens[b, al - 1] < w.V
            assert np.all(r.tokens[b, al:] == -1)


@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
def test_equal_draft_accepts_everything(T):
    w = make("c3", 11, B=16, V=3000)
    tgt = w.target_f32()
    draft = tgt[:, :w.D].copy()
    rng = np.random.default_rng(0)
    lens = rng.integers(0, w.D + 1, w.B).astype(np.int32)
    temp = np.full(w.B, T, np.float32)
    r = verify(tgt, draft, w.tokens.clip(0), lens, w.uniforms, temp)
    assert np.array_equal(r.accept_len, lens + 1)
    assert np.all(r.final_mode == 3)


def test_greedy_equals_autoregressive_argmax_chain():
    w = make("c4", 4, V=3000)
    g = w.temperature == 0
    tgt = w.target_f32()
    r = verify_workload(w)
    greedy_tokens = np.argmax(tgt, axis=-1)                    # [B][D+1]: greedy decode
    match = np.cumprod(w.tokens == greedy_tokens[:, :w.D], axis=1)
    expected_al = 1 + match.sum(axis=1)
    assert np.array_equal(r.accept_len[g], expected_al[g])
    for b in np.nonzero(g)[0]:
        al = expected_al[b]
        assert np.array_equal(r.tokens[b, :al], greedy_tokens[b, :al])
    # perturb: make every draft the target argmax -> all accepted, bonus = argmax of row D
    toks = greedy_tokens[:, :w.D].astype(np.int32)
    r2 = verify(tgt, w.draft_f32(), toks, None, w.uniforms, np.zeros(w.B, np.float32))
    assert np.all(r2.accept_len == w.D + 1)
    assert np.array_equal(r2.tokens, greedy_tokens.astype(np.int32))


def test_greedy_ties_take_lowest_index():
    V, D = 16, 2
    tgt = np.zeros((1, D + 1, V), np.float32)
    tgt[0, :, 3] = 5.0
    tgt[0, :, 9] = 5.0
    r = verify(tgt, np.zeros((1, D, V), np.float32), np.array([[3, 9]], np.int32), None,
               np.zeros((1, D + 1), np.float32), np.zeros(1, np.float32))
    assert r.accept_len[0] == 2 and list(r.tokens[0]) == [3, 3, -1]


def test_no_draft_is_plain_inverse_cdf():
    rng = np.random.default_rng(3)
    B, V = 200, 257
    tgt = (rng.standard_normal((B, 1, V)) * 3).astype(np.float32)
    u = rng.random((B, 1), dtype=np.float32)
    T = 0.8
    r = verify(tgt, np.zeros((B, 0, V), np.float32), np.zeros((B, 0), np.int32),
               np.zeros(B, np.int32), u, np.full(B, T, np.float32))
    for b in range(B):
        p = scipy.special.softmax(tgt[b, 0].astype(np.float64) / T)
        c = np.cumsum(p)
        k = int(np.searchsorted(c, float(u[b, 0]) * c[-1], side="right"))
        if not r.flagged[b]:
            assert r.tokens[b, 0] == k
    assert np.all(r.accept_len == 1)


def test_power_of_two_scaling_of_logits_and_temperature():
    w = make("c2", 9, V=2000)
    a = verify_workload(w)
    s = np.float32(4.0)
    b = verify(w.target * s, w.draft * s, w.tokens, None, w.uniforms, w.temperature * s)
    assert np.array_equal(a.accept_len, b.accept_len)
    assert np.array_equal(a.tokens, b.tokens)


def test_invalid_rows_are_marked():
    w = make("c3", 1, B=6, V=500)
    tgt, dr = w.target_f32(), w.draft_f32()
    toks = w.tokens.copy()
    lens = np.full(6, w.D, np.int32)
    temp = np.ones(6, np.float32)
    toks[0, 2] = w.V            # token out of range at an evaluated position
    toks[1, 0] = -1
    lens[2] = w.D + 1           # length out of range
    lens[3] = -1
    temp[4] = np.nan            # bad temperature
    temp[5] = -0.5
    r = verify(tgt, dr, toks, lens, w.uniforms, temp)
    assert np.all(r.accept_len == 0) and np.all(r.tokens == -1)
    # a bad token beyond L is ignored
    lens2 = np.full(6, 1, np.int32)
    toks2 = w.tokens.copy()
    toks2[:, 3] = 10 ** 6
    r2 = verify(tgt, dr, toks2, lens2, w.uniforms, np.ones(6, np.float32))
    assert np.all(r2.accept_len >= 1)


def test_padding_rows_are_never_read():
    w = make("c5", 3, B=24, V=3000)
    n = make("c5", 3, B=24, V=3000, pad="nan")
    a, b = verify_workload(w), verify_workload(n)
    assert np.array_equal(a.accept_len, b.accept_len) and np.array_equal(a.tokens, b.tokens)


def test_flag_rate_estimator_is_small_on_full_headline_config():
    w = make("c3", 0)
    r = verify_workload(w)
    assert r.flag_measure.mean() < 1e-4
    assert 1.8 < r.accept_len.mean() < 4.0


def test_ratio_beyond_the_double_range_accepts():
    """q(x) far below p(x) (log-ratio 1500): q <= p, so the draft is accepted whatever the
    uniform (step 1 of the rule, SD recap), and the call is then a bonus draw from p_1."""
    V = 4
    target = np.zeros((1, 2, V), np.float32)
    draft = np.zeros((1, 1, V), np.float32)
    draft[0, 0, 1] = 1500.0                       # q(0) ~ exp(-1500), p(0) = 1/4
    tokens = np.array([[0]], np.int32)
    u = np.array([[0.999999, 0.3]], np.float32)
    r = verify(target, draft, tokens, None, u, np.ones(1, np.float32))
    assert r.accept_len[0] == 2 and r.tokens[0, 0] == 0
    assert r.tokens[0, 1] == 1                    # inverse CDF of uniform p at 0.3: bin 1


def test_residual_below_fp64_resolution_is_flagged():
    """A rejection where p and q agree except far out in the tail: the residual mass is about
    1e-12, below the absolute window (the rounding bound of any fp64 evaluation of the weights),
    so every uniform is flagged: the draw is left to rounding. The same shape with a clear
    difference is not flagged."""
    target = np.array([[[0.0, -4e-12, -50.0], [0.0, 0.0, 0.0]]], np.float64)
    draft = np.array([[[0.0, 0.0, -40.0]]], np.float64)
    tokens = np.array([[2]], np.int32)
    u = np.array([[0.5, 0.3]], np.float32)
    r = verify(target, draft, tokens, None, u, np.ones(1, np.float32))
    assert r.accept_len[0] == 1 and r.final_mode[0] == 2      # q(2) = e^10 p(2): rejected
    assert r.flagged[0]
    target[0, 0, 1] = -0.5                                    # residual mass about 0.12
    r = verify(target, draft, tokens, None, u, np.ones(1, np.float32))
    assert r.accept_len[0] == 1 and not r.flagged[0] and r.tokens[0, 0] == 0

"""Pins of the epilogue oracle (window of the most recent tokens and sequence lengths, moved by
the accepted length; "Accélérer Sonar par la Spéculation", section "Calendrier MTP pour un jeton
unique").

The pins do not re-type the oracle's slide. They check it against the window's definition as a
suffix of the whole token stream: after any number of steps, a sequence's window must equal the
last W tokens of (initial window ++ every token emitted so far), and its length the initial
length plus every AL. A wrong index in the slide (off by one, the emitted tokens reversed or
placed at the front) breaks that identity.
"""
import numpy as np
import pytest

from oracle import advance, verify_workload
from workloads import make


def test_hand_worked_example():
    # window [10 11 12 13], AL = 3 with emitted [7 8 9]: slide by three, append
    ids, lens = advance(np.array([3]), np.array([[7, 8, 9, -1]]), 3, np.array([[10, 11, 12, 13]]),
                        np.array([40]))
    assert ids.tolist() == [[13, 7, 8, 9]] and lens.tolist() == [43]
    # AL = 1: only the final token enters
    ids, _ = advance(np.array([1]), np.array([[5, -1, -1]]), 2, np.array([[1, 2, 3]]))
    assert ids.tolist() == [[2, 3, 5]]
    # a window shorter than AL keeps the last W emitted tokens
    ids, _ = advance(np.array([4]), np.array([[4, 5, 6, 7]]), 3, np.array([[0, 1]]))
    assert ids.tolist() == [[6, 7]]


@pytest.mark.parametrize("W", [1, 2, 5, 8, 40])
def test_window_is_the_suffix_of_the_token_stream(W):
    rng = np.random.default_rng(W)
    B, D, steps = 12, 5, 9
    ids = rng.integers(0, 1000, (B, W)).astype(np.int32)
    lens = rng.integers(0, 100, B).astype(np.int32)
    stream = [list(ids[b]) for b in range(B)]
    total = lens.astype(np.int64).copy()
    for _ in range(steps):
        al = rng.integers(1, D + 2, B).astype(np.int32)
        toks = np.full((B, D + 1), -1, np.int32)
        for b in range(B):
            toks[b, :al[b]] = rng.integers(0, 1000, al[b])
            stream[b].extend(toks[b, :al[b]].tolist())
        total += al
        ids, lens = advance(al, toks, D, ids, lens)
        for b in range(B):
            assert ids[b].tolist() == stream[b][-W:]
        assert np.array_equal(lens, total)


def test_invalid_lengths_leave_the_sequence_unchanged():
    D, W = 3, 6
    ids0 = np.arange(5 * W, dtype=np.int32).reshape(5, W)
    lens0 = np.array([7, 7, -1, 2 ** 31 - 3, 5], np.int32)
    al = np.array([0, D + 2, 2, 3, -4], np.int32)   # AL 0, too long, bad length, overflow, < 0
    toks = np.full((5, D + 1), 99, np.int32)
    ids, lens = advance(al, toks, D, ids0, lens0)
    assert np.array_equal(ids, ids0) and np.array_equal(lens, lens0)
    # with no length array only the AL range decides: row 2 and 3 now move
    ids, none = advance(al, toks, D, ids0)
    assert none is None
    assert np.array_equal(ids[[0, 1, 4]], ids0[[0, 1, 4]])
    assert ids[2].tolist() == ids0[2, 2:].tolist() + [99, 99]
    assert ids[3].tolist() == ids0[3, 3:].tolist() + [99, 99, 99]


def test_after_verification_the_window_ends_with_the_emitted_tokens():
    """Verifier output fed to the epilogue: the window's tail is exactly the accepted drafts
    followed by the final token, and the old window's newest tokens precede them."""
    w = make("c5", 1, B=32, V=2000)
    r = verify_workload(w)
    W = w.D + 3
    ids0 = np.arange(w.B * W, dtype=np.int32).reshape(w.B, W) + 10 ** 6
    ids, lens = advance(r.accept_len, r.tokens, w.D, ids0, np.zeros(w.B, np.int32))
    for b in range(w.B):
        a = r.accept_len[b]
        assert ids[b, W - a:].tolist() == w.tokens[b, :a - 1].tolist() + [r.tokens[b, a - 1]]
        assert ids[b, :W - a].tolist() == ids0[b, a:].tolist()
    assert np.array_equal(lens, r.accept_len)

"""Seeded input generator: shapes, rounding, per-config structure, determinism."""
import numpy as np
import pytest
import scipy.stats
import torch

from workloads import CONFIGS, make, bf16_round, bf16_decode
from workloads.gen import _gumbel_argmax

SMALL = dict(c1={}, c2=dict(V=3000), c3=dict(B=8, V=5000), c4=dict(B=40, V=5000),
             c5=dict(B=32, V=5000), mtp=dict(B=64, V=5000))


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
def test_shapes_and_dtypes(cfg):
    w = make(cfg, 3, **SMALL[cfg])
    B, D, V = w.B, w.D, w.V
    assert w.target.shape == (B, D + 1, V) and w.draft.shape == (B, D, V)
    assert w.target.dtype == (np.uint16 if w.dtype == "bf16" else np.float32)
    assert w.tokens.shape == (B, D) and w.tokens.dtype == np.int32
    assert w.uniforms.shape == (B, D + 1) and w.uniforms.dtype == np.float32
    assert np.all((w.uniforms >= 0) & (w.uniforms < 1))
    assert w.temperature.shape == (B,) and w.lens.shape == (B,)
    for b in range(B):
        L = w.lens[b]
        assert np.all((w.tokens[b, :L] >= 0) & (w.tokens[b, :L] < V))
        assert np.all(w.tokens[b, L:] == -1)
    assert np.all(np.isfinite(w.target_f32())) and np.all(np.isfinite(w.draft_f32()))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 20,
                        # exact ties between two bf16 values: both parities of the kept bit
                        bf16_decode(np.arange(0x3F00, 0x3F40, dtype=np.uint16)) +
                        np.float32(2.0 ** -9),
                        np.array([0.0, -0.0, 1e-30, -3e38], np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_round(x), ref)


def test_determinism_and_seed_dependence():
    a = make("c3", 5, B=4, V=2000)
    b = make("c3", 5, B=4, V=2000)
    c = make("c3", 6, B=4, V=2000)
    for f in ("target", "draft", "tokens", "uniforms", "temperature", "lens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.target, c.target)
    # a sequence's data does not depend on B
    d = make("c3", 5, B=2, V=2000)
    assert np.array_equal(a.target[:2], d.target) and np.array_equal(a.tokens[:2], d.tokens)


def test_c4_structure():
    w = make("c4", 1, V=3000)
    assert w.B == 256 and w.D == 3
    greedy = w.temperature == 0
    assert greedy.sum() == 128
    assert np.all(w.temperature[~greedy] == np.float32(0.7))
    equal = np.array([np.array_equal(w.draft[b], w.target[b, :3]) for b in range(w.B)])
    assert equal.sum() == 25
    # greedy draft tokens are the draft argmax
    dd = w.draft_f32()
    for b in np.nonzero(greedy)[0]:
        assert np.array_equal(w.tokens[b], np.argmax(dd[b], axis=-1))


def test_c5_ragged_and_padding():
    w = make("c5", 2, B=64, V=1000)
    assert w.lens_given and w.lens.min() >= 1 and w.lens.max() <= 7
    assert len(np.unique(w.lens)) > 3
    for b in range(w.B):
        L = w.lens[b]
        assert np.all(w.target[b, L + 1:] == 0) and np.all(w.draft[b, L:] == 0)
    n = make("c5", 2, B=64, V=1000, pad="nan")
    tf, df = n.target_f32(), n.draft_f32()
    for b in range(n.B):
        L = n.lens[b]
        assert np.all(np.isnan(tf[b, L + 1:])) and np.all(np.isnan(df[b, L:]))
        assert np.array_equal(n.target[b, :L + 1], w.target[b, :L + 1])
    assert np.array_equal(n.tokens, w.tokens)


def test_full_size_headline_shapes():
    w = make("c3", 0)
    assert (w.B, w.D, w.V) == (64, 7, 128256) and w.dtype == "bf16"
    assert w.target.nbytes == 131_334_144 and w.draft.nbytes == 114_917_376


def test_gumbel_draft_sampler_distribution():
    """The draft-token construction draws from softmax(l / T) (chi-square vs scipy softmax)."""
    rng = np.random.default_rng(7)
    row = rng.standard_normal(6).astype(np.float32)
    T = 0.7
    n = 60000
    counts = np.bincount([_gumbel_argmax(row, T, rng) for _ in range(n)], minlength=6)
    p = scipy.special.softmax(row.astype(np.float64) / T)
    assert scipy.stats.chisquare(counts, n * p).pvalue > 1e-3

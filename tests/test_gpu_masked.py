"""GPU parity with masked tokens: logits of -inf (the usual mask of top-k or top-p filtering and
of grammar constraints) carry probability 0. Target and draft rows are masked to different
supports, so draft tokens can fall outside the target's support (p(x) = 0: a certain rejection
whose residual max(0, p - q) lives on the target's support); whole 32 KB chunks are masked; the
most extreme case keeps one token per row (one-hot distributions). Draft tokens are redrawn from
the masked draft distributions. bf16 and fp32 logits, sampled and greedy sequences."""
import numpy as np
import pytest

from oracle import verify_workload
from workloads import make

pytestmark = pytest.mark.gpu

from tests import gpu_util as G  # noqa: E402

BF16_NEG_INF = np.uint16(0xFF80)


def _keep_top(vals, k, rng, extra):
    """Mask every row of vals [..., V] (fp32) to its k largest logits plus a random fraction
    `extra` of the others (so that supports of target and draft rows differ); returns a boolean
    keep mask."""
    V = vals.shape[-1]
    k = min(k, V)
    top = np.argpartition(-vals, k - 1, axis=-1)[..., :k]
    keep = np.zeros(vals.shape, bool)
    np.put_along_axis(keep, top, True, axis=-1)
    keep |= rng.random(vals.shape) < extra
    return keep


def _masked_workload(cfg, seed, k, greedy_every=0, extra=0.01):
    w = make(cfg, seed, B=16, V=20011)
    rng = np.random.default_rng([seed, k])
    tv, dv = w.target_f32(), w.draft_f32()
    kt, kd = _keep_top(tv, k, rng, extra), _keep_top(dv, k, rng, extra)
    if w.dtype == "bf16":
        w.target[~kt] = BF16_NEG_INF
        w.draft[~kd] = BF16_NEG_INF
    else:
        w.target[~kt] = -np.inf
        w.draft[~kd] = -np.inf
    if greedy_every:
        w.temperature[::greedy_every] = 0.0
    d = w.draft_f32()
    for b in range(w.B):
        T = float(w.temperature[b])
        for i in range(w.D):
            row = d[b, i].astype(np.float64)
            if T == 0.0:
                w.tokens[b, i] = int(np.argmax(row))
            else:
                g = row / T - np.log(rng.standard_exponential(row.shape[0]))
                w.tokens[b, i] = int(np.argmax(g))
    return w


@pytest.mark.parametrize("cfg", ["c3", "c2"])
@pytest.mark.parametrize("k", [1, 40, 3000])
def test_masked_logits_match_the_oracle(cfg, k):
    for seed in range(3):
        w = _masked_workload(cfg, 70 + seed, k, greedy_every=4)
        ref = verify_workload(w)
        al, toks = G.run(w)
        G.compare(ref, al, toks, f"{cfg} top-{k} seed {seed}")
        assert np.all(al >= 1)


def test_masked_one_hot_rows_are_deterministic():
    """Top-1 masks: every distribution is one-hot, so every outcome is forced (a draft token
    equal to the target's only token is accepted, any other is rejected and the residual is the
    target's token)."""
    w = _masked_workload("c3", 80, 1, extra=0.0)
    ref = verify_workload(w)
    al, toks = G.run(w)
    G.compare(ref, al, toks, "one-hot")
    t = w.target_f32()
    for b in range(w.B):
        j = al[b] - 1
        assert toks[b, j] == int(np.argmax(t[b, j]))

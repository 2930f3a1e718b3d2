"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Bar: accept lengths and tokens bit-exact on every row the oracle does not flag; flagged rows
(a uniform within 1e-5 of an accept boundary, or u*Z within 1e-5 of the chosen bin's width from
its edges) are excused and counted; greedy rows bit-exact; per-row statistics and p(x), q(x)
within 1e-5 relative (1e-5 absolute on their logarithms)."""
import numpy as np
import pytest
import torch

from oracle import verify, verify_workload
from workloads import make

pytestmark = pytest.mark.gpu


from tests import gpu_util as G  # noqa: E402

# seeds per workload: 2000 / 1024 / 1024 / 2048 / 2048 / 2048 rows
SEEDS = dict(c1=2000, c2=64, c3=16, c4=8, c5=4, mtp=2)


def _parity(cfg, seeds, **kw):
    flagged = mism = rows = 0
    measure = 0.0
    for seed in range(seeds):
        w = make(cfg, seed, **kw)
        ref = verify_workload(w)
        al, toks = G.run(w)
        f, m = G.compare(ref, al, toks, f"{cfg} seed {seed}")
        flagged += f
        mism += m
        rows += w.B
        measure += float(ref.flag_measure.sum())
    print(f"{cfg}: rows={rows} flagged={flagged} (mismatched among them {mism}) "
          f"E[flags/row]={measure / rows:.2e}", flush=True)
    G.check_flag_rate(flagged, measure, rows, cfg)
    return flagged, mism


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4", "c5", "mtp"])
def test_parity_full_size(cfg):
    _parity(cfg, SEEDS[cfg])


def _close_log(a, b, tol=1e-5):
    """Element by element: |a - b| <= tol * max(1, |b|) wherever the oracle computed b."""
    m = ~np.isnan(b)
    assert np.all(~np.isnan(a[m]))
    d = np.abs(a[m].astype(np.float64) - b[m])
    bound = tol * np.maximum(1.0, np.abs(b[m]))
    assert np.all(d <= bound), float(np.max(d / bound))


@pytest.mark.parametrize("cfg,kw", [("c2", {}), ("c3", {}), ("c5", dict(B=64)),
                                    ("c4", dict(B=64))])
def test_row_statistics_and_ratios(cfg, kw):
    w = make(cfg, 1, **kw)
    ref = verify_workload(w)
    al, toks, stats, argm, lpq = G.run(w, debug=True)
    D = w.D
    # row maxima of logits/T and ln sum exp, where the oracle computed them
    _close_log(stats[:, :D + 1, 0], ref.row_max_t)
    _close_log(stats[:, :D + 1, 1], ref.row_logsum_t)
    _close_log(stats[:, D + 1:, 0], ref.row_max_d)
    _close_log(stats[:, D + 1:, 1], ref.row_logsum_d)
    # log p(x), log q(x) at the performed tests: within 1e-5 => p, q within 1e-5 relative
    m = ~np.isnan(ref.logp_x)
    assert np.all(np.abs(lpq[..., 0][m] - ref.logp_x[m]) < 1e-5)
    assert np.all(np.abs(lpq[..., 1][m] - ref.logq_x[m]) < 1e-5)
    g = ref.greedy_argmax >= 0
    assert np.array_equal(argm[g], ref.greedy_argmax[g])


def test_greedy_rows_bit_exact():
    for seed in range(4):
        w = make("c4", 100 + seed)
        ref = verify_workload(w)
        al, toks = G.run(w)
        g = w.temperature == 0
        assert np.array_equal(al[g], ref.accept_len[g])
        assert np.array_equal(toks[g], ref.tokens[g])


def test_equal_draft_accepts_all_on_gpu():
    w = make("c3", 3, B=32, V=20011)
    w.draft[:] = w.target[:, :w.D]
    rng = np.random.default_rng(1)
    w.lens = rng.integers(0, w.D + 1, w.B).astype(np.int32)
    w.lens_given = True
    al, toks = G.run(w)
    assert np.array_equal(al, w.lens + 1)
    ref = verify_workload(w)
    G.compare(ref, al, toks, "equal draft")


def test_nan_padding_is_never_read():
    w = make("c5", 7, B=128, pad="nan")
    ref = verify_workload(w)
    al, toks = G.run(w)
    G.compare(ref, al, toks, "nan padding")


def test_repeat_calls_are_bit_identical():
    w = make("c3", 2)
    a = G.run(w)
    b = G.run(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("V", [1, 7, 1001, 16383, 16385, 40000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_vocab_sizes(V, dtype):
    cfg = "c2" if dtype == "f32" else "c3"
    for seed in range(3):
        w = make(cfg, 50 + seed, B=24, V=V)
        ref = verify_workload(w)
        al, toks = G.run(w)
        G.compare(ref, al, toks, f"{dtype} V={V}")


@pytest.mark.parametrize("D", [0, 1, 2, 9])
def test_draft_lengths(D):
    w = make("c5", 9, B=40, V=3001, D=D)
    ref = verify_workload(w)
    al, toks = G.run(w)
    G.compare(ref, al, toks, f"D={D}")


def test_zero_length_drafts_and_single_sequence():
    w = make("c3", 4, B=1, V=128256)
    w.lens = np.zeros(1, np.int32)
    w.lens_given = True
    ref = verify_workload(w)
    al, toks = G.run(w)
    assert al[0] == 1
    G.compare(ref, al, toks, "L=0")


def test_invalid_rows_marked_on_gpu():
    w = make("c3", 5, B=8, V=3000)
    w.tokens[0, 2] = w.V
    w.tokens[1, 0] = -5
    w.lens = np.full(8, w.D, np.int32)
    w.lens[2] = w.D + 1
    w.lens[3] = -1
    w.lens_given = True
    w.temperature[4] = np.nan
    w.temperature[5] = -1.0
    w.temperature[6] = np.inf
    ref = verify_workload(w)
    al, toks = G.run(w)
    assert np.all(al[:7] == 0) and np.all(toks[:7] == -1)
    assert al[7] >= 1
    G.compare(ref, al, toks, "invalid rows")


def test_caller_workspace_matches_library_workspace():
    import sampling_spec_verify_02_amd as sv
    w = make("c5", 11, B=96)
    # a workspace needs no initialisation: start from arbitrary bytes
    g = torch.Generator().manual_seed(5)
    n = sv.workspace_bytes(w.B, w.D, w.V)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to("cuda:0")
    a = G.run(w)
    b = G.run(w, workspace=ws)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_lossless_chi_square_on_gpu():
    import scipy.special
    import scipy.stats
    V, D, n = 8, 2, 1_000_000
    rng = np.random.default_rng(123)
    tgt = (rng.standard_normal((D + 1, V)) * 1.3).astype(np.float32)
    drf = (tgt[:D] + rng.standard_normal((D, V)) * 1.1).astype(np.float32)
    q = scipy.special.softmax(drf.astype(np.float64), axis=-1)
    toks = np.stack([rng.choice(V, size=n, p=q[i]) for i in range(D)], axis=1).astype(np.int32)
    u = rng.random((n, D + 1), dtype=np.float32)
    dev = G.device()
    import sampling_spec_verify_02_amd as sv
    T = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(tgt, (n, D + 1, V)))).to(dev)
    Dd = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(drf, (n, D, V)))).to(dev)
    al, out = sv.spec_verify(T, Dd, torch.from_numpy(toks).to(dev), None,
                             torch.from_numpy(u).to(dev), 1.0)
    torch.cuda.synchronize()
    al, out = al.cpu().numpy(), out.cpu().numpy()
    p = scipy.special.softmax(tgt.astype(np.float64), axis=-1)
    for j in range(D + 1):
        sel = al > j
        counts = np.bincount(out[sel, j], minlength=V)
        assert scipy.stats.chisquare(counts, sel.sum() * p[j]).pvalue > 1e-3
    # and the same rows agree with the oracle exactly
    k = 20000
    ref = verify(np.broadcast_to(tgt, (k, D + 1, V)), np.broadcast_to(drf, (k, D, V)),
                 toks[:k], None, u[:k], np.ones(k, np.float32))
    ok = ~ref.flagged
    assert np.array_equal(al[:k][ok], ref.accept_len[ok])
    assert np.array_equal(out[:k][ok], ref.tokens[ok])


def test_workspace_reuse_across_batch_sizes():
    """One workspace serves calls of different batch sizes in turn: nothing a call leaves in it
    may leak into the next call's results."""
    import sampling_spec_verify_02_amd as sv
    ws = torch.zeros(sv.workspace_bytes(300, 7, 129280), dtype=torch.uint8, device="cuda:0")
    for B, seed in ((40, 1), (300, 2), (17, 3), (300, 4)):
        w = make("c5", 20 + seed, B=B)
        ref = verify_workload(w)
        for wsp in (None, ws):
            al, toks = G.run(w, workspace=wsp)
            G.compare(ref, al, toks, f"B={B} caller_ws={wsp is not None}")


def test_bf16_logits_beyond_the_packed_max_range():
    """bf16 logits of magnitude 2^121 and above sit on fp16's inf / NaN bit patterns, where the
    packed row maximum does not order them; chunks holding them are redone with exact maxima.
    Sampled rows (T = 1 and 0.7) get such values at seeded places, including rows that decide
    the accept tests and the final draw."""
    w = make("c3", 3, B=16, V=20011)
    rng = np.random.default_rng(77)
    # bf16 bit patterns: +2^121 (fp16 +inf), +2^122 (fp16 signalling NaN), -2^122, 1.5 * 2^125
    # (fp16 quiet NaN), -1.5 * 2^125
    # Target rows of sequences 0-7 and draft rows of 8-15 only: where both p(x) and q(x) lie
    # some 1e36 below their rows' maxima, log p(x) - log q(x) is lost to cancellation on both
    # sides and no answer is defined.
    huge = np.array([0x7C00, 0x7C80, 0xFC80, 0x7E40, 0xFE40], np.uint16)
    for arr, rows, seqs in ((w.target, w.D + 1, range(0, 8)), (w.draft, w.D, range(8, 16))):
        for _ in range(12):
            b, r, v = rng.choice(list(seqs)), rng.integers(rows), rng.integers(w.V)
            arr[b, r, v] = huge[rng.integers(huge.size)]
    w.temperature[::2] = 0.7
    ref = verify_workload(w)
    al, toks = G.run(w)
    G.compare(ref, al, toks, "huge bf16 logits")


def test_maximum_draft_length():
    """D = 31, the largest the boundary accepts: 63 rows per sequence, one lane each in the
    outcome."""
    w = make("c5", 12, B=24, V=5003, D=31)
    ref = verify_workload(w)
    al, toks = G.run(w)
    G.compare(ref, al, toks, "D=31")


@pytest.mark.parametrize("dtype,V", [("bf16", 300007), ("f32", 200003)])
def test_large_vocabularies(dtype, V):
    """More than eight 32 KB chunks per row: the outcome merges the chunk partials in several
    batches."""
    w = make("c3" if dtype == "bf16" else "c2", 13, B=6, V=V)
    ref = verify_workload(w)
    al, toks = G.run(w)
    G.compare(ref, al, toks, f"{dtype} V={V}")


@pytest.mark.parametrize("T", [1e-3, 0.05, 10.0, 1000.0])
def test_temperature_extremes(T):
    """Near-greedy and near-uniform sampling: exponent ranges of the fp32 row sums and of the
    fp64 final-draw weights far from the headline's."""
    w = make("c3", 14, B=16, V=20011)
    w.temperature[:] = np.float32(T)
    ref = verify_workload(w)
    al, toks = G.run(w)
    G.compare(ref, al, toks, f"T={T}")


def test_concurrent_calls_on_two_streams():
    """Two streams, each with its own library workspace, run interleaved calls on different
    batches (one with the in-kernel pick, one with the outcome and pick kernels) without host
    synchronisation between them; every result matches the oracle."""
    import sampling_spec_verify_02_amd as sv
    dev = G.device()
    works = [make("c3", 60, B=32, V=30011), make("c5", 61, B=300)]
    refs = [verify_workload(w) for w in works]
    args = [G.to_dev(w, dev) for w in works]
    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    outs = [[], []]
    torch.cuda.synchronize()
    for rep in range(3):
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                a = args[i]
                outs[i].append(sv.spec_verify(a["target"], a["draft"], a["tokens"], a["lens"],
                                              a["uniforms"], a["temperature"]))
    torch.cuda.synchronize()
    for i in (0, 1):
        for al, toks in outs[i]:
            G.compare(refs[i], al.cpu().numpy(), toks.cpu().numpy(), f"stream {i}")

"""GPU parity of threshold acceptance (spec_verify_threshold through the C ABI) against the fp64
oracle: accept lengths and tokens bit-exact on every row the oracle does not flag, at the
workloads' full sizes, at the limits tau = 0 and tau = 1, with NaN in every padded row, and
without any draft logits on the device."""
import numpy as np
import pytest
import torch

import sampling_spec_verify_02_amd as sv
from oracle import verify_threshold_workload, verify_workload
from workloads import make

pytestmark = pytest.mark.gpu

from tests import gpu_util as G  # noqa: E402


def run_threshold(w, tau):
    t = G.to_dev(w)
    al, toks = sv.spec_verify_threshold(t["target"], t["tokens"], t["lens"], t["uniforms"],
                                        t["temperature"], tau)
    torch.cuda.synchronize()
    return al.cpu().numpy(), toks.cpu().numpy()


def _check(w, tau, label):
    ref = verify_threshold_workload(w, tau)
    al, toks = run_threshold(w, tau)
    G.compare(ref, al, toks, label)
    return ref, al


@pytest.mark.parametrize("cfg,seeds,tau", [("c3", 4, 1e-3), ("c3", 2, 0.05), ("c2", 4, 1e-2),
                                           ("c4", 2, 1e-2), ("c5", 1, 1e-3), ("mtp", 1, 0.05)])
def test_threshold_parity_full_size(cfg, seeds, tau):
    """Parity at full size; the prefix tests' window measure (the draft token's chance of a
    prefix score within 1e-5 per term of ln tau) and the final draws' give the expected number
    of flagged rows, gated like the standard rule's."""
    rows = flagged = 0
    measure = 0.0
    for seed in range(seeds):
        ref, al = _check(make(cfg, 40 + seed), tau, f"{cfg} seed {seed} tau={tau}")
        rows += al.size
        flagged += int(ref.flagged.sum())
        measure += float(ref.flag_measure.sum())
    print(f"{cfg} tau={tau}: rows={rows} flagged={flagged} E[flags/row]={measure / rows:.2e}",
          flush=True)
    G.check_flag_rate(flagged, measure, rows, f"{cfg} tau={tau}")


def test_threshold_limits():
    w = make("c3", 9, B=32, V=20011)
    ref, al = _check(w, 0.0, "tau=0")
    assert np.array_equal(al, w.lens + 1)
    ref, al = _check(w, 1.0, "tau=1")
    assert np.all(al == 1)


def test_threshold_greedy_rows_match_standard_verify():
    w = make("c4", 11, B=128)
    al, toks = run_threshold(w, 0.01)
    ref = verify_workload(w)
    g = w.temperature == 0
    assert np.array_equal(al[g], ref.accept_len[g]) and np.array_equal(toks[g], ref.tokens[g])


def test_threshold_never_reads_padding_or_drafts():
    w = make("c5", 12, B=128, pad="nan")
    w.draft[:] = np.uint16(0x7FC0)           # never passed to the device anyway
    _check(w, 1e-3, "nan padding")


@pytest.mark.parametrize("D", [0, 1, 31])
def test_threshold_draft_lengths(D):
    w = make("c5", 13, B=40, V=3001, D=D)
    _check(w, 1e-4, f"D={D}")


def test_threshold_batches_beyond_one_grid_slice():
    """70,000 sequences: the row grid is launched in three slices of sequences and the item grid
    in two; every slice must see its own sequences' partials."""
    rng = np.random.default_rng(21)
    B, D, V = 70000, 2, 40
    tgt = (rng.standard_normal((B, D + 1, V)) * 1.5).astype(np.float32)
    toks = rng.integers(0, V, (B, D)).astype(np.int32)
    u = rng.random((B, D + 1), dtype=np.float32)
    T = np.ones(B, np.float32)
    from oracle import verify_threshold
    ref = verify_threshold(tgt, toks, None, u, T, 0.05)
    dev = G.device()
    al, out = sv.spec_verify_threshold(torch.from_numpy(tgt).to(dev), torch.from_numpy(toks).to(dev),
                                       None, torch.from_numpy(u).to(dev),
                                       torch.from_numpy(T).to(dev), 0.05)
    torch.cuda.synchronize()
    G.compare(ref, al.cpu().numpy(), out.cpu().numpy(), "B=70000")


@pytest.mark.parametrize("T", [1e-3, 0.05, 10.0, 1000.0])
def test_threshold_temperature_extremes(T):
    """Near-greedy and near-uniform target distributions: prefix log-scores far from the
    headline's range."""
    w = make("c3", 15, B=16, V=20011)
    w.temperature[:] = np.float32(T)
    for tau in (1e-6, 0.3):
        _check(w, tau, f"T={T} tau={tau}")

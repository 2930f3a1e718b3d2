"""Staged row launches (spec_verify_row_stages): after the first launch, the rows past a
sequence's first rejection among the positions already read are not read. Poisoning exactly
those rows with NaN must leave every output equal to the oracle's on the clean inputs."""
import ctypes

import numpy as np
import pytest
import torch

import sampling_spec_verify_02_amd as sv
from oracle import verify_workload
from sampling_spec_verify_02_amd import _lib
from workloads import make

pytestmark = pytest.mark.gpu

from tests import gpu_util as G  # noqa: E402


def _cuts(w):
    c = (ctypes.c_int * 8)()
    n = _lib.lib().spec_verify_row_stages(1 if w.dtype == "bf16" else 0, w.B, w.D, w.V, c, 8)
    assert n >= 1
    return [c[i] for i in range(n + 1)]


# c3: one cut at 2; c4: one cut at 2 of four positions; mtp: one cut at 1; c5 at B=160 (620 MB
# of rows, ragged lengths): two cuts, at 1 and 3; c2's generator at B=32 D=7 V=128256: fp32 rows
# (246 MB), one cut at 2
@pytest.mark.parametrize("cfg,kw", [("c3", {}), ("c4", {}), ("mtp", dict(B=512)),
                                    ("c5", dict(B=160)), ("c2", dict(B=32, D=7, V=128256))])
def test_rows_past_a_known_rejection_are_not_read(cfg, kw):
    w = make(cfg, 41, **kw)
    cuts = _cuts(w)
    print(f"workload {cfg} B={w.B} D={w.D} V={w.V} stages {cuts}", flush=True)
    assert len(cuts) > 2, "the workload should be staged"
    ref = verify_workload(w)
    lens = w.lens if w.lens_given else np.full(w.B, w.D)
    nan = np.uint16(0x7fc0) if w.dtype == "bf16" else np.float32(np.nan)
    poisoned = 0
    for b in range(w.B):
        j = int(ref.accept_len[b]) - 1
        if j >= int(lens[b]) or ref.flagged[b]:
            continue                            # bonus draw or excused: every row may be read
        # the first cut above j: launches from there on skip the rows past j
        stop = next(c for c in cuts[1:] if c > j)
        if stop >= cuts[-1]:
            continue
        for p in range(stop, w.D + 1):
            w.target[b, p, :] = nan
            if p < w.D:
                w.draft[b, p, :] = nan
            poisoned += 1
    assert poisoned > 0
    al, toks = G.run(w)
    G.compare(ref, al, toks, f"{cfg} poisoned")
    assert np.array_equal(al[~ref.flagged], ref.accept_len[~ref.flagged])


def test_staged_batches_beyond_one_grid_slice():
    """40,000 sequences, D = 3, V = 256 bf16 (143 MB of rows): staged row launches, each in two
    slices of sequences, the decision kernel over the whole batch between them, and item and
    outcome grids of more than one round. Drafts close to the target, so that many sequences
    reach the second launch."""
    from oracle import verify
    from workloads.gen import bf16_decode, bf16_round
    rng = np.random.default_rng(22)
    B, D, V = 40000, 3, 256
    tgt32 = (rng.standard_normal((B, D + 1, V)) * 2.0).astype(np.float32)
    drf32 = tgt32[:, :D] + (rng.standard_normal((B, D, V)) * 0.3).astype(np.float32)
    tgt, drf = bf16_round(tgt32), bf16_round(drf32)
    toks = rng.integers(0, V, (B, D)).astype(np.int32)
    u = rng.random((B, D + 1), dtype=np.float32)
    T = np.ones(B, np.float32)
    c = (ctypes.c_int * 8)()
    n = _lib.lib().spec_verify_row_stages(1, B, D, V, c, 8)
    cuts = [c[i] for i in range(n + 1)]
    print(f"B={B} D={D} V={V} bf16 stages {cuts}", flush=True)
    assert len(cuts) > 2, "the batch should be staged"
    ref = verify(bf16_decode(tgt), bf16_decode(drf), toks, None, u, T)
    assert np.mean(ref.accept_len >= 3) > 0.1      # the second launch has rows to read
    dev = G.device()
    al, out = sv.spec_verify(G.logits_to_dev(tgt, "bf16", dev), G.logits_to_dev(drf, "bf16", dev),
                             torch.from_numpy(toks).to(dev), None, torch.from_numpy(u).to(dev),
                             torch.from_numpy(T).to(dev))
    torch.cuda.synchronize()
    G.compare(ref, al.cpu().numpy(), out.cpu().numpy(), "B=40000 staged")

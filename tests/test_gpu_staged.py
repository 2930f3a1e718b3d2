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
# of rows, ragged lengths): two cuts, at 1 and 3
@pytest.mark.parametrize("cfg,kw", [("c3", {}), ("c4", {}), ("mtp", dict(B=512)),
                                    ("c5", dict(B=160))])
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

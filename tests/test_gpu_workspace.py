"""The library-owned workspace of the plain entry points: growth in stream order (a small call,
then larger ones on the same stream with no host synchronisation between them, each checked
against the oracle), spec_verify_release followed by a fresh allocation, and the refusal to grow
under graph capture (SV_ENOMEM, nothing enqueued, the capture still valid)."""
import numpy as np
import pytest
import torch

import sampling_spec_verify_02_amd as sv
from oracle import verify_workload
from sampling_spec_verify_02_amd import _lib
from workloads import make

pytestmark = pytest.mark.gpu

from tests import gpu_util as G  # noqa: E402


def _launch(w, t):
    return sv.spec_verify(t["target"], t["draft"], t["tokens"], t["lens"], t["uniforms"],
                          t["temperature"])


def test_growth_is_stream_ordered_and_release_reallocates():
    dev = G.device()
    s = torch.cuda.Stream(dev)
    loads = [make("c1", 3), make("c2", 4, B=6), make("c3", 5, B=12, V=50021)]
    for w in loads:                   # each needs a larger workspace than the one before
        print(f"workload {w.name} B={w.B} D={w.D} V={w.V} ws={sv.workspace_bytes(w.B, w.D, w.V)}",
              flush=True)
    sizes = [sv.workspace_bytes(w.B, w.D, w.V) for w in loads]
    assert sizes == sorted(sizes) and len(set(sizes)) == len(sizes)
    tensors = [G.to_dev(w, dev) for w in loads]
    torch.cuda.synchronize()
    outs = []
    with torch.cuda.stream(s):
        for w, t in zip(loads, tensors):   # no synchronisation between the calls
            outs.append(_launch(w, t))
    s.synchronize()
    for w, (al, toks) in zip(loads, outs):
        G.compare(verify_workload(w), al.cpu().numpy(), toks.cpu().numpy(), w.name)

    with torch.cuda.stream(s):
        sv.release(s)
        sv.release(s)                 # nothing held: still SV_OK
        al, toks = _launch(loads[2], tensors[2])
    s.synchronize()
    G.compare(verify_workload(loads[2]), al.cpu().numpy(), toks.cpu().numpy(), "after release")
    sv.release(s)
    s.synchronize()


def test_growth_under_capture_is_refused():
    dev = G.device()
    w = make("c2", 6, B=4)
    t = G.to_dev(w, dev)
    s = torch.cuda.Stream(dev)
    sv.release(s)                     # the stream holds no workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(sv.SpecVerifyError) as e:
        with torch.cuda.graph(g, stream=s):
            _launch(w, t)
    assert e.value.code == _lib.SV_ENOMEM
    torch.cuda.synchronize()
    # outside the capture the same call allocates and runs
    with torch.cuda.stream(s):
        al, toks = _launch(w, t)
    s.synchronize()
    G.compare(verify_workload(w), al.cpu().numpy(), toks.cpu().numpy(), "after capture")
    sv.release(s)
    s.synchronize()

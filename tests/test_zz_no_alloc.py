"""The entry point that allocates nothing (spec_verify_noalloc, its workspace the library's fixed
per-GPU scratch) gives the caller-workspace entry point's results: two calls in a row, the second
on a smaller problem (so that it runs over what the first left in the scratch), each checked bit
for bit against spec_verify_ws on the same inputs and against the oracle on unflagged rows."""
import numpy as np
import pytest
import torch

import sampling_spec_verify_02_amd as sv
from oracle import verify_workload
from workloads import make

pytestmark = pytest.mark.gpu

from tests import gpu_util as G  # noqa: E402


def _outputs(w, dev):
    return (torch.full((w.B,), -7, dtype=torch.int32, device=dev),
            torch.full((w.B, w.D + 1), -7, dtype=torch.int32, device=dev))


def test_noalloc_matches_the_caller_workspace_entry_point():
    dev = G.device()
    works = [make("c5", 90), make("c3", 91, B=40, V=50021)]     # 10.3 MB, then a smaller one
    args = [G.to_dev(w, dev) for w in works]
    outs = []
    for w, a in zip(works, args):            # both no-allocation calls first, back to back
        al, toks = _outputs(w, dev)
        sv.spec_verify_noalloc(a["target"], a["draft"], a["tokens"], a["lens"], a["uniforms"],
                               a["temperature"], al, toks)
        outs.append((al, toks))
    torch.cuda.synchronize()
    for w, a, (al, toks) in zip(works, args, outs):
        ws = torch.empty(sv.workspace_bytes(w.B, w.D, w.V), dtype=torch.uint8, device=dev)
        al_w, toks_w = sv.spec_verify(a["target"], a["draft"], a["tokens"], a["lens"],
                                      a["uniforms"], a["temperature"], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(al, al_w) and torch.equal(toks, toks_w)
        G.compare(verify_workload(w), al.cpu().numpy(), toks.cpu().numpy(), f"noalloc {w.name}")


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    dev = G.device()
    w = make("mtp", 92, B=8)
    a = G.to_dev(w, dev)
    B = 4096                                  # 70 MB of workspace at D = 1, V = 129280
    rep = B // w.B
    big = {k: (v.repeat(rep, *([1] * (v.dim() - 1))) if v is not None else v)
           for k, v in a.items()}
    al = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.empty((B, w.D + 1), dtype=torch.int32, device=dev)
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.spec_verify_noalloc(big["target"], big["draft"], big["tokens"], big["lens"],
                               big["uniforms"], big["temperature"], al, toks)
    assert e.value.code == -6

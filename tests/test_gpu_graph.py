"""One serving step captured in a HIP graph and replayed: Saguaro reshaping of the draft rows,
verification with a caller workspace (spec_verify_ws: no allocation, no synchronisation, no
memset inside the call), then the epilogue that moves each sequence's token window by AL. The
step (the reshaping also with a caller workspace) is captured once and replayed three times,
with eager work (restoring the inputs) and synchronisations between the replays; every replay must equal the eager step and, on rows the
oracle does not flag, the oracles' chain (reshape, verify, advance)."""
import numpy as np
import pytest
import torch

import sampling_spec_verify_02_amd as sv
from oracle import advance, verify
from oracle.saguaro import reshape_draft
from workloads import make

pytestmark = pytest.mark.gpu

from tests import gpu_util as G  # noqa: E402


@pytest.mark.parametrize("cfg,kw", [("c5", dict(B=48, V=9001)), ("c3", dict(B=16, V=40009))])
def test_captured_step_replays_match_eager_and_oracle(cfg, kw):
    dev = G.device()
    w = make(cfg, 85, **kw)
    W = 10
    rng = np.random.default_rng(12)
    ids0 = rng.integers(0, 1000, (w.B, W)).astype(np.int32)
    len0 = rng.integers(0, 100, w.B).astype(np.int32)

    lens = w.lens if w.lens_given else None
    shaped = reshape_draft(w.draft, w.dtype, lens, w.temperature, 0.4, 5)
    dec = (shaped.astype(np.uint32) << np.uint32(16)).view(np.float32) if w.dtype == "bf16" \
        else shaped
    ref = verify(w.target_f32(), dec, w.tokens, lens, w.uniforms, w.temperature)
    ref_ids, ref_len = advance(ref.accept_len, ref.tokens, w.D, ids0, len0)
    ok = ~ref.flagged

    t = G.to_dev(w, dev)
    pristine = t["draft"].clone()
    ws = torch.empty(sv.workspace_bytes(w.B, w.D, w.V), dtype=torch.uint8, device=dev)
    sag_ws = torch.empty(sv.saguaro_workspace_bytes(w.B, w.D, w.V), dtype=torch.uint8, device=dev)
    al = torch.empty(w.B, dtype=torch.int32, device=dev)
    toks = torch.empty((w.B, w.D + 1), dtype=torch.int32, device=dev)
    d_ids = torch.empty((w.B, W), dtype=torch.int32, device=dev)
    d_len = torch.empty(w.B, dtype=torch.int32, device=dev)
    h_ids, h_len = torch.from_numpy(ids0).to(dev), torch.from_numpy(len0).to(dev)

    def restore():                    # eager work between replays
        t["draft"].copy_(pristine)
        d_ids.copy_(h_ids)
        d_len.copy_(h_len)
        al.fill_(-7)
        toks.fill_(-7)

    def step():
        sv.spec_verify_saguaro_reshape(t["draft"], t["lens"], t["temperature"], 0.4, 5,
                                       workspace=sag_ws)
        sv.spec_verify(t["target"], t["draft"], t["tokens"], t["lens"], t["uniforms"],
                       t["temperature"], out_accept_len=al, out_tokens=toks, workspace=ws)
        sv.spec_verify_advance(al, toks, d_ids, d_len)

    def snapshot():
        return tuple(x.cpu().numpy().copy() for x in (al, toks, d_ids, d_len))

    # eager step on a side stream first (warm-up before capture), then its outputs
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        restore()
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    eager = snapshot()
    G.compare(ref, eager[0], eager[1], f"{cfg} eager")

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager step"
        G.compare(ref, got[0], got[1], f"{cfg} replay {rep}")
        assert np.array_equal(got[2][ok], ref_ids[ok]) and np.array_equal(got[3][ok], ref_len[ok])

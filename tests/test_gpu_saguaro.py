"""GPU parity of Saguaro draft reshaping (spec_verify_saguaro_reshape through the C ABI) against
the CPU oracle: the reshaped logits bit-exact for bf16 and fp32 rows, every k, vocabularies
smaller than a workgroup and with ties, greedy, invalid and ragged sequences left alone; then
reshaping followed by verification on the GPU against the oracle's reshaping and verification."""
import numpy as np
import pytest
import torch

import sampling_spec_verify_02_amd as sv
from oracle import verify
from oracle.saguaro import reshape_draft
from workloads import make

pytestmark = pytest.mark.gpu

from tests import gpu_util as G  # noqa: E402


def _reshape_on_gpu(w, factor, k):
    d = G.logits_to_dev(w.draft, w.dtype, G.device())
    lens = torch.from_numpy(w.lens).to(G.device()) if w.lens_given else None
    sv.spec_verify_saguaro_reshape(d, lens, torch.from_numpy(w.temperature).to(G.device()),
                                   factor, k)
    torch.cuda.synchronize()
    out = d.cpu()
    return out.view(torch.int16).numpy().view(np.uint16) if w.dtype == "bf16" else out.numpy()


@pytest.mark.parametrize("cfg,kw,factor,k", [
    ("c3", dict(B=24), 0.5, 5), ("c3", dict(B=8, V=1000), 0.05, 8), ("c3", dict(B=8, V=7), 0.3, 5),
    ("c2", dict(B=8), 0.5, 1), ("c2", dict(B=6, V=100), 0.9, 8), ("c4", dict(B=40), 0.25, 5),
    ("c5", dict(B=48), 0.5, 5),
    # rows that are not 16-byte multiples (element loads), rows of many chunks with a ragged
    # last chunk, a chunk smaller than k
    ("c3", dict(B=6, V=1001), 0.5, 5), ("c3", dict(B=4, V=200003), 0.3, 8),
    ("c2", dict(B=4, V=70001), 0.7, 4), ("c3", dict(B=5, V=2 * 16384 + 3), 0.5, 8),
    ("c2", dict(B=5, V=3 * 8192 + 5), 0.5, 8),
    # merge slot counts that spread 2 and 3 per lane (96 and 160 slots; k = 8 leaves lane groups
    # without candidates)
    ("c2", dict(B=4, V=5 * 2048 + 7), 0.5, 8), ("c3", dict(B=4, V=9 * 4096 + 1), 0.5, 5)])
def test_reshape_matches_oracle(cfg, kw, factor, k):
    w = make(cfg, 70, **kw)
    if cfg == "c5":
        w.lens[5] = w.D + 3            # invalid length: the sequence is left alone
    got = _reshape_on_gpu(w, factor, k)
    want = reshape_draft(w.draft, w.dtype, w.lens if w.lens_given else None, w.temperature,
                         factor, k)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_reshape_top_k_across_chunk_boundaries():
    """The row's top k spread over several chunks, with ties across chunk boundaries and
    inside one chunk (lowest indices win), bf16 and fp32."""
    for cfg, ce in (("c3", 16384), ("c2", 8192)):
        w = make(cfg, 74, B=3, V=4 * ce + 17)
        rows = w.draft.reshape(-1, w.V)
        hi = np.float32(40.0)
        val = (np.uint16(np.float32(hi).view(np.uint32) >> 16) if w.dtype == "bf16" else hi)
        for r in range(rows.shape[0]):
            for pos in (ce - 1, ce, 2 * ce + 5, 4 * ce + 16, 7, 3 * ce - 1):
                rows[r, pos] = val
        got = _reshape_on_gpu(w, 0.5, 5)
        want = reshape_draft(w.draft, w.dtype, None, w.temperature, 0.5, 5)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), cfg


def test_reshape_caller_workspace_is_reusable():
    """spec_verify_saguaro_reshape_ws: one workspace, filled with garbage first, serves calls of
    different shapes in a row on one stream, matching the oracle each time."""
    dev = G.device()
    loads = [make("c3", 75, B=6, V=40000), make("c2", 76, B=8, V=9000),
             make("c5", 77, B=12, V=20011)]
    size = max(sv.saguaro_workspace_bytes(w.B, w.D, w.V) for w in loads)
    ws = torch.randint(0, 256, (size,), dtype=torch.uint8, device=dev)
    for rep in range(2):
        outs = []
        for w in loads:
            d = G.logits_to_dev(w.draft, w.dtype, dev)
            lens = torch.from_numpy(w.lens).to(dev) if w.lens_given else None
            sv.spec_verify_saguaro_reshape(d, lens, torch.from_numpy(w.temperature).to(dev),
                                           0.5, 5, workspace=ws)
            outs.append(d)
        torch.cuda.synchronize()
        for w, d in zip(loads, outs):
            got = d.cpu()
            got = got.view(torch.int16).numpy().view(np.uint16) if w.dtype == "bf16" \
                else got.numpy()
            want = reshape_draft(w.draft, w.dtype, w.lens if w.lens_given else None,
                                 w.temperature, 0.5, 5)
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (rep, w.name)


def test_reshape_ties_take_lowest_indices():
    rng = np.random.default_rng(3)
    w = make("c2", 71, B=6, V=3000)
    w.draft[:] = rng.integers(-2, 3, w.draft.shape).astype(np.float32)   # thousands of ties
    got = _reshape_on_gpu(w, 0.5, 8)
    want = reshape_draft(w.draft, "f32", None, w.temperature, 0.5, 8)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("cfg,kw", [("c3", dict(B=32, V=20011)), ("c5", dict(B=64, V=9001))])
def test_reshape_then_verify(cfg, kw):
    w = make(cfg, 72, **kw)
    shaped = reshape_draft(w.draft, w.dtype, w.lens if w.lens_given else None, w.temperature,
                           0.3, 5)
    dec = (shaped.astype(np.uint32) << np.uint32(16)).view(np.float32) if w.dtype == "bf16" \
        else shaped
    ref = verify(w.target_f32(), dec, w.tokens, w.lens if w.lens_given else None, w.uniforms,
                 w.temperature)
    t = G.to_dev(w)
    sv.spec_verify_saguaro_reshape(t["draft"], t["lens"], t["temperature"], 0.3, 5)
    al, toks = sv.spec_verify(t["target"], t["draft"], t["tokens"], t["lens"], t["uniforms"],
                              t["temperature"])
    torch.cuda.synchronize()
    G.compare(ref, al.cpu().numpy(), toks.cpu().numpy(), f"{cfg} reshaped")


def test_reshape_verify_advance_loop_on_one_stream():
    """Three steps of a serving loop on one stream with no host synchronisation in between:
    reshape the draft rows, verify, move the token windows; the windows and lengths equal the
    oracles' chain on every sequence no step flagged."""
    from oracle import advance
    dev = G.device()
    B, W = 32, 10
    rng = np.random.default_rng(9)
    ids0 = rng.integers(0, 1000, (B, W)).astype(np.int32)
    d_ids = torch.from_numpy(ids0).to(dev)
    d_len = torch.zeros(B, dtype=torch.int32, device=dev)
    ref_ids, ref_len = ids0, np.zeros(B, np.int32)
    excused = np.zeros(B, bool)
    keep = []
    for step in range(3):
        w = make("c5", 80 + step, B=B, V=6007)
        t = G.to_dev(w, dev)
        sv.spec_verify_saguaro_reshape(t["draft"], t["lens"], t["temperature"], 0.4, 5)
        al, toks = sv.spec_verify(t["target"], t["draft"], t["tokens"], t["lens"],
                                  t["uniforms"], t["temperature"])
        sv.spec_verify_advance(al, toks, d_ids, d_len)
        keep.append((t, al, toks))
        shaped = reshape_draft(w.draft, w.dtype, w.lens, w.temperature, 0.4, 5)
        dec = (shaped.astype(np.uint32) << np.uint32(16)).view(np.float32)
        r = verify(w.target_f32(), dec, w.tokens, w.lens, w.uniforms, w.temperature)
        excused |= r.flagged
        ref_ids, ref_len = advance(r.accept_len, r.tokens, w.D, ref_ids, ref_len)
    torch.cuda.synchronize()
    ok = ~excused
    assert ok.sum() > 0.9 * B
    assert np.array_equal(d_ids.cpu().numpy()[ok], ref_ids[ok])
    assert np.array_equal(d_len.cpu().numpy()[ok], ref_len[ok])


@pytest.mark.parametrize("T", [1e-3, 1000.0])
def test_reshape_temperature_extremes(T):
    """Tiny and huge shifts T ln c (bf16 rounding of the shifted logits included)."""
    w = make("c3", 73, B=8, V=20011)
    w.temperature[:] = np.float32(T)
    got = _reshape_on_gpu(w, 0.5, 5)
    want = reshape_draft(w.draft, w.dtype, None, w.temperature, 0.5, 5)
    assert np.array_equal(got, want)


def test_reshape_batches_beyond_one_grid_slice():
    """70,000 sequences: the unit and merge grids are launched in two slices of sequences; each
    slice must write its own rows and read its own candidate slots."""
    rng = np.random.default_rng(23)
    B, D, V = 70000, 1, 100
    draft = (rng.standard_normal((B, D, V)) * 2.0).astype(np.float32)
    T = np.ones(B, np.float32)
    dev = G.device()
    d = torch.from_numpy(draft).to(dev)
    sv.spec_verify_saguaro_reshape(d, None, torch.from_numpy(T).to(dev), 0.5, 5)
    torch.cuda.synchronize()
    want = reshape_draft(draft, "f32", None, T, 0.5, 5)
    assert np.array_equal(d.cpu().numpy().view(np.uint8), want.view(np.uint8))

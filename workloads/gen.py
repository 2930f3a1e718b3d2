"""Seeded synthetic inputs for the speculative-decoding verification sampler.

This module builds inputs only. It holds none of the verifier's arithmetic
(no softmax, no acceptance test, no residual): both the fp64 oracle and the
HIP path consume what it returns, and neither one's results ever feed back
into it.

Workloads (the method's shapes: B sequences, D draft positions, vocabulary V):

  c1  B=1   D=4  V=1024    fp32  T=1     target ~ N(0, 2^2) iid, draft = target + N(0, 0.5^2)
  c2  B=16  D=4  V=32000   fp32  T=1     Zipf(1.1)+N(0,1) target, draft = target + N(0, 1)
  c3  B=64  D=7  V=128256  bf16  T=1     Zipf target, draft = target + N(0, 1)
  c4  B=256 D=3  V=128256  bf16  half T=0 (greedy), half T=0.7; 10% of sequences have
                                  draft == target bit for bit; others draft = target + N(0, 1.5^2)
  c5  B=512 D=7  V=129280  bf16  T=1     ragged draft lengths L_b ~ U{1..7}, draft noise
                                  sigma_b ~ U[0.25, 2.0] per sequence, unused rows padded
  mtp B=1024 D=1 V=129280  bf16  T=1     single-token (MTP-style) verification of a large decode
                                  batch: Zipf target, draft = target + N(0, 1)

Zipf target (c2..c5): logit(v) = -1.1 * ln(pi(v) + 1) - ln H_{V,1.1} + N(0, 1), where pi is one
seeded permutation of the vocabulary per call (pi(v) = rank of token v) and
H_{V,1.1} = sum_{k=1..V} k^-1.1.

Draft tokens: x_i is a draw from the tempered draft distribution of the *stored* (rounded)
draft logits, made with the Gumbel-max construction x = argmax_v(l_v / T - ln E_v),
E_v ~ Exp(1) iid. Greedy sequences (T=0) take the draft argmax (lowest index on ties).

Uniforms: [B][D+1] fp32 U[0,1): columns 0..D-1 are the accept tests, column D is the one
final-sample uniform of the sequence.

Rounding to bf16 is round-to-nearest-even of the fp32 value. Everything downstream consumes
the rounded values. bf16 arrays are returned as their uint16 bit patterns.

Random streams: every (stream, sequence) pair has its own numpy Generator seeded with
[config id, seed, stream id, sequence], so a sequence's data does not depend on B or on the
order in which sequences are generated.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# stream ids
_S_PERM, _S_TARGET, _S_SEQ, _S_DRAFT, _S_TOKEN, _S_UNIF, _S_BATCH = range(7)

CONFIGS = {
    "c1": dict(cid=1, B=1, D=4, V=1024, dtype="f32"),
    "c2": dict(cid=2, B=16, D=4, V=32000, dtype="f32"),
    "c3": dict(cid=3, B=64, D=7, V=128256, dtype="bf16"),
    "c4": dict(cid=4, B=256, D=3, V=128256, dtype="bf16"),
    "c5": dict(cid=5, B=512, D=7, V=129280, dtype="bf16"),
    "mtp": dict(cid=6, B=1024, D=1, V=129280, dtype="bf16"),
}

BF16_QNAN = np.uint16(0x7FC0)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    B: int
    D: int
    V: int
    dtype: str                 # "f32" or "bf16"
    target: np.ndarray         # [B][D+1][V] float32, or uint16 bf16 bit patterns
    draft: np.ndarray          # [B][D][V]
    tokens: np.ndarray         # [B][D] int32, -1 at padded positions
    lens: np.ndarray           # [B] int32, per-sequence draft length L_b
    lens_given: bool           # False: every L_b == D and the call may pass no length array
    uniforms: np.ndarray       # [B][D+1] float32 in [0, 1)
    temperature: np.ndarray    # [B] float32; 0 => greedy

    def target_f32(self) -> np.ndarray:
        return decode(self.target, self.dtype)

    def draft_f32(self) -> np.ndarray:
        return decode(self.draft, self.dtype)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def _rng(cid: int, seed: int, stream: int, b: int = 0) -> np.random.Generator:
    return np.random.default_rng([cid, seed, stream, b])


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_decode(arr) if dtype == "bf16" else arr


def zipf_base(V: int, perm: np.ndarray) -> np.ndarray:
    """-1.1 ln(rank+1) - ln H_{V,1.1} for each token, rank = perm[token]."""
    k = np.arange(1, V + 1, dtype=np.float64)
    log_h = np.log(np.sum(k ** -1.1))
    return (-1.1 * np.log(perm.astype(np.float64) + 1.0) - log_h).astype(np.float32)


def _gumbel_argmax(row: np.ndarray, T: float, rng: np.random.Generator) -> int:
    e = rng.standard_exponential(row.shape[0])
    return int(np.argmax(row.astype(np.float64) / T - np.log(e)))


def make(config: str, seed: int = 0, *, B: int | None = None, V: int | None = None,
         D: int | None = None, pad: str = "zero", threads: int = 8) -> Workload:
    """Build one seeded workload. B, V and D may be overridden to make smaller instances
    that keep the config's generator (used by CPU tests); pad="nan" fills every padded
    logit with NaN (robustness variant: those rows must never be read)."""
    cfg = CONFIGS[config]
    cid = cfg["cid"]
    B = cfg["B"] if B is None else B
    V = cfg["V"] if V is None else V
    D = cfg["D"] if D is None else D
    dtype = cfg["dtype"]
    assert B >= 1 and V >= 1 and D >= 0 and pad in ("zero", "nan")

    # ---- per-batch choices
    brng = _rng(cid, seed, _S_BATCH)
    temperature = np.ones(B, dtype=np.float32)
    equal = np.zeros(B, dtype=bool)
    if config == "c4":
        order = brng.permutation(B)
        temperature[order[: B // 2]] = 0.0
        temperature[order[B // 2:]] = np.float32(0.7)
        equal[brng.permutation(B)[: (B // 10)]] = True
    lens = np.full(B, D, dtype=np.int32)
    sigma = np.ones(B, dtype=np.float64)
    if config == "c4":
        sigma[:] = 1.5
    if config == "c5":
        for b in range(B):
            r = _rng(cid, seed, _S_SEQ, b)
            lens[b] = r.integers(1, D + 1) if D >= 1 else 0
            sigma[b] = r.uniform(0.25, 2.0)

    if config == "c1":
        base = None
    else:
        perm = _rng(cid, seed, _S_PERM).permutation(V)
        base = zipf_base(V, perm)

    store = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((B, D + 1, V), dtype=store)
    draft = np.empty((B, D, V), dtype=store)
    tokens = np.full((B, D), -1, dtype=np.int32)
    pad_val = (BF16_QNAN if dtype == "bf16" else np.float32(np.nan)) if pad == "nan" else 0

    def one(b: int) -> None:
        tr = _rng(cid, seed, _S_TARGET, b)
        if base is None:
            t32 = (tr.standard_normal((D + 1, V), dtype=np.float32) * np.float32(2.0))
        else:
            t32 = base[None, :] + tr.standard_normal((D + 1, V), dtype=np.float32)
        dr = _rng(cid, seed, _S_DRAFT, b)
        if equal[b]:
            d32 = None
        else:
            s = 0.5 if config == "c1" else sigma[b]
            d32 = t32[:D] + (dr.standard_normal((D, V), dtype=np.float32) * np.float32(s))
        if dtype == "bf16":
            target[b] = bf16_round(t32)
            draft[b] = target[b, :D] if d32 is None else bf16_round(d32)
        else:
            target[b] = t32
            draft[b] = target[b, :D] if d32 is None else d32
        L = int(lens[b])
        target[b, L + 1:] = pad_val
        draft[b, L:] = pad_val
        krng = _rng(cid, seed, _S_TOKEN, b)
        dd = decode(draft[b], dtype)
        T = float(temperature[b])
        for i in range(L):
            tokens[b, i] = int(np.argmax(dd[i])) if T == 0.0 else _gumbel_argmax(dd[i], T, krng)

    if threads > 1 and B > 1:
        with ThreadPoolExecutor(max_workers=min(threads, B)) as ex:
            list(ex.map(one, range(B)))
    else:
        for b in range(B):
            one(b)

    uniforms = _rng(cid, seed, _S_UNIF).random((B, D + 1), dtype=np.float32)
    return Workload(name=config, seed=seed, B=B, D=D, V=V, dtype=dtype, target=target,
                    draft=draft, tokens=tokens, lens=lens, lens_given=(config == "c5"),
                    uniforms=uniforms, temperature=temperature)


def algorithmic_bytes(w: Workload) -> int:
    """Bytes of logits the method must read: every valid row once (target rows 0..L_b,
    draft rows 0..L_b-1; draft rows of greedy sequences are not needed), plus the small
    per-sequence arrays (tokens, lengths, uniforms, temperature, outputs)."""
    rows = 0
    for b in range(w.B):
        L = int(w.lens[b])
        rows += (L + 1) + (0 if w.temperature[b] == 0 else L)
    small = w.B * (w.D * 4 + 4 + (w.D + 1) * 4 + 4 + 4 + (w.D + 1) * 4)
    return rows * w.V * w.elem_bytes + small

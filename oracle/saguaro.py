"""Plain CPU oracle of Saguaro-style draft reshaping.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs this file: only
the tests use it. It shares no code with the HIP library and does not import it.

Source: "Speculative Speculative Decoding - асинхронизируй это" (x0ct.com), the paragraphs on
saguaro sampling: the draft's five most likely tokens get their probabilities artificially
lowered when the draft is generated, so that the residual distribution the target samples from
after a rejection concentrates on those same tokens. The page gives neither the factor nor the
formula.

Reading adopted: the draft is sampled from q' = normalise(q with its top-k tokens multiplied by a
factor c, 0 < c <= 1); in logits, l' = l + T ln c on the row's top-k tokens (ties: lowest index)
and l elsewhere, since softmax(l'/T) is then exactly q'. Verification must use the distribution
the draft was actually sampled from, so the verifier runs unchanged on the reshaped draft
logits, and stays lossless for any c. The arithmetic is fixed for bit-exact parity: c is an fp32
value (the boundary takes it as one), ln c is rounded to fp32, delta = fp32(T * ln c), the new
logit = fp32(l + delta), rounded to bf16 (nearest, ties to even) for bf16 storage. Greedy sequences (T = 0: delta = 0), rows at
positions >= L_b and sequences with an invalid length or temperature are left unchanged.
"""
from __future__ import annotations

import math

import numpy as np


def top_k_indices(row: np.ndarray, k: int) -> np.ndarray:
    """The k largest logits of a row, ties broken by the lowest index (value descending, then
    index ascending)."""
    idx = np.arange(row.shape[0])
    order = np.lexsort((idx, -row.astype(np.float64)))
    return order[:min(k, row.shape[0])]


def _bf16_rne(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def reshape_draft(draft: np.ndarray, dtype: str, lens, temperature: np.ndarray, factor: float,
                  k: int = 5) -> np.ndarray:
    """Return reshaped draft logits in their storage form (uint16 bf16 patterns or float32).

    draft [B][D][V]: uint16 bf16 patterns (dtype "bf16") or float32 values (dtype "f32")."""
    out = np.array(draft, copy=True)
    B, D, V = draft.shape
    if lens is None:
        lens = np.full(B, D, np.int32)
    lnf = np.float32(math.log(float(np.float32(factor))))   # ln of the fp32 factor
    for b in range(B):
        L, T = int(lens[b]), float(temperature[b])
        if not (0 <= L <= D) or not (math.isfinite(T) and T > 0.0):
            continue
        delta = np.float32(np.float32(temperature[b]) * lnf)
        for i in range(L):
            vals = (out[b, i].astype(np.uint32) << np.uint32(16)).view(np.float32) \
                if dtype == "bf16" else out[b, i].astype(np.float32)
            sel = top_k_indices(vals, k)
            new = (vals[sel] + delta).astype(np.float32)
            if dtype == "bf16":
                out[b, i, sel] = _bf16_rne(new)
            else:
                out[b, i, sel] = new
    return out

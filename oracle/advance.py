"""Plain CPU oracle of the device-side epilogue that follows verification.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or runs this file: only
the tests use it. It shares no code with the HIP library and does not import it.

Source: "Accélérer Sonar par la Spéculation" (Perplexity), section "Calendrier MTP pour un
jeton unique": after the accepted length is known, the target's input tokens are shifted and a
kernel writes the newly produced tokens into their slots, so that no GPU-to-CPU synchronisation
is needed before the next step; section "Inférence avec décodage spéculatif": the accepted count
sets each sequence's length for the next run. Section "MTP": the draft's input-token buffer is
the target's shifted by one step, i.e. a window that moves along the token stream.

Reading adopted (the page gives no layout): every sequence b keeps a window of its W most recent
tokens, input_ids[b][0..W-1], oldest first, and a length seq_len[b]. A verification step that
emitted AL tokens (tokens[b][0..AL-1]: the accepted drafts, then the final token) moves the
window AL places towards the newest token and writes the AL tokens into the freed slots at the
end; when AL > W only the last W of them remain. seq_len[b] grows by AL. A sequence whose AL is
outside [1, D + 1] (0 marks a row the verifier rejected as invalid), or whose length is negative
or would pass 2^31 - 1, is left exactly as it was.
"""
from __future__ import annotations

import numpy as np

INT32_MAX = 2 ** 31 - 1


def advance(accept_len, tokens, D, input_ids, seq_len=None):
    """Return (new_input_ids [B][W] int32, new_seq_len [B] int32 or None).

    accept_len [B] int32; tokens [B][D+1] int32 (verifier output); input_ids [B][W] int32;
    seq_len [B] int32 or None. The inputs are not modified."""
    accept_len = np.asarray(accept_len)
    tokens = np.asarray(tokens)
    ids = np.array(input_ids, dtype=np.int32, copy=True)
    lens = None if seq_len is None else np.array(seq_len, dtype=np.int64, copy=True)
    B, W = ids.shape
    for b in range(B):
        a = int(accept_len[b])
        if a < 1 or a > D + 1:
            continue
        if lens is not None and (lens[b] < 0 or lens[b] > INT32_MAX - a):
            continue
        # slide: slot j takes the token that sat a places further on, and the last a slots
        # take the emitted tokens in order
        row = ids[b].copy()
        for j in range(W):
            src = j + a
            ids[b, j] = row[src] if src < W else tokens[b, src - W]
        if lens is not None:
            lens[b] += a
    return ids, (None if lens is None else lens.astype(np.int32))

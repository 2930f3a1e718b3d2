"""Python binding of the verification sampler. Argument marshalling only: every step of the
computation runs in the HIP library; torch supplies device memory and the current stream."""
from __future__ import annotations

import ctypes

import torch

from ._lib import (DTYPE_BF16, DTYPE_F32, SV_MAX_D, SV_OK, SpecVerifyError, lib)

_DT = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _prepare(target, draft, draft_tokens, draft_lens, uniforms, temperature,
             out_accept_len, out_tokens):
    if target.dim() != 3:
        raise ValueError("target_logits must be [B][D+1][V]")
    B, D1, V = target.shape
    D = D1 - 1
    if D > SV_MAX_D:
        raise ValueError(f"D={D} exceeds the supported maximum {SV_MAX_D}")
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("target_logits must be a GPU tensor")
    if target.dtype not in _DT:
        raise TypeError(f"logits dtype must be bfloat16 or float32, got {target.dtype}")
    _check(target, "target_logits", target.dtype, (B, D + 1, V), dev)
    if draft is not None:              # None only for threshold acceptance (no draft logits)
        _check(draft, "draft_logits", target.dtype, (B, D, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, D), dev)
    if draft_lens is not None:
        _check(draft_lens, "draft_lens", torch.int32, (B,), dev)
    _check(uniforms, "uniforms", torch.float32, (B, D + 1), dev)
    if not torch.is_tensor(temperature):
        temperature = torch.full((B,), float(temperature), dtype=torch.float32, device=dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    if out_accept_len is None:
        out_accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
    _check(out_accept_len, "out_accept_len", torch.int32, (B,), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, D + 1), dev)
    return B, D, V, temperature, out_accept_len, out_tokens


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def spec_verify(target_logits, draft_logits, draft_tokens, draft_lens, uniforms, temperature,
                out_accept_len=None, out_tokens=None, workspace=None):
    """Verify a batch on the GPU. Returns (accept_len [B] int32, tokens [B][D+1] int32).

    target_logits [B][D+1][V] and draft_logits [B][D][V]: bfloat16 or float32 (same dtype);
    draft_tokens [B][D] int32; draft_lens [B] int32 or None (all D); uniforms [B][D+1] float32;
    temperature: [B] float32 tensor or a Python float. workspace: optional uint8 GPU tensor of
    at least workspace_bytes(B, D, V) bytes (no initialisation needed); the library's own
    buffer is used otherwise.
    The work is enqueued on torch's current stream; nothing is synchronised."""
    B, D, V, temperature, out_accept_len, out_tokens = _prepare(
        target_logits, draft_logits, draft_tokens, draft_lens, uniforms, temperature,
        out_accept_len, out_tokens)
    L = lib()
    st = _stream(target_logits.device)
    args = (_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(draft_lens),
            _ptr(uniforms), B, D, V, _ptr(temperature), _ptr(out_accept_len), _ptr(out_tokens))
    if workspace is not None:
        rc = L.spec_verify_ws(_DT[target_logits.dtype], *args, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), st)
    elif target_logits.dtype == torch.bfloat16:
        rc = L.spec_verify_bf16(*args, st)
    else:
        rc = L.spec_verify_f32(*args, st)
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify")
    return out_accept_len, out_tokens


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, draft_lens, uniforms,
                        temperature, out_accept_len, out_tokens):
    """spec_verify through the entry point that allocates no device memory (its workspace is the
    library's fixed per-GPU scratch; calls that overlap on one GPU race). The outputs must be
    given. Returns (accept_len, tokens); enqueued on torch's current stream."""
    B, D, V, temperature, out_accept_len, out_tokens = _prepare(
        target_logits, draft_logits, draft_tokens, draft_lens, uniforms, temperature,
        out_accept_len, out_tokens)
    rc = lib().spec_verify_noalloc(_DT[target_logits.dtype], _ptr(target_logits),
                                   _ptr(draft_logits), _ptr(draft_tokens), _ptr(draft_lens),
                                   _ptr(uniforms), B, D, V, _ptr(temperature),
                                   _ptr(out_accept_len), _ptr(out_tokens),
                                   _stream(target_logits.device))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_noalloc")
    return out_accept_len, out_tokens


def spec_verify_threshold(target_logits, draft_tokens, draft_lens, uniforms, temperature, tau,
                          out_accept_len=None, out_tokens=None):
    """Threshold acceptance on the GPU: keep the longest draft prefix whose target probability is
    above tau, then draw one more token from the target at the first position not kept. No draft
    logits are taken. Returns (accept_len [B] int32, tokens [B][D+1] int32); enqueued on torch's
    current stream, nothing is synchronised."""
    B, D, V, temperature, out_accept_len, out_tokens = _prepare(
        target_logits, None, draft_tokens, draft_lens, uniforms, temperature,
        out_accept_len, out_tokens)
    rc = lib().spec_verify_threshold(_DT[target_logits.dtype], _ptr(target_logits),
                                     _ptr(draft_tokens), _ptr(draft_lens), _ptr(uniforms), B, D,
                                     V, _ptr(temperature), float(tau), _ptr(out_accept_len),
                                     _ptr(out_tokens), _stream(target_logits.device))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_threshold")
    return out_accept_len, out_tokens


def spec_verify_debug(target_logits, draft_logits, draft_tokens, draft_lens, uniforms,
                      temperature):
    """spec_verify plus the kernels' per-row statistics: returns (accept_len, tokens,
    row_stats [B][2D+1][2] (max of logits/T, ln sum exp), row_argmax [B][D+1],
    logpq_x [B][D][2] (log p_i(x_i), log q_i(x_i)))."""
    B, D, V, temperature, al, toks = _prepare(target_logits, draft_logits, draft_tokens,
                                              draft_lens, uniforms, temperature, None, None)
    dev = target_logits.device
    stats = torch.empty((B, 2 * D + 1, 2), dtype=torch.float32, device=dev)
    am = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
    lpq = torch.empty((B, max(D, 1), 2), dtype=torch.float32, device=dev)[:, :D]
    rc = lib().spec_verify_debug(_DT[target_logits.dtype], _ptr(target_logits),
                                 _ptr(draft_logits), _ptr(draft_tokens), _ptr(draft_lens),
                                 _ptr(uniforms), B, D, V, _ptr(temperature), _ptr(al),
                                 _ptr(toks), _ptr(stats), _ptr(am), _ptr(lpq),
                                 _stream(dev))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_debug")
    return al, toks, stats, am, lpq


def workspace_bytes(B: int, D: int, V: int) -> int:
    return int(lib().spec_verify_workspace_bytes(B, D, V))


def release(stream=None):
    """Frees the library workspace held for (current device, `stream`) in stream order
    (torch's current stream when None); call it before destroying a stream that used the plain
    entry points."""
    if stream is None:
        stream = torch.cuda.current_stream()
    rc = lib().spec_verify_release(ctypes.c_void_p(stream.cuda_stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_release")


def spec_verify_advance(accept_len, tokens, input_ids, seq_len=None):
    """Epilogue of a verification step, on the GPU: each sequence's window of recent tokens
    input_ids [B][W] int32 moves by its AL and takes the emitted tokens at its end; seq_len [B]
    int32 (optional) grows by AL. accept_len [B] and tokens [B][D+1] are spec_verify's outputs.
    Updates input_ids and seq_len in place on torch's current stream; nothing is synchronised."""
    if tokens.dim() != 2 or input_ids.dim() != 2:
        raise ValueError("tokens must be [B][D+1] and input_ids [B][W]")
    B, D1 = tokens.shape
    dev = tokens.device
    if dev.type != "cuda":
        raise ValueError("tokens must be a GPU tensor")
    _check(accept_len, "accept_len", torch.int32, (B,), dev)
    _check(tokens, "tokens", torch.int32, (B, D1), dev)
    _check(input_ids, "input_ids", torch.int32, (B, input_ids.shape[1]), dev)
    if seq_len is not None:
        _check(seq_len, "seq_len", torch.int32, (B,), dev)
    rc = lib().spec_verify_advance(_ptr(accept_len), _ptr(tokens), B, D1 - 1, _ptr(input_ids),
                                   int(input_ids.shape[1]), _ptr(seq_len), _stream(dev))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_advance")
    return input_ids, seq_len


def saguaro_workspace_bytes(B: int, D: int, V: int) -> int:
    return int(lib().spec_verify_saguaro_workspace_bytes(B, D, V))


def spec_verify_saguaro_reshape(draft_logits, draft_lens, temperature, factor, k=5,
                                workspace=None):
    """Saguaro reshaping of draft logits [B][D][V] (bfloat16 or float32, in place): the top-k
    logits of every needed row move by T ln(factor), so that the row's softmax is q with its
    top k scaled by `factor` and renormalised. draft_lens [B] int32 or None; temperature: [B]
    float32 tensor or a Python float. workspace: optional uint8 GPU tensor of at least
    saguaro_workspace_bytes(B, D, V) bytes (no initialisation needed); the library's own buffer
    is used otherwise. Enqueued on torch's current stream."""
    if draft_logits.dim() != 3:
        raise ValueError("draft_logits must be [B][D][V]")
    B, D, V = draft_logits.shape
    dev = draft_logits.device
    if draft_logits.dtype not in _DT:
        raise TypeError(f"logits dtype must be bfloat16 or float32, got {draft_logits.dtype}")
    _check(draft_logits, "draft_logits", draft_logits.dtype, (B, D, V), dev)
    if draft_lens is not None:
        _check(draft_lens, "draft_lens", torch.int32, (B,), dev)
    if not torch.is_tensor(temperature):
        temperature = torch.full((B,), float(temperature), dtype=torch.float32, device=dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    if workspace is not None:
        rc = lib().spec_verify_saguaro_reshape_ws(
            _DT[draft_logits.dtype], _ptr(draft_logits), _ptr(draft_lens), _ptr(temperature),
            B, D, V, float(factor), int(k), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(dev))
    else:
        rc = lib().spec_verify_saguaro_reshape(_DT[draft_logits.dtype], _ptr(draft_logits),
                                               _ptr(draft_lens), _ptr(temperature), B, D, V,
                                               float(factor), int(k), _stream(dev))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_saguaro_reshape")
    return draft_logits

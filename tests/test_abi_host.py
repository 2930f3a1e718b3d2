"""The C-ABI library loads, exports every symbol include/spec_verify.h declares, and rejects bad
arguments on the host before touching any device."""
import ctypes
import os
import re

import pytest
import torch

from sampling_spec_verify_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(spec_verify\w*)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ("spec_verify_bf16", "spec_verify_f32", "spec_verify_ws",
                 "spec_verify_workspace_bytes", "spec_verify_debug", "spec_verify_strerror",
                 "spec_verify_advance", "spec_verify_threshold", "spec_verify_saguaro_reshape"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_static_queries():
    lib = _lib.lib()
    assert lib.spec_verify_version() >= 100
    assert lib.spec_verify_workspace_bytes(64, 7, 128256) > 0
    assert lib.spec_verify_workspace_bytes(0, 7, 128256) == 0
    assert lib.spec_verify_workspace_bytes(4, -1, 10) == 0
    assert lib.spec_verify_workspace_bytes(4, _lib.SV_MAX_D + 1, 10) == 0
    assert lib.spec_verify_workspace_bytes(4, 2, 0) == 0
    for code in (0, -1, -2, -3, -4, -5, -6, 7):
        assert isinstance(_lib.strerror(code), str)


FAKE = ctypes.c_void_p(4096)      # never dereferenced: every case fails before any launch
NUL = ctypes.c_void_p(0)


def _call(fn, B=2, D=3, V=100, t=FAKE, d=FAKE, tok=FAKE, u=FAKE, temp=FAKE, ol=FAKE, ot=FAKE):
    lib = _lib.lib()
    if fn == "ws":
        return lib.spec_verify_ws(1, t, d, tok, NUL, u, B, D, V, temp, ol, ot, FAKE, 1 << 30, NUL)
    if fn == "noalloc":
        return lib.spec_verify_noalloc(1, t, d, tok, NUL, u, B, D, V, temp, ol, ot, NUL)
    return getattr(lib, fn)(t, d, tok, NUL, u, B, D, V, temp, ol, ot, NUL)


@pytest.mark.parametrize("fn", ["spec_verify_bf16", "spec_verify_f32", "ws", "noalloc"])
def test_bad_arguments_return_einval(fn):
    E = _lib.SV_EINVAL
    assert _call(fn, B=0) == E
    assert _call(fn, B=-3) == E
    assert _call(fn, D=-1) == E
    assert _call(fn, D=_lib.SV_MAX_D + 1) == E
    assert _call(fn, V=0) == E
    assert _call(fn, t=NUL) == E
    assert _call(fn, d=NUL) == E
    assert _call(fn, tok=NUL) == E
    assert _call(fn, u=NUL) == E
    assert _call(fn, temp=NUL) == E
    assert _call(fn, ol=NUL) == E
    assert _call(fn, ot=NUL) == E
    assert _call(fn, B=1 << 30, D=63, V=1 << 30) == E      # element count overflow guard


def test_bad_dtype_and_workspace():
    lib = _lib.lib()
    args = (FAKE, FAKE, FAKE, NUL, FAKE, 2, 3, 100, FAKE, FAKE, FAKE)
    assert lib.spec_verify_ws(7, *args, FAKE, 1 << 30, NUL) == _lib.SV_EDTYPE
    assert lib.spec_verify_ws(1, *args, NUL, 1 << 30, NUL) == _lib.SV_EINVAL
    assert lib.spec_verify_ws(1, *args, FAKE, 16, NUL) == _lib.SV_ENOMEM
    assert lib.spec_verify_ws(1, *args, ctypes.c_void_p(4096 + 8), 1 << 30, NUL) == _lib.SV_ENOMEM


def test_noalloc_rejects_problems_beyond_its_scratch():
    """The no-allocation entry point refuses, before any device call, a problem whose workspace
    exceeds its fixed scratch; the limit is the one the header states."""
    lib = _lib.lib()
    assert "SV_NOALLOC_SCRATCH_BYTES (32u << 20)" in open(HEADER).read()
    assert _lib.SV_NOALLOC_SCRATCH_BYTES == 32 << 20
    for B, D, V in ((4096, 1, 129280), (2048, 7, 129280), (100000, 3, 32000)):
        assert lib.spec_verify_workspace_bytes(B, D, V) > _lib.SV_NOALLOC_SCRATCH_BYTES
        assert _call("noalloc", B=B, D=D, V=V) == _lib.SV_ESCRATCH
    assert lib.spec_verify_noalloc(7, FAKE, FAKE, FAKE, NUL, FAKE, 2, 3, 100, FAKE, FAKE, FAKE,
                                   NUL) == _lib.SV_EDTYPE
    assert lib.spec_verify_workspace_bytes(1024, 1, 129280) <= _lib.SV_NOALLOC_SCRATCH_BYTES
    assert lib.spec_verify_workspace_bytes(512, 7, 129280) <= _lib.SV_NOALLOC_SCRATCH_BYTES


def test_d0_allows_null_draft_pointers():
    lib = _lib.lib()
    # D = 0: draft logits and tokens are not needed; with no device the call ends in ENODEV
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present: this host-only case would launch")
    rc = lib.spec_verify_bf16(FAKE, NUL, NUL, NUL, FAKE, 2, 0, 100, FAKE, FAKE, FAKE, NUL)
    assert rc == _lib.SV_ENODEV


def test_no_device_is_reported():
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present: this host-only case would launch")
    assert _call("spec_verify_bf16") == _lib.SV_ENODEV
    assert _call("spec_verify_f32") == _lib.SV_ENODEV
    assert _call("noalloc") == _lib.SV_ENODEV


def test_advance_bad_arguments():
    lib = _lib.lib()
    E = _lib.SV_EINVAL
    ok = dict(al=FAKE, tok=FAKE, B=4, D=3, ids=FAKE, W=8, lens=NUL)

    def call(**kw):
        a = {**ok, **kw}
        return lib.spec_verify_advance(a["al"], a["tok"], a["B"], a["D"], a["ids"], a["W"],
                                       a["lens"], NUL)
    assert call(B=0) == E and call(B=-1) == E
    assert call(D=-1) == E and call(D=_lib.SV_MAX_D + 1) == E
    assert call(W=0) == E and call(W=-5) == E
    assert call(al=NUL) == E and call(tok=NUL) == E and call(ids=NUL) == E
    if torch.cuda.device_count() == 0:
        assert call() == _lib.SV_ENODEV


def test_threshold_bad_arguments():
    lib = _lib.lib()
    E = _lib.SV_EINVAL

    def call(tau=0.01, dtype=1, t=FAKE, tok=FAKE, B=2, D=3, V=100):
        return lib.spec_verify_threshold(dtype, t, tok, NUL, FAKE, B, D, V, FAKE, tau, FAKE,
                                         FAKE, NUL)
    assert call(tau=float("nan")) == E and call(tau=-0.5) == E and call(tau=float("inf")) == E
    assert call(t=NUL) == E and call(tok=NUL) == E and call(B=0) == E and call(V=0) == E
    assert call(dtype=5) == _lib.SV_EDTYPE
    if torch.cuda.device_count() == 0:        # no draft pointer is needed
        assert call() == _lib.SV_ENODEV


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No CPU fallback: with the shared library absent the binding raises instead of computing
    anything another way."""
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libspecverify.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.lib()


def test_saguaro_bad_arguments():
    lib = _lib.lib()
    E = _lib.SV_EINVAL

    def call(dtype=1, d=FAKE, temp=FAKE, B=2, D=3, V=100, factor=0.5, k=5):
        return lib.spec_verify_saguaro_reshape(dtype, d, NUL, temp, B, D, V, factor, k, NUL)
    assert call(factor=0.0) == E and call(factor=1.5) == E and call(factor=float("nan")) == E
    assert call(k=0) == E and call(k=9) == E
    assert call(B=0) == E and call(V=0) == E and call(D=-1) == E and call(D=_lib.SV_MAX_D + 1) == E
    assert call(d=NUL) == E and call(temp=NUL) == E
    assert call(dtype=3) == _lib.SV_EDTYPE
    if torch.cuda.device_count() == 0:
        assert call() == _lib.SV_ENODEV


def test_row_stage_plan():
    """spec_verify_row_stages: boundaries from 0 to D + 1, strictly increasing; one stage for
    small problems and for D = 0; bad arguments give SV_EINVAL."""
    lib = _lib.lib()
    cuts = (ctypes.c_int * 8)()
    for dt, B, D, V in [(1, 64, 7, 128256), (1, 512, 7, 129280), (1, 256, 3, 128256),
                        (1, 1024, 1, 129280), (0, 16, 4, 32000), (0, 1, 4, 1024),
                        (1, 4096, 0, 129280), (0, 3000, 31, 100000)]:
        n = lib.spec_verify_row_stages(dt, B, D, V, cuts, 8)
        assert 1 <= n <= 3, (dt, B, D, V, n)
        c = [cuts[i] for i in range(n + 1)]
        assert c[0] == 0 and c[-1] == D + 1 and all(a < b for a, b in zip(c, c[1:])), c
        rows_bytes = B * (2 * D + 1) * V * (2 if dt == 1 else 4)
        if D == 0 or rows_bytes < (64 << 20):
            assert n == 1, (dt, B, D, V, c)
    assert lib.spec_verify_row_stages(5, 64, 7, 100, cuts, 8) == _lib.SV_EINVAL
    assert lib.spec_verify_row_stages(1, 0, 7, 100, cuts, 8) == _lib.SV_EINVAL
    assert lib.spec_verify_row_stages(1, 4, 7, 100, None, 8) == _lib.SV_EINVAL

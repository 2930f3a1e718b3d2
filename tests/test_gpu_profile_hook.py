"""The benchmark's timing hook (spec_verify_profile_start / _stop): one event pair per row-kernel
launch, in launch order, each launch's own start and end stamps."""
import ctypes

import numpy as np
import pytest
import torch

from sampling_spec_verify_02_amd import _lib
from workloads import make

pytestmark = pytest.mark.gpu

from tests import gpu_util as G  # noqa: E402


def _stages(w):
    c = (ctypes.c_int * 8)()
    n = _lib.lib().spec_verify_row_stages(1 if w.dtype == "bf16" else 0, w.B, w.D, w.V, c, 8)
    assert n >= 1
    return n


@pytest.mark.parametrize("cfg,kw", [("c3", {}), ("c2", dict(B=4))])
def test_one_event_pair_per_row_launch(cfg, kw):
    w = make(cfg, 31, **kw)
    launches = _stages(w)                 # B < 32768: one slice per stage
    lib = _lib.lib()
    G.run(w)                              # library workspace in place before timing
    assert lib.spec_verify_profile_start(8) == 0
    for _ in range(2):
        G.run(w)
    out = (ctypes.c_float * 8)()
    n = ctypes.c_int(-1)
    assert lib.spec_verify_profile_stop(out, 8, ctypes.byref(n)) == 0
    assert n.value == 2 * launches
    ms = np.array(out[:n.value])
    assert np.all(ms > 0) and np.all(ms < 50), ms
    assert lib.spec_verify_profile_stop(out, 8, ctypes.byref(n)) == _lib.SV_EINVAL

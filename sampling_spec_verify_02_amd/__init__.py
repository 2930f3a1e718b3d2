"""MI355X-native speculative-decoding verification sampler (HIP for gfx950 behind a C ABI)."""
from ._lib import LIB_PATH, SpecVerifyError, lib, strerror
from .api import (spec_verify, spec_verify_advance, spec_verify_debug, spec_verify_noalloc,
                  saguaro_workspace_bytes, spec_verify_saguaro_reshape,
                  spec_verify_threshold, release, workspace_bytes)

__all__ = ["spec_verify", "spec_verify_advance", "spec_verify_debug", "spec_verify_noalloc",
           "spec_verify_threshold",
           "spec_verify_saguaro_reshape",
           "workspace_bytes", "saguaro_workspace_bytes", "release", "lib", "strerror",
           "SpecVerifyError", "LIB_PATH"]

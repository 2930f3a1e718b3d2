"""MI355X-native speculative-decoding verification sampler (HIP for gfx950 behind a C ABI)."""
from ._lib import LIB_PATH, SpecVerifyError, lib, strerror
from .api import (spec_verify, spec_verify_advance, spec_verify_debug, spec_verify_noalloc,
                  spec_verify_saguaro_reshape, spec_verify_threshold, workspace_bytes)

__all__ = ["spec_verify", "spec_verify_advance", "spec_verify_debug", "spec_verify_noalloc",
           "spec_verify_threshold",
           "spec_verify_saguaro_reshape",
           "workspace_bytes", "lib", "strerror", "SpecVerifyError", "LIB_PATH"]

"""CPU oracles of the verification sampler (fp64) and of the epilogue that follows it. Test
infrastructure only: used by tests/, the smoke check and the benchmark's CPU-baseline leg, never
by the product path."""
from .oracle import (Result, verify, verify_workload, tempered_log_softmax, softmax, accepts,
                     residual_weights, inverse_cdf, accept_window_measure, final_window,
                     final_window_measure, FLAG_TOL, ABS_WINDOW, EVAL_REL)
from .advance import advance
from .threshold import verify_threshold, verify_threshold_workload

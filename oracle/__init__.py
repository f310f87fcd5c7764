"""CPU oracles for the CfC K-loop and the batched MLP step (mlp_oracle) --
TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this package.  The GPU library never does, and this package imports
nothing from it.
"""
from .oracle import (  # noqa: F401
    fwd_step, bwd_step, forward, train, reduce_axis0_f64, sum_axis0, input_projection, adamw_step, lib_path,
    set_threads, threads,
)

"""CPU oracle of the DiLoCo outer-step merge.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check
and the CPU-baseline leg of the benchmark, never by the product library.
"""
from .oracle import (  # noqa: F401
    F32, BF16, LIB_PATH, Oracle, load, fold_mean, finalize_mean, fold_delta, outer_nesterov,
    ema_update, mean_round, nesterov_fragment_round, swa_average, snapshot_average, adopt_keep_drift,
    threads,
    set_threads,
)

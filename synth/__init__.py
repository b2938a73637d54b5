"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This package holds data generation only: random draws, dtype rounding and the
workload shapes.  It contains none of the recurrence's arithmetic, so that the
oracle (``oracle/``) and the GPU library (``scan_linear_rnn_amd``) share no
compute code.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    LAYER,
    LAYER_TINY,
    MINMAX,
    SCAN,
    STEP,
    TENSOR_IDS,
    T_BLOCK,
    bf16_round,
    decay_rates,
    device_normal,
    device_uniform,
    gaps,
    normal_bt,
    normal_mat,
    normal_vec,
    uniform_bt,
    uniform_vec,
)

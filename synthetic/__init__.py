"""Seeded synthetic inputs for the OSCAR INT2 decode path.

This package is the only code shared by the CPU oracle (``oracle/``), the GPU
tests and ``bench.py``.  It draws random tensors and builds the fixed offline
parameters the hot path consumes (the rotations R_K, R_V and the clip
thresholds), following the calibration recipe the OSCAR pages describe
(MarkTechPost article, "What OSCAR Does Differently": R = U * H_Had * P_br with
U the eigenvectors of the query covariance C_Q for keys and of the
score-weighted value covariance C_S for values).

It holds none of the hot path's arithmetic: no rotation of cache tokens, no
clipping, quantization or packing, no attention.  Those live, independently,
in ``oracle/`` (plain CPU reference) and in the HIP library.
"""

from .recipes import (  # noqa: F401
    CONFIGS,
    Workload,
    Calibration,
    Inputs,
    bit_reversal_permutation,
    calibrate,
    draw_inputs,
    hadamard_matrix,
    make_workload,
    random_page_table,
)

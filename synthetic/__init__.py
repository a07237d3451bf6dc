"""Seeded synthetic inputs for the OSCAR INT2 decode path.

This package is the only code shared by the CPU oracle (``oracle/``), the GPU
tests and ``bench.py``.  It draws random tensors only: workload shapes,
calibration activations, cache contents, queries and page tables.

It holds none of the method's arithmetic: no covariance, eigenbasis, rotation
construction or clip threshold, no rotation of cache tokens, no quantization
or packing, no attention.  Those live, independently, in ``oracle/`` (plain
CPU reference) and in the HIP library.  The offline parameters the cache
tensors depend on (values are stored multiplied by R_V) are passed in.
"""

from .recipes import (  # noqa: F401
    CALIB_TOKENS,
    CONFIGS,
    Workload,
    Calibration,
    CalibrationDraw,
    Inputs,
    draw_calibration,
    draw_inputs,
    make_calibration,
    make_workload,
    query_eigenvalues,
    random_page_table,
)

"""Seeded synthetic inputs for the 1-bit Adam compression-phase step.

This package holds workload descriptions (tensor shape lists, worker counts,
value distributions) and seeded random generators.  It contains none of the
method's arithmetic: both the oracle and the HIP path receive its output as
plain arrays, and neither is imported here.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    padded_layout,
    tensor_list,
)
from .generate import (  # noqa: F401
    init_state,
    grads_for_step,
    host_slice,
)

"""MI355X (gfx950) linear-recurrence scans for RL credit assignment.

Seven estimators and the generic segmented affine scan, one C-ABI call each
(include/lrs.h), backed by hand-written HIP kernels in csrc/.  The Python functions here only marshal torch tensors
into those calls; nothing runs on the CPU.
"""
from .api import (  # noqa: F401
    LrsError,
    compute_affine_scan,
    compute_discounted_returns,
    compute_eligibility_traces,
    compute_episodic_prefix_sum,
    compute_gae,
    compute_lambda_returns,
    compute_retrace,
    compute_vtrace,
    lib_path,
    load,
    set_schedule,
    set_time_major_waves,
    workspace_state,
)

__all__ = [
    "compute_gae", "compute_vtrace", "compute_retrace", "compute_lambda_returns",
    "compute_discounted_returns", "compute_eligibility_traces", "compute_episodic_prefix_sum",
    "compute_affine_scan",
    "LrsError", "load", "lib_path", "set_schedule", "set_time_major_waves", "workspace_state",
]

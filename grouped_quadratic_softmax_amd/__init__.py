"""OAL causal grouped-quadratic linear attention for MI355X (gfx950).

The compute path is the HIP library ``liboal.so`` (C ABI in include/oal.h);
this package is its thin torch binding plus host-side grouping utilities.
"""

from ._lib import OalError, lib  # noqa: F401
from .grouping import bootstrap_indices, group_dims, group_dims_budget, groups_from_contribution  # noqa: F401
from .ops import (  # noqa: F401
    Coeffs,
    ContribPlan,
    DecodePlan,
    PrefillPlan,
    Prep,
    StepPlan,
    bwd,
    calibrate,
    bwd_workspace_bytes,
    coeffs_from_factor,
    contrib,
    decode_step,
    decode_workspace_bytes,
    feature_count,
    fwd,
    fwd_workspace_bytes,
    fwd_workspace_bytes_for,
    state_floats,
)


def version() -> str:
    return lib().oal_version().decode()

"""MI355X-native shard GEMMs of a 3D-parallel FC layer.

One GPU's three local bf16 products of a fully connected layer under the 3D
parallel matrix multiply (sciencestack.ai/paper/2502.08145, Figure 1):
forward Y = X.W, backward-data dX = dY.W^T, backward-weight dW = X^T.dY,
computed by hand-written gfx950 MFMA kernels behind a C ABI
(include/fcshard.h, libfcshard.so). This package holds the HIP sources
(csrc/), their build script and the thin ctypes binding.
"""
from .fcshard import (  # noqa: F401
    COL,
    OP_BWD_DATA,
    OP_BWD_WEIGHT,
    OP_FWD,
    OUT_BF16,
    OUT_F32,
    ROW,
    FcError,
    fc_bwd_data,
    fc_bwd_weight,
    fc_fwd,
    fc_plan_count,
    fc_plan_describe,
    fc_plans_load,
    fc_plans_save,
    fc_release,
    fc_set_plan,
    fc_tune,
    status_str,
)

"""Context-parallel causal attention for one CP rank's shard on MI355X.

The work happens in ``libcpattn.so`` (C ABI in ``include/cp_attn.h``): the
zigzag / interleave shard planner and restore index on the host, and HIP
kernels for gfx950 for the causal varlen attention forward and the
log-sum-exp merge.  This package is the thin ctypes binding over it.
"""
from ._lib import (  # noqa: F401
    CP_BF16, CP_F32, CP_INTERLEAVE, CP_ZIGZAG, EXPORTS, LIB_PATH, CpError, Segment,
    ShardPlan, attn_fwd, attn_workspace_size, lse_merge, restore_index, shard_plan,
    status_str, version,
)

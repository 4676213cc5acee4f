"""Context-parallel causal attention for one CP rank's shard on MI355X.

The work happens in ``libcpattn.so`` (C ABI in ``include/cp_attn.h``): the
zigzag / interleave shard planner, restore index and pass-KV / pass-Q
selector on the host, and HIP kernels for gfx950 for the causal varlen
attention forward, the decode shard, the log-sum-exp merge and the restore
gather.  This package is the thin ctypes binding over it.
"""
from ._lib import (  # noqa: F401
    CP_BF16, CP_F32, CP_INTERLEAVE, CP_ZIGZAG, EXPORTS, LIB_PATH, PASS_KV, PASS_Q, CpError,
    Segment, ShardPlan, attn_fwd, attn_fwd_noalloc, attn_workspace_size, calib_copy, calib_mfma, choose_pass,
    lse_merge, restore_apply,
    restore_index, ring_pad_len, shard_plan, status_str, version,
)

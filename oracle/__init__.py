"""CPU oracle for context-parallel causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing here is part of the product path: only the
tests, the smoke check and the bench's ``cpu_baseline`` leg may import it.
It shares no code with the HIP library and does not import it.

* ``index_oracle``  -- zigzag / interleave shard plans, segments, restore
  index, causal tile loads (pure Python integers).
* ``attn_oracle``   -- causal attention for a shard (full or partial key set)
  and the log-sum-exp merge, in NumPy float64.
* ``scalar_oracle`` -- the same attention as scalar Python loops, for tiny
  shapes; it pins ``attn_oracle``.
* ``select_oracle`` -- the pass-KV / pass-Q rule, ring message padding and
  the restore gather.
"""

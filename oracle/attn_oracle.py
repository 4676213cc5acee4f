"""Attention and merge oracle, NumPy float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What is computed, written out from its definition:

* Causal attention of a query row i against a key set (pages: "Prefill
  Context Parallelism", sections "Zigzag strategy" and "Interleave strategy":
  every query block attends to its own causal history, cached prefix
  included; "What is Context Parallelism", section 2.1: each rank computes the
  attention output of its own queries against the full KV).  With visible set
  V(i) = {keys j of the same request with kv_pos_j <= q_pos_i} and
  s_ij = scale * <q_i, k_j>:
      lse_i = ln sum_{j in V(i)} exp(s_ij)
      o_i   = sum_{j in V(i)} exp(s_ij - lse_i) * v_j
  An empty V(i) gives o_i = 0 and lse_i = -inf.  The maximum is subtracted
  before exponentiating only to keep float64 in range; that is the same
  number, not a different algorithm.
* Partial attention over a key subset (same blog, sections 3.1 and 3.3:
  each ring round / each KV shard yields a normalised partial output O_j and
  its log-sum L_j): the formula above with V(i) restricted to the subset.
* The log-sum-exp merge (same blog, section 3.6; the page lost the display
  formula in extraction, so this is the reading from the surrounding text,
  which presents the merge as FlashAttention's online-softmax rescaling
  applied to whole partial results):
      L = ln sum_j exp(L_j),   O = sum_j exp(L_j - L) * O_j
  computed with m = max_j L_j; partials with L_j = -inf contribute nothing;
  all partials empty gives O = 0, L = -inf.

GQA (same blog, section 4.1): several query heads share one KV head; query
head h reads KV head h // (hq // hkv).
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

NEG_INF = -np.inf


def attend(q, k, v, q_pos, kv_pos, scale: float, causal: bool = True):
    """Attention of rows ``q`` [n, dqk] over keys ``k`` [L, dqk], values
    ``v`` [L, dv]; ``q_pos`` [n] and ``kv_pos`` [L] are absolute positions.
    Returns (o [n, dv], lse [n]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    n, L = q.shape[0], k.shape[0]
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full((n,), NEG_INF, dtype=np.float64)
    if n == 0 or L == 0:
        return o, lse
    s = scale * (q @ k.T)                                   # [n, L]
    if causal:
        visible = kv_pos[None, :] <= q_pos[:, None]
    else:
        visible = np.ones((n, L), dtype=bool)
    s = np.where(visible, s, NEG_INF)
    has = visible.any(axis=1)
    m = np.where(has, s.max(axis=1, initial=NEG_INF), 0.0)
    e = np.where(visible, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    safe_l = np.where(has, l, 1.0)
    o = np.where(has[:, None], (e @ v) / safe_l[:, None], 0.0)
    lse = np.where(has, m + np.log(safe_l), NEG_INF)
    return o, lse


def shard_attention(q, k, v, segs: Sequence, hq: int, hkv: int, scale: float,
                    kv_pos=None, rows: Optional[Iterable[int]] = None,
                    causal: bool = True, heads: Optional[Iterable[int]] = None):
    """Attention for one rank's local rows, segment by segment.

    ``q`` [N, hq, dqk] local rows; ``k`` [Lkv, hkv, dqk], ``v`` [Lkv, hkv, dv]
    the KV buffer the segments index.  Each segment gives its rows
    [q_begin, q_end), their positions pos_begin + i * pos_stride and the KV
    rows [kv_begin, kv_end) of its request.  Key positions are ``kv_pos[row]``
    when given, else ``row - kv_begin``.  ``rows``/``heads`` restrict which
    outputs are computed; the others stay O = 0, LSE = -inf."""
    N = q.shape[0]
    dv = v.shape[2]
    G = hq // hkv
    o = np.zeros((N, hq, dv), dtype=np.float64)
    lse = np.full((N, hq), NEG_INF, dtype=np.float64)
    row_set = None if rows is None else set(int(x) for x in rows)
    head_list = list(range(hq)) if heads is None else [int(h) for h in heads]
    for sg in segs:
        q_begin, q_end = int(sg.q_begin), int(sg.q_end)
        kv_begin, kv_end = int(sg.kv_begin), int(sg.kv_end)
        idx = [i for i in range(q_begin, q_end) if row_set is None or i in row_set]
        if not idx:
            continue
        idx = np.asarray(idx, dtype=np.int64)
        qp = int(sg.pos_begin) + (idx - q_begin) * int(sg.pos_stride)
        if kv_pos is None:
            kp = np.arange(kv_end - kv_begin, dtype=np.int64)
        else:
            kp = np.asarray(kv_pos[kv_begin:kv_end], dtype=np.int64)
        for h in head_list:
            kh = h // G
            oo, ll = attend(q[idx, h, :], k[kv_begin:kv_end, kh, :],
                            v[kv_begin:kv_end, kh, :], qp, kp, scale, causal)
            o[idx, h, :] = oo
            lse[idx, h] = ll
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Merge P partials: ``o_parts`` [P, ..., dv], ``lse_parts`` [P, ...]."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)                                # [...]
    any_part = np.isfinite(m)
    m0 = np.where(any_part, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m0[None]), 0.0)
    wsum = w.sum(axis=0)
    safe = np.where(any_part, wsum, 1.0)
    o = (w[..., None] * o_parts).sum(axis=0) / safe[..., None]
    o = np.where(any_part[..., None], o, 0.0)
    lse = np.where(any_part, m0 + np.log(safe), NEG_INF)
    return o, lse

"""Scalar attention oracle: plain Python loops over one query row at a time,
``math.exp``/``math.log`` only.  Slow; tiny shapes only.  It exists to pin
``attn_oracle`` with an implementation that uses no array library.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Definition (pages: "What is Context Parallelism", sections 2.1 and 3.6;
"Prefill Context Parallelism", section "Zigzag strategy"): for query q at
position p, the visible keys are those of its request at positions <= p;
the row's log-sum is the log of the sum of exp(scale * <q, k>) over them and
the output is the softmax-weighted sum of their values.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple


def attend_row(q: Sequence[float], keys: Sequence[Sequence[float]],
               vals: Sequence[Sequence[float]], q_pos: int,
               key_pos: Sequence[int], scale: float,
               causal: bool = True) -> Tuple[List[float], float]:
    scores = []
    for j in range(len(keys)):
        if causal and key_pos[j] > q_pos:
            continue
        dot = 0.0
        for a, b in zip(q, keys[j]):
            dot += a * b
        scores.append((scale * dot, j))
    dv = len(vals[0]) if vals else 0
    if not scores:
        return [0.0] * dv, -math.inf
    top = max(s for s, _ in scores)
    total = 0.0
    for s, _ in scores:
        total += math.exp(s - top)
    lse = top + math.log(total)
    out = [0.0] * dv
    for s, j in scores:
        w = math.exp(s - lse)
        for d in range(dv):
            out[d] += w * vals[j][d]
    return out, lse


def merge_row(outs: Sequence[Sequence[float]], lses: Sequence[float]):
    """Merge partial (O_j, L_j) of one row: L = ln sum exp(L_j),
    O = sum exp(L_j - L) O_j; empty partials (L_j = -inf) are skipped."""
    live = [(o, l) for o, l in zip(outs, lses) if l != -math.inf]
    dv = len(outs[0]) if outs else 0
    if not live:
        return [0.0] * dv, -math.inf
    top = max(l for _, l in live)
    total = sum(math.exp(l - top) for _, l in live)
    lse = top + math.log(total)
    out = [0.0] * dv
    for o, l in live:
        w = math.exp(l - lse)
        for d in range(dv):
            out[d] += w * o[d]
    return out, lse

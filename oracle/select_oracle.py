"""pass-KV / pass-Q selection, ring message padding and the restore gather.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"What is Context Parallelism" (blog), section 3.5, pass-KV / pass-Q switch:

* miss rate = T / (T + P) with T new tokens and P cached tokens;
* passing Q gives the smaller message iff T / (T + P) <= 2 * N_kv / N_h
  (the section's threshold is 12.5 % for N_h = 128, N_kv = 8);
* the empirical fit h(T, P) = -1.059 log T + 1.145 log(T / (T + P)) + 12.112,
  h > 0 choosing pass-KV.  The pages print the coefficients and the constant
  but no value of h and no log base; what they fix holds under any base and
  is pinned (constant, ratio of the coefficients, signs, logarithmic form).
  The base is a reading: natural logarithm, parity unpinned (the switch
  point quoted beside the fit, about 5 % miss rate at 128K tokens, CP 4, is
  not reproduced by the printed fit under a natural, base-2 or base-10
  logarithm);
* ring messages are padded to max_i P_i + ceil(T / N).

Section 2.1 (engineering notes) / 5.1: the rank-major all-gathered rows,
gathered by the restore index, are in causal order -- ``restore_apply`` is
that gather written out (numpy fancy indexing).
"""
import math
from fractions import Fraction

import numpy as np

PASS_KV, PASS_Q = 0, 1


def miss_rate(T: int, P: int) -> Fraction:
    return Fraction(T, T + P)


def choose_pass(T: int, P: int, n_heads: int, n_kv_heads: int) -> int:
    """PASS_Q iff the miss rate is within 2 * N_kv / N_h (exact fractions)."""
    return PASS_Q if miss_rate(T, P) <= Fraction(2 * n_kv_heads, n_heads) else PASS_KV


def h_score(T: int, P: int) -> float:
    return -1.059 * math.log(T) + 1.145 * math.log(T / (T + P)) + 12.112


def ring_pad_len(cached_per_rank, T: int) -> int:
    N = len(cached_per_rank)
    return max(cached_per_rank) + -(-T // N)


def restore_apply(index, src, fill=0):
    """dst[i] = src[index[i]]; an index outside [0, len(src)) gives a row of
    ``fill``."""
    src = np.asarray(src)
    index = np.asarray(index, dtype=np.int64)
    dst = np.full((len(index),) + src.shape[1:], fill, dtype=src.dtype)
    ok = (index >= 0) & (index < len(src))
    dst[ok] = src[index[ok]]
    return dst

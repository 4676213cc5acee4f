"""Pins of oracle.select_oracle against what the pages fix ("What is Context
Parallelism", section 3.5): the 12.5 % threshold printed for N_h = 128,
N_kv = 8, decode (T = 1) choosing pass-Q, full prefill choosing pass-KV;
ring padding on a hand-worked case; the restore gather against the
definition on a hand-worked permutation.  h(T, P) is unpinned (see the
oracle's docstring)."""
from fractions import Fraction

import numpy as np

from oracle import index_oracle as ix
from oracle import select_oracle as so


def test_threshold_405b():
    # 2 * 8 / 128 = 1/8: a miss rate of exactly 12.5 % is still pass-Q
    assert Fraction(2 * 8, 128) == Fraction(1, 8)
    assert so.choose_pass(1, 7, 128, 8) == so.PASS_Q          # 1/8
    assert so.choose_pass(16384, 114688, 128, 8) == so.PASS_Q  # 1/8 at 128K
    assert so.choose_pass(16385, 114687, 128, 8) == so.PASS_KV
    assert so.choose_pass(125, 875, 128, 8) == so.PASS_Q       # 12.5 %
    assert so.choose_pass(126, 874, 128, 8) == so.PASS_KV      # 12.6 %


def test_decode_and_full_prefill():
    assert so.choose_pass(1, 131071, 128, 8) == so.PASS_Q     # decode
    assert so.choose_pass(131072, 0, 128, 8) == so.PASS_KV    # full prefill
    # MHA: 2 N_kv / N_h = 2 > any miss rate -- a Q message (T N_h d) is always
    # smaller than the K and V message (2 (T + P) N_kv d)
    assert so.choose_pass(131072, 0, 8, 8) == so.PASS_Q
    assert so.choose_pass(1, 0, 8, 8) == so.PASS_Q
    assert so.miss_rate(3, 9) == Fraction(1, 4)


def test_ring_pad_len():
    # max P_i = 300, ceil(10 / 3) = 4
    assert so.ring_pad_len([100, 300, 200], 10) == 304
    assert so.ring_pad_len([0, 0, 0, 0], 8) == 2
    assert so.ring_pad_len([5], 0) == 5


def test_restore_apply_definition():
    src = np.arange(12).reshape(6, 2)
    got = so.restore_apply([5, 0, 3, -1, 6], src, fill=-7)
    assert got.tolist() == [[10, 11], [0, 1], [6, 7], [-7, -7], [-7, -7]]


def test_restore_apply_restores_causal_order():
    # gathering the rank-major buffer (slot -> flattened index) by restore
    # gives 0, 1, 2, ... (the planner's restore pins live in the index tests)
    for strategy, C, lens in (("zigzag", 4, [16]), ("interleave", 4, [5, 3]), ("zigzag", 3, [7, 10])):
        restore, pad = ix.restore_index(strategy, C, lens)
        gathered = np.array(ix.gathered_global_idx(strategy, C, lens))
        assert len(gathered) == C * pad
        assert so.restore_apply(restore, gathered).tolist() == list(range(sum(lens)))

"""Pins of oracle.select_oracle against what the pages fix ("What is Context
Parallelism", section 3.5): the 12.5 % threshold printed for N_h = 128,
N_kv = 8, decode (T = 1) choosing pass-Q, full prefill choosing pass-KV;
ring padding on a hand-worked case; the restore gather against the
definition on a hand-worked permutation.  For the empirical fit h(T, P)
the section prints three numbers (two coefficients and a constant) but no
value of h and no log base; the pins below hold under ANY log base and fix
what the printed numbers fix: the constant (h(1, 0)), the ratio of the two
coefficients, the sign of each term and that both terms are logarithmic.
The log base itself stays a reading (natural log), parity unpinned."""
import math
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


# ---------------------------------------------------------------- h(T, P)
C_H, A_T, B_MISS = 12.112, 1.059, 1.145   # the section's printed fit


def test_h_constant():
    # T = 1, P = 0: log 1 = 0 and the miss rate is 1 under any base, so only
    # the constant is left (a dropped or mistyped constant fails here)
    assert so.h_score(1, 0) == C_H


def test_h_coefficient_ratio_any_base():
    # h(T, 0) - c = -a log T and h(1, T - 1) - c = b log(1 / T) = -b log T:
    # their ratio is a / b whatever the base (a swapped or dropped
    # coefficient, or a term on the wrong argument, fails here)
    for T in (2, 3, 17, 1000, 131072, 10 ** 7):
        r = (so.h_score(T, 0) - C_H) / (so.h_score(1, T - 1) - C_H)
        assert abs(r - A_T / B_MISS) <= 1e-12, T


def test_h_terms_are_logarithmic_and_signed():
    # at a fixed miss rate h moves by -a log(scale factor): doubling T and P
    # twice moves it exactly twice as far as doubling once (any base), and
    # downwards (a wrong sign on the log T term fails)
    for T, P in ((1, 0), (100, 300), (4096, 131072 - 4096)):
        d1 = so.h_score(2 * T, 2 * P) - so.h_score(T, P)
        d2 = so.h_score(4 * T, 4 * P) - so.h_score(T, P)
        assert d1 < 0 and abs(d2 - 2 * d1) <= 1e-12 * max(1.0, abs(d2))
    # at fixed T more cached tokens lower the miss rate and so lower h (a
    # wrong sign on the miss-rate term fails)
    for T in (1, 64, 16384):
        vals = [so.h_score(T, P) for P in (0, 1, 10, 1000, 10 ** 6)]
        assert all(a > b for a, b in zip(vals, vals[1:])), T


def test_h_log_base_reading():
    # the reading is the natural logarithm: with it the fit's two terms are
    # -a ln T and b ln(miss rate) exactly (this checks the reading as stated,
    # not the page: the page does not fix the base)
    T, P = 5000, 20000
    assert abs(so.h_score(T, P) - (C_H - A_T * math.log(T) + B_MISS * math.log(T / (T + P)))) \
        <= 1e-12

"""Pins for the index oracle: the pages' worked examples, the causal tile
balance figure, closed forms and brute-force invariants.  CPU only."""
import json
import os
import random

import pytest

from oracle import index_oracle as ix


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_zigzag_printed_example(golden_dir):
    g = _load(golden_dir, "zigzag_cp4_t16.json")
    C, lens = g["cp_size"], g["new_lens"]
    assert [list(b) for b in ix.zigzag_blocks(lens[0], C)] == g["blocks"]
    for r in range(C):
        toks = ix.rank_tokens("zigzag", C, r, lens, [0])
        assert [t.g for t in toks] == g["rank_tokens"][r]
        # rank r owns blocks r and 2C-1-r, early block first
        blocks = ix.zigzag_blocks(lens[0], C)
        want = []
        for k in g["rank_blocks"][r]:
            want += list(range(*blocks[k]))
        assert [t.t for t in toks] == want


def test_interleave_printed_example(golden_dir):
    g = _load(golden_dir, "interleave_cp4_t16.json")
    C, lens = g["cp_size"], g["new_lens"]
    for r in range(C):
        toks = ix.rank_tokens("interleave", C, r, lens, [0])
        assert [t.g for t in toks] == g["rank_tokens"][r]
        assert [t.pos for t in toks] == g["rank_tokens"][r]  # positions keep their values


def test_interleave_two_requests_printed(golden_dir):
    g = _load(golden_dir, "interleave_cp4_lens5_3.json")
    C, lens = g["cp_size"], g["new_lens"]
    pr = g["printed"]
    for r, want in pr["rank_tokens"].items():
        toks = ix.rank_tokens("interleave", C, int(r), lens, [0, 0])
        assert [t.g for t in toks] == want
    # index 5 is the second request's first new token
    allt = {t.g: t for r in range(C) for t in ix.rank_tokens("interleave", C, r, lens, [0, 0])}
    assert (allt[5].req, allt[5].t) == (pr["index_5"]["req"], pr["index_5"]["t"])
    # the same rule, not printed: ranks 2 and 3 own {2, 6} and {3, 7}
    assert [t.g for t in ix.rank_tokens("interleave", C, 2, lens, [0, 0])] == [2, 6]
    assert [t.g for t in ix.rank_tokens("interleave", C, 3, lens, [0, 0])] == [3, 7]
    # per-request metadata keeps each request's own positions
    toks1 = ix.rank_tokens("interleave", C, 1, lens, [0, 0])
    assert [(t.req, t.pos) for t in toks1] == [(0, 1), (1, 0)]


def test_causal_tile_loads_figure(golden_dir):
    g = _load(golden_dir, "causal_tile_loads_cp4.json")
    C = g["cp_size"]
    assert ix.causal_tile_loads(ix.block_owners("sequential", C), C) == g["sequential"]
    assert ix.causal_tile_loads(ix.block_owners("zigzag", C), C) == g["zigzag"]


@pytest.mark.parametrize("C", range(1, 9))
def test_tile_load_closed_forms(C):
    seq = ix.causal_tile_loads(ix.block_owners("sequential", C), C)
    zz = ix.causal_tile_loads(ix.block_owners("zigzag", C), C)
    assert seq == [4 * r + 3 for r in range(C)]
    assert zz == [2 * C + 1] * C
    assert sum(seq) == sum(zz) == (2 * C) * (2 * C + 1) // 2


@pytest.mark.parametrize("T,C,P,want", [
    (256, 4, 0, 8224),
    (8192, 8, 1024, 5243392),
    (131072, 8, 0, 1073750016),
])
def test_zigzag_equal_pairs_per_rank(T, C, P, want):
    pairs = [ix.visible_pairs("zigzag", C, r, [T], [P]) for r in range(C)]
    assert pairs == [want] * C
    assert sum(pairs) == T * P + T * (T + 1) // 2


def test_remainder_rule_early_blocks():
    # 18 tokens over 8 blocks: the two earliest blocks take one extra token
    assert [e - s for s, e in ix.zigzag_blocks(18, 4)] == [3, 3, 2, 2, 2, 2, 2, 2]
    assert [e - s for s, e in ix.zigzag_blocks(3, 4)] == [1, 1, 1, 0, 0, 0, 0, 0]
    assert ix.zigzag_blocks(0, 2) == [(0, 0)] * 4


def _random_batches(seed, n):
    rnd = random.Random(seed)
    for _ in range(n):
        C = rnd.randint(1, 8)
        B = rnd.randint(1, 4)
        lens = [rnd.randint(0, 64) for _ in range(B)]
        pre = [rnd.choice([0, 0, rnd.randint(0, 40)]) for _ in range(B)]
        yield C, lens, pre


@pytest.mark.parametrize("strategy", ["zigzag", "interleave"])
def test_brute_force_invariants(strategy):
    for C, lens, pre in _random_batches(7 if strategy == "zigzag" else 8, 300):
        total = sum(lens)
        seen = []
        pad = ix.padded_local(strategy, C, lens, pre)
        kvoff = [sum(p + t for p, t in zip(pre[:b], lens[:b])) for b in range(len(lens))]
        for r in range(C):
            toks = ix.rank_tokens(strategy, C, r, lens, pre)
            assert len(toks) <= pad
            seen += [t.g for t in toks]
            for t in toks:
                assert t.pos == pre[t.req] + t.t
                assert t.g == sum(lens[:t.req]) + t.t
            segs = ix.segments(strategy, C, r, lens, pre)
            rows = 0
            for sg in segs:
                assert sg.q_end > sg.q_begin == rows
                rows = sg.q_end
                last = sg.pos_begin + (sg.q_end - sg.q_begin - 1) * sg.pos_stride
                assert sg.kv_begin == kvoff[sg.req]
                assert sg.kv_end - sg.kv_begin == last + 1     # causal extent incl. prefix
                assert last < pre[sg.req] + lens[sg.req]
            assert rows == len(toks)
        # the ranks' token sets partition the batch's new tokens
        assert sorted(seen) == list(range(total))
        # restore undoes the rank-major gather
        restore, pad2 = ix.restore_index(strategy, C, lens)
        assert pad2 == ix.padded_local(strategy, C, lens)
        gathered = ix.gathered_global_idx(strategy, C, lens)
        assert len(gathered) == C * pad2
        assert [gathered[s] for s in restore] == list(range(total))
        # total work is the dense causal work
        pairs = sum(ix.visible_pairs(strategy, C, r, lens, pre) for r in range(C))
        assert pairs == sum(T * P + T * (T + 1) // 2 for T, P in zip(lens, pre))


def test_zigzag_blocks_properties():
    for T in range(0, 70):
        for C in range(1, 9):
            b = ix.zigzag_blocks(T, C)
            sizes = [e - s for s, e in b]
            assert len(b) == 2 * C and sum(sizes) == T
            assert max(sizes) - min(sizes) <= 1
            assert sizes == sorted(sizes, reverse=True)
            assert all(b[i][1] == b[i + 1][0] for i in range(2 * C - 1))


def test_c1_is_identity():
    lens, pre = [5, 0, 9], [2, 3, 0]
    for s in ("zigzag", "interleave"):
        toks = ix.rank_tokens(s, 1, 0, lens, pre)
        assert [t.g for t in toks] == list(range(14))
        restore, pad = ix.restore_index(s, 1, lens)
        assert restore == list(range(14)) and pad == 14


def test_interleave_empty_segment_for_short_request():
    # lengths 5 and 3 (then more): rank 0 owns none of request 1's tokens 5, 6, 7
    segs = ix.segments("interleave", 4, 0, [5, 3, 8], [0, 0, 0])
    assert [s.req for s in segs] == [0, 2]


def test_bad_arguments():
    with pytest.raises(ValueError):
        ix.rank_tokens("zigzag", 0, 0, [4], [0])
    with pytest.raises(ValueError):
        ix.rank_tokens("zigzag", 2, 2, [4], [0])
    with pytest.raises(ValueError):
        ix.rank_tokens("ring", 2, 0, [4], [0])
    with pytest.raises(ValueError):
        ix.rank_tokens("zigzag", 2, 0, [-1], [0])

"""Pins for the attention / merge oracle against things other than itself:
the scalar loop oracle, torch's scaled_dot_product_attention on the CPU in
float64 (an independent library routine), closed forms and special cases.
CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attn_oracle as ao
from oracle import index_oracle as ix
from oracle import scalar_oracle as so


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("seed", range(6))
def test_attend_matches_scalar_loops(seed):
    rng = np.random.default_rng(seed)
    n, L, dqk, dv = 5, 9, 6, 4
    q, k, v = _rand(rng, n, dqk), _rand(rng, L, dqk), _rand(rng, L, dv)
    q_pos = rng.integers(-2, 12, size=n)          # some rows see nothing
    kv_pos = np.sort(rng.choice(20, size=L, replace=False))
    scale = 0.37
    o, lse = ao.attend(q, k, v, q_pos, kv_pos, scale)
    for i in range(n):
        oo, ll = so.attend_row(q[i].tolist(), k.tolist(), v.tolist(), int(q_pos[i]),
                               kv_pos.tolist(), scale)
        if ll == -math.inf:
            assert lse[i] == -np.inf and np.all(o[i] == 0)
        else:
            assert abs(lse[i] - ll) < 1e-12
            assert np.max(np.abs(o[i] - np.array(oo))) < 1e-12


def test_zero_query_closed_form():
    # q = 0: every visible score is 0, so LSE = ln(#visible), O = mean(V visible)
    rng = np.random.default_rng(11)
    L, dv = 40, 5
    k, v = _rand(rng, L, 8), _rand(rng, L, dv)
    q = np.zeros((L, 8))
    pos = np.arange(L)
    o, lse = ao.attend(q, k, v, pos, pos, 0.5)
    for i in range(L):
        assert abs(lse[i] - math.log(i + 1)) < 1e-13
        assert np.max(np.abs(o[i] - v[: i + 1].mean(axis=0))) < 1e-13


def test_single_visible_key():
    rng = np.random.default_rng(12)
    k, v = _rand(rng, 6, 4), _rand(rng, 6, 3)
    q = _rand(rng, 1, 4)
    o, lse = ao.attend(q, k, v, [0], np.arange(6), 0.25)
    assert np.allclose(o[0], v[0], atol=0, rtol=0)
    assert abs(lse[0] - 0.25 * float(q[0] @ k[0])) < 1e-15


def test_noncausal_and_empty():
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 3, 4), _rand(rng, 5, 4), _rand(rng, 5, 2)
    o, lse = ao.attend(q, k, v, [-1, -1, -1], np.arange(5), 1.0)
    assert np.all(lse == -np.inf) and np.all(o == 0)
    o2, lse2 = ao.attend(q, k, v, [-1, -1, -1], np.arange(5), 1.0, causal=False)
    ref = F.scaled_dot_product_attention(torch.tensor(q)[None], torch.tensor(k)[None],
                                         torch.tensor(v)[None], scale=1.0)[0].numpy()
    assert np.max(np.abs(o2 - ref)) < 1e-12


def _sdpa_causal_request(q_full, k, v, scale):
    """torch SDPA on one request as a full causal sequence (queries for every
    position, top-left causal = standard when Lq == Lk), GQA by enable_gqa."""
    qt = torch.tensor(q_full).permute(1, 0, 2)[None]   # [1, hq, L, d]
    kt = torch.tensor(k).permute(1, 0, 2)[None]
    vt = torch.tensor(v).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale,
                                       enable_gqa=qt.shape[1] != kt.shape[1])
    return o[0].permute(1, 0, 2).numpy()                # [L, hq, dv]


@pytest.mark.parametrize("strategy", ["zigzag", "interleave"])
@pytest.mark.parametrize("C", [1, 2, 3, 4])
def test_shard_attention_equals_dense_causal(strategy, C):
    """Every rank's shard, reassembled by flattened index, equals dense
    causal attention of each request (prefix included), checked against
    torch's SDPA."""
    rng = np.random.default_rng(100 + C)
    lens, pre = [13, 5, 3, 21], [0, 7, 2, 4]
    hq, hkv, dqk, dv, scale = 6, 2, 5, 3, 0.41
    # full per-request sequences (prefix queries exist only for SDPA)
    kv_rows = sum(p + t for p, t in zip(pre, lens))
    k, v = _rand(rng, kv_rows, hkv, dqk), _rand(rng, kv_rows, hkv, dv)
    q_seq = _rand(rng, kv_rows, hq, dqk)
    dense = np.zeros((sum(lens), hq, dv))
    g = 0
    off = 0
    for T, P in zip(lens, pre):
        o = _sdpa_causal_request(q_seq[off:off + P + T], k[off:off + P + T],
                                 v[off:off + P + T], scale)
        dense[g:g + T] = o[P:]
        g += T
        off += P + T
    # new-token queries in flattened order
    q_new = np.concatenate([q_seq[sum(p + t for p, t in zip(pre[:b], lens[:b])) + pre[b]:
                                  sum(p + t for p, t in zip(pre[:b + 1], lens[:b + 1]))]
                            for b in range(len(lens))])
    got = np.zeros_like(dense)
    for r in range(C):
        toks = ix.rank_tokens(strategy, C, r, lens, pre)
        gidx = [t.g for t in toks]
        segs = ix.segments(strategy, C, r, lens, pre)
        o, lse = ao.shard_attention(q_new[gidx], k, v, segs, hq, hkv, scale)
        got[gidx] = o
        assert np.all(np.isfinite(lse))
    assert np.max(np.abs(got - dense)) < 1e-12


def test_merge_special_cases():
    rng = np.random.default_rng(21)
    o1, l1 = _rand(rng, 4, 3, 5), _rand(rng, 4, 3)
    o, l = ao.lse_merge(o1[None], l1[None])
    assert np.array_equal(o, o1) and np.array_equal(l, l1)
    # an empty partial changes nothing
    o, l = ao.lse_merge(np.stack([o1, np.zeros_like(o1)]),
                        np.stack([l1, np.full_like(l1, -np.inf)]))
    assert np.max(np.abs(o - o1)) < 1e-15 and np.max(np.abs(l - l1)) < 1e-15
    # two identical partials: O unchanged, L + ln 2
    o, l = ao.lse_merge(np.stack([o1, o1]), np.stack([l1, l1]))
    assert np.max(np.abs(o - o1)) < 1e-14 and np.max(np.abs(l - (l1 + math.log(2)))) < 1e-14
    # all empty
    o, l = ao.lse_merge(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)


@pytest.mark.parametrize("seed", range(4))
def test_merge_of_key_partition_is_dense(seed):
    """Partials over any partition of the keys merge to dense attention,
    both all at once and hop by hop (pass-Q accumulator)."""
    rng = np.random.default_rng(seed)
    n, L, d = 7, 23, 4
    q, k, v = _rand(rng, n, d), _rand(rng, L, d), _rand(rng, L, d)
    q_pos = rng.integers(0, 30, size=n)
    kv_pos = np.sort(rng.choice(30, size=L, replace=False))
    q_pos[0] = -5                                          # a row with no key at all
    full_o, full_l = ao.attend(q, k, v, q_pos, kv_pos, 0.3)
    parts = rng.integers(0, 4, size=L)
    os_, ls_ = [], []
    for j in range(4):
        sel = parts == j
        o, l = ao.attend(q, k[sel], v[sel], q_pos, kv_pos[sel], 0.3)
        os_.append(o)
        ls_.append(l)
    mo, ml = ao.lse_merge(np.stack(os_), np.stack(ls_))
    assert np.max(np.abs(mo - full_o)) < 1e-12
    fin = np.isfinite(full_l)
    assert np.array_equal(np.isfinite(ml), fin)
    assert np.max(np.abs(ml[fin] - full_l[fin])) < 1e-12
    acc_o, acc_l = os_[0], ls_[0]
    for j in range(1, 4):
        acc_o, acc_l = ao.lse_merge(np.stack([acc_o, os_[j]]), np.stack([acc_l, ls_[j]]))
    assert np.max(np.abs(acc_o - full_o)) < 1e-12
    # scalar merge agrees on a row
    i = 3
    so_o, so_l = so.merge_row([o[i].tolist() for o in os_], [float(l[i]) for l in ls_])
    assert abs(so_l - full_l[i]) < 1e-12 and np.max(np.abs(np.array(so_o) - full_o[i])) < 1e-12


def test_ring_partials_over_zigzag_pairs_merge_to_dense():
    """Ring style (pass-KV): rank r's queries against each rank j's zigzag KV
    pair, masked by absolute positions, merged, equal dense causal."""
    C, T = 4, 40
    rng = np.random.default_rng(5)
    hq = hkv = 2
    d = 4
    q_all, k_all, v_all = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    dense = _sdpa_causal_request(q_all, k_all, v_all, 0.5)
    for r in range(C):
        mine = [t.g for t in ix.rank_tokens("zigzag", C, r, [T], [0])]
        segs = [ix.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, 0)
                for s in ix.segments("zigzag", C, r, [T], [0])]
        os_, ls_ = [], []
        for j in range(C):
            kv_rows = [t.g for t in ix.rank_tokens("zigzag", C, j, [T], [0])]
            sj = [ix.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0,
                             len(kv_rows)) for s in segs]
            o, l = ao.shard_attention(q_all[mine], k_all[kv_rows], v_all[kv_rows], sj,
                                      hq, hkv, 0.5, kv_pos=np.asarray(kv_rows))
            os_.append(o)
            ls_.append(l)
        mo, _ = ao.lse_merge(np.stack(os_), np.stack(ls_))
        assert np.max(np.abs(mo - dense[mine])) < 1e-12


def test_decode_shards_merge_to_dense():
    """Decode CP: KV token i stored on shard i mod W; each shard gives a
    partial for the new query (which sees the whole context); merged equals
    attention over the whole context (torch SDPA, no mask)."""
    W, ctx, hq, d, dv = 4, 37, 8, 6, 4
    rng = np.random.default_rng(9)
    q = _rand(rng, 1, hq, d)
    kv = _rand(rng, ctx, 1, d)
    v = kv[:, :, :dv]                       # V is a prefix of the latent K
    ref = F.scaled_dot_product_attention(
        torch.tensor(q).permute(1, 0, 2)[None], torch.tensor(kv).permute(1, 0, 2)[None],
        torch.tensor(v).permute(1, 0, 2)[None], scale=0.2,
        enable_gqa=True)[0].permute(1, 0, 2).numpy()
    os_, ls_ = [], []
    for j in range(W):
        keys = np.arange(j, ctx, W)
        seg = [ix.Segment(0, 0, 1, ctx, 1, 0, len(keys))]
        o, l = ao.shard_attention(q, kv[keys], v[keys], seg, hq, 1, 0.2, kv_pos=keys)
        os_.append(o)
        ls_.append(l)
    mo, _ = ao.lse_merge(np.stack(os_), np.stack(ls_))
    assert np.max(np.abs(mo - ref)) < 1e-12

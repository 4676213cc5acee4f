"""GPU parity of cp_attn_fwd against the oracle on small shapes: several
tiles with ragged tails, every kernel variant, zigzag and interleave with
cached prefixes, GQA, explicit key positions (ring partials), empty rows,
non-causal, fp32 output."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
from oracle import attn_oracle as ao
from oracle import index_oracle as ix
from gpu_helpers import compare, f64, oracle_segments, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _tensors(n_new, n_kv, hq, hkv, dqk, dv, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn((n_new, hq, dqk), generator=g, device=DEV).to(td)
    k = torch.randn((n_kv, hkv, dqk), generator=g, device=DEV).to(td)
    v = torch.randn((n_kv, hkv, dv), generator=g, device=DEV).to(td)
    return q, k, v


CASES = [
    # strategy, C, lens, prefixes, hq, hkv, dqk, dv, dtype
    ("zigzag", 2, [300, 77], [50, 0], 8, 2, 128, 128, "bf16"),
    ("zigzag", 3, [517], [33], 4, 4, 192, 128, "bf16"),
    ("interleave", 4, [5, 3, 200, 130], [0, 7, 100, 0], 4, 1, 64, 64, "bf16"),
    ("interleave", 3, [129, 1, 260], [300, 0, 5], 8, 8, 192, 128, "bf16"),
    ("zigzag", 4, [256], [0], 4, 4, 64, 64, "f32"),
    ("interleave", 2, [70, 131], [3, 40], 4, 2, 128, 128, "f32"),
    ("zigzag", 1, [190], [0], 2, 1, 128, 128, "bf16"),
    # GQA packing (4 query heads of one KV head per workgroup): 4 and 8 per group
    ("zigzag", 2, [700, 45], [60, 0], 16, 4, 192, 128, "bf16"),
    ("interleave", 3, [260, 1, 515], [0, 30, 7], 8, 1, 128, 128, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-C{c[1]}-{c[6]}x{c[7]}-{c[8]}" for c in CASES])
def test_shard_attention_small(case):
    strategy, C, lens, pre, hq, hkv, dqk, dv, dtype = case
    n_new, n_kv = sum(lens), sum(p + t for p, t in zip(pre, lens))
    q, k, v = _tensors(n_new, n_kv, hq, hkv, dqk, dv, dtype, seed=sum(lens) + C)
    k64, v64, q64 = f64(k), f64(v), f64(q)
    scale = 1.0 / np.sqrt(dqk)
    for r in range(C):
        say(f"attn {strategy} C={C} r={r} lens={lens} pre={pre} heads={hq}/{hkv} d={dqk}/{dv} {dtype}")
        plan = cp.shard_plan(strategy, C, r, lens, pre)
        if plan.num_local == 0:
            continue
        gidx = torch.from_numpy(plan.global_idx.astype(np.int64)).to(DEV)
        o, lse = cp.attn_fwd(q.index_select(0, gidx), k, v, plan, scale)
        torch.cuda.synchronize()
        toks = ix.rank_tokens(strategy, C, r, lens, pre)
        segs = oracle_segments(strategy, C, r, lens, pre)
        ro, rl = ao.shard_attention(q64[[t.g for t in toks]], k64, v64, segs, hq, hkv, scale)
        compare(f64(o), f64(lse), ro, rl, range(plan.num_local), dtype, f"rank {r}")


@pytest.mark.parametrize("dqk,dv", [(192, 128), (128, 128), (64, 64)])
def test_ring_partials_with_key_positions(dqk, dv):
    """Rank r's queries against rank j's zigzag KV pair, masked by explicit
    key positions; partials vs oracle, merged vs dense."""
    C, T, H = 4, 640, 2
    q, k, v = _tensors(T, T, H, H, dqk, dv, "bf16", seed=dqk + dv)
    q64, k64, v64 = f64(q), f64(k), f64(v)
    scale = 1.0 / np.sqrt(dqk)
    for r in (0, 3):
        plan = cp.shard_plan("zigzag", C, r, [T], [0])
        mine = plan.global_idx.astype(np.int64)
        q_loc = q.index_select(0, torch.from_numpy(mine).to(DEV))
        o_parts, l_parts = [], []
        for j in range(C):
            say(f"ring d={dqk}/{dv} rank {r} kv pair {j}")
            rows_j = cp.shard_plan("zigzag", C, j, [T], [0]).global_idx.astype(np.int64)
            idx = torch.from_numpy(rows_j).to(DEV)
            kj, vj = k.index_select(0, idx), v.index_select(0, idx)
            kv_pos = idx.to(torch.int32)
            segs = [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, len(rows_j))
                    for s in plan.segments]
            o, l = cp.attn_fwd(q_loc, kj, vj, segs, scale, kv_pos=kv_pos)
            torch.cuda.synchronize()
            osegs = [ix.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0,
                                len(rows_j)) for s in oracle_segments("zigzag", C, r, [T], [0])]
            ro, rl = ao.shard_attention(q64[mine], k64[rows_j], v64[rows_j], osegs, H, H, scale,
                                        kv_pos=rows_j)
            compare(f64(o), f64(l), ro, rl, range(len(mine)), "bf16", f"partial {j}")
            o_parts.append(o)
            l_parts.append(l)
        mo, ml = cp.lse_merge(torch.stack(o_parts), torch.stack(l_parts))
        torch.cuda.synchronize()
        dense_o, dense_l = ao.shard_attention(q64[mine], k64, v64,
                                              oracle_segments("zigzag", C, r, [T], [0]), H, H, scale)
        compare(f64(mo), f64(ml), dense_o, dense_l, range(len(mine)), "bf16", "merged")


@pytest.mark.parametrize("case", ["ring-diagonal", "zigzag-prefix", "interleave-varlen", "split"])
def test_segment_order_invariant(case):
    """The planner reorders a launch's segments (most keys first; among
    equal key ranges of a causal call, later positions first).  Passing the
    segments in the opposite order must give bit-identical O and LSE: every
    row is computed by one workgroup over the same tiles whatever the order."""
    H, dqk, dv = 4, 192, 128
    scale = 1.0 / np.sqrt(dqk)
    kv_pos = None
    if case == "ring-diagonal":      # rank 0's own zigzag pair: equal key ranges
        C, T = 4, 2048
        q, k, v = _tensors(T, T, H, H, dqk, dv, "bf16", seed=61)
        plan = cp.shard_plan("zigzag", C, 0, [T], [0])
        idx = torch.from_numpy(plan.global_idx.astype(np.int64)).to(DEV)
        q, k, v, kv_pos = q.index_select(0, idx), k.index_select(0, idx), v.index_select(0, idx), \
            idx.to(torch.int32)
        segs = [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, plan.num_local)
                for s in plan.segments]
    elif case == "split":            # small call: keys split into chunks
        q, k, v = _tensors(600, 5000, H, H, dqk, dv, "bf16", seed=62)
        segs = [cp.Segment(0, 0, 300, 2200, 1, 0, 2500), cp.Segment(1, 300, 600, 2200, 1, 2500, 5000)]
    else:
        strategy = "zigzag" if case == "zigzag-prefix" else "interleave"
        lens, pre = ([3000], [500]) if strategy == "zigzag" else ([700, 5, 1300, 2000], [100, 0, 900, 0])
        C = 2 if strategy == "zigzag" else 3
        n_kv = sum(lens) + sum(pre)
        q, k, v = _tensors(sum(lens), n_kv, H, 2, dqk, dv, "bf16", seed=63)
        plan = cp.shard_plan(strategy, C, 1, lens, pre)
        q = q.index_select(0, torch.from_numpy(plan.global_idx.astype(np.int64)).to(DEV))
        segs = plan.segments
    say(f"segment order {case}: {len(segs)} segments")
    o1, l1 = cp.attn_fwd(q, k, v, list(segs), scale, kv_pos=kv_pos)
    o2, l2 = cp.attn_fwd(q, k, v, list(segs)[::-1], scale, kv_pos=kv_pos)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_kv_segment_and_noncausal_and_f32_out():
    hq = hkv = 2
    q, k, v = _tensors(40, 64, hq, hkv, 128, 128, "bf16", seed=5)
    q64, k64, v64 = f64(q), f64(k), f64(v)
    segs = [cp.Segment(0, 0, 10, 0, 1, 0, 0),       # sees no KV row at all
            cp.Segment(1, 10, 40, 3, 2, 5, 64)]     # stride-2 positions
    say("empty-kv segment + causal, bf16 out")
    o, l = cp.attn_fwd(q, k, v, segs, 0.1)
    torch.cuda.synchronize()
    osegs = [ix.Segment(*s.astuple()) for s in segs]
    ro, rl = ao.shard_attention(q64, k64, v64, osegs, hq, hkv, 0.1)
    compare(f64(o), f64(l), ro, rl, range(40), "bf16", "causal")
    say("non-causal, fp32 out")
    o, l = cp.attn_fwd(q, k, v, segs, 0.1, causal=False, o_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = ao.shard_attention(q64, k64, v64, osegs, hq, hkv, 0.1, causal=False)
    compare(f64(o), f64(l), ro, rl, range(40), "bf16", "non-causal")


def test_zero_query_closed_form_small():
    """q = 0: every visible score is 0, so LSE = ln(#visible keys)."""
    lens, pre, C = [1000, 37], [200, 5], 2
    for dqk, dv in [(128, 128), (192, 128), (64, 64)]:
        _, k, v = _tensors(1, sum(p + t for p, t in zip(pre, lens)), 4, 2, dqk, dv, "bf16", 3)
        for r in range(C):
            plan = cp.shard_plan("zigzag", C, r, lens, pre)
            q = torch.zeros((plan.num_local, 4, dqk), device=DEV, dtype=torch.bfloat16)
            o, l = cp.attn_fwd(q, k, v, plan, 0.3)
            torch.cuda.synchronize()
            want = np.log(plan.positions.astype(np.float64) + 1.0)
            assert np.max(np.abs(f64(l) - want[:, None])) < 1e-3


def test_repeatable_bitwise():
    q, k, v = _tensors(300, 300, 4, 4, 192, 128, "bf16", seed=11)
    plan = cp.shard_plan("zigzag", 1, 0, [300], [0])
    a = cp.attn_fwd(q, k, v, plan, 0.07)
    b = cp.attn_fwd(q, k, v, plan, 0.07)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


GROWTH = [(300, 4, 4, 0.1, 1, 192), (300, 4, 4, 0.5, 1, 192), (4096, 128, 128, 0.5, 1, 192),
          (300, 4, 4, 0.36, 1, 192), (4096, 128, 128, 0.23, 2, 192),
          (4096, 128, 128, 0.146, 1, 128), (4096, 128, 128, 0.5415, 1, 128),
          (300, 8, 2, 0.36, 1, 192), (4096, 128, 32, 0.5, 1, 192), (4096, 64, 16, 0.146, 1, 128)]
GROWTH_IDS = ["small-2^27", "small-2^138", "large-2^138", "small-2^100", "large-2x2^63.6",
              "large-d128-2^27", "large-d128-2^100", "small-gqa-2^100", "large-gqa-2^138",
              "large-gqa-d128-2^27"]


@pytest.mark.parametrize("accumulate", [False, True], ids=["write", "accumulate"])
@pytest.mark.parametrize("rows,hq,hkv,val,nbig,dqk", GROWTH, ids=GROWTH_IDS)
def test_reference_growth(rows, hq, hkv, val, nbig, dqk, accumulate):
    """Keys, in a late tile, far above every score of the first tile: with
    q = 1 and keys 0 except keys 900.. = val (d dims, scale 1) the row max
    grows by d*val*log2(e) in log2 units -- 2^27 (kept by the main pass),
    2^100 or 2^138 (probabilities above 2^64, or beyond fp32 range: the
    workgroup is flagged and recomputed), or twice 2^63.6 (no probability
    above 2^64 but a row sum above it: flagged as well).  128-row and
    256-row workgroups (4096 rows x 128 heads: the split-role main pass, at
    qk 192 and 128); the plain definition decides.
    accumulate: keys 0..449 are first written by a plain call, then keys
    450..999 (with the large ones) are merged into that running (O, LSE) by
    an accumulating call; a flagged workgroup must merge exactly once (in
    the exact pass), which the dense result over all keys checks.
    hkv < hq: GQA packing puts 4 query heads of one KV head in a workgroup;
    every fourth query head has q = 0 (no growth), so a flagged workgroup
    holds heads that would not have been flagged on their own."""
    n_kv, dv = 1000, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(rows + hq)
    q = torch.ones((rows, hq, dqk), device=DEV, dtype=torch.bfloat16)
    if hkv < hq:
        q[:, 1::4] = 0
    k = torch.zeros((n_kv, hkv, dqk), device=DEV, dtype=torch.bfloat16)
    k[900:900 + nbig] = val
    v = torch.randn((n_kv, hkv, dv), generator=g, device=DEV).to(torch.bfloat16)
    say(f"reference growth rows={rows} hq={hq} hkv={hkv} val={val} keys={nbig} accumulate={accumulate}")
    if not accumulate:
        # every row sees all keys (positions n_kv .. n_kv + rows - 1)
        segs = [cp.Segment(0, 0, rows, n_kv, 1, 0, n_kv)]
        o, lse = cp.attn_fwd(q, k, v, segs, 1.0)
    else:
        cut = 450
        pos = torch.arange(n_kv, device=DEV, dtype=torch.int32)
        o, lse = cp.attn_fwd(q, k[:cut], v[:cut], [cp.Segment(0, 0, rows, n_kv, 1, 0, cut)], 1.0,
                             kv_pos=pos[:cut].contiguous())
        cp.attn_fwd(q, k[cut:], v[cut:], [cp.Segment(0, 0, rows, n_kv, 1, 0, n_kv - cut)], 1.0,
                    kv_pos=pos[cut:].contiguous(), o=o, lse=lse, accumulate=True)
    torch.cuda.synchronize()
    sample = sorted(set([0, 1, rows // 2, rows - 1]))
    q64, k64, v64 = f64(q), f64(k), f64(v)
    for h in sorted(set([0, 1, hq - 1])):
        kh = h // (hq // hkv)
        ro, rl = ao.attend(q64[sample, h], k64[:, kh], v64[:, kh], [n_kv + i for i in sample],
                           np.arange(n_kv), 1.0)
        compare(f64(o[sample, h]), f64(lse[sample, h]), ro, rl, range(len(sample)), "bf16",
                f"head {h}")


@pytest.mark.parametrize("rows,hq", [(300, 4), (4096, 128)], ids=["128-row", "256-row"])
def test_huge_values_overflow_guard(rows, hq):
    """Probabilities within the main pass's range (a key 2^60 above the
    first tile's scores) times value rows near 2^70 overflow an fp32
    accumulator (2^130) although the exact output, a convex combination of
    V rows, is finite: the workgroup must be flagged and recomputed.  Values
    are O(2^70), so O is compared after scaling by 2^-70 (the output is
    linear in V), with the bf16 tolerance."""
    n_kv, dqk, dv, big = 1000, 192, 128, 2.0 ** 70
    g = torch.Generator(device=DEV)
    g.manual_seed(7 + rows)
    q = torch.ones((rows, hq, dqk), device=DEV, dtype=torch.bfloat16)
    k = torch.zeros((n_kv, hq, dqk), device=DEV, dtype=torch.bfloat16)
    k[900] = 0.2166          # bf16 0.216797: growth 192 * 0.216797 * log2(e) = 2^60.05
    v = torch.randn((n_kv, hq, dv), generator=g, device=DEV)
    v[880:920] *= big        # the large key's row and its neighbours
    v = v.to(torch.bfloat16)
    segs = [cp.Segment(0, 0, rows, n_kv, 1, 0, n_kv)]
    say(f"huge values rows={rows} hq={hq}")
    o, lse = cp.attn_fwd(q, k, v, segs, 1.0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()), "non-finite O"
    sample = sorted(set([0, 1, rows // 2, rows - 1]))
    q64, k64, v64 = f64(q), f64(k), f64(v)
    for h in sorted(set([0, hq - 1])):
        ro, rl = ao.attend(q64[sample, h], k64[:, h], v64[:, h], [n_kv + i for i in sample],
                           np.arange(n_kv), 1.0)
        compare(f64(o[sample, h]) / big, f64(lse[sample, h]), ro / big, rl, range(len(sample)),
                "bf16", f"head {h} (O / 2^70)")


@pytest.mark.parametrize("dqk,dv,dtype,odt,C,T,H,HK", [
    (192, 128, "bf16", torch.float32, 4, 640, 2, 2),       # 128-row workgroups
    (128, 128, "bf16", torch.bfloat16, 4, 640, 2, 2),
    (192, 128, "bf16", torch.float32, 2, 2048, 128, 128),  # 256-row workgroups
    (128, 128, "bf16", torch.bfloat16, 2, 2048, 128, 128),
    (192, 128, "bf16", torch.float32, 2, 2048, 128, 32),   # GQA packing, 4 heads x 64 rows
    (128, 128, "bf16", torch.bfloat16, 2, 2048, 64, 8),
    (64, 64, "f32", torch.float32, 4, 256, 4, 4),          # fp32 kernel
], ids=["192-f32acc", "128-bf16acc", "192-f32acc-256rows", "128-bf16acc-256rows",
        "192-f32acc-gqa-packed", "128-bf16acc-gqa-packed", "fp32"])
def test_ring_accumulate_in_place(dqk, dv, dtype, odt, C, T, H, HK):
    """Pass-Q style running accumulator: the C ring partials of a rank merged
    in the attention epilogue (accumulate=1), starting from an empty (LSE =
    -inf) accumulator, must equal the dense attention of the rank's rows;
    partial calls whose rows see no key leave the accumulator untouched."""
    q, k, v = _tensors(T, T, H, HK, dqk, dv, dtype, seed=dqk + C)
    q64, k64, v64 = f64(q), f64(k), f64(v)
    scale = 1.0 / np.sqrt(dqk)
    for r in sorted({0, C - 1}):
        plan = cp.shard_plan("zigzag", C, r, [T], [0])
        mine = plan.global_idx.astype(np.int64)
        q_loc = q.index_select(0, torch.from_numpy(mine).to(DEV))
        o = torch.full((len(mine), H, dv), 7.0, device=DEV, dtype=odt)   # not read while LSE = -inf
        lse = torch.full((len(mine), H), -np.inf, device=DEV, dtype=torch.float32)
        for j in reversed(range(C)):
            say(f"accumulate d={dqk}/{dv} {dtype} rank {r} pair {j}")
            rows_j = cp.shard_plan("zigzag", C, j, [T], [0]).global_idx.astype(np.int64)
            idx = torch.from_numpy(rows_j).to(DEV)
            segs = [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, len(rows_j))
                    for s in plan.segments]
            cp.attn_fwd(q_loc, k.index_select(0, idx), v.index_select(0, idx), segs, scale,
                        kv_pos=idx.to(torch.int32), o=o, lse=lse, accumulate=True)
        torch.cuda.synchronize()
        dense_o, dense_l = ao.shard_attention(q64[mine], k64, v64,
                                              oracle_segments("zigzag", C, r, [T], [0]), H, HK, scale)
        compare(f64(o), f64(lse), dense_o, dense_l, range(len(mine)),
                "bf16" if dtype == "bf16" else "f32", f"rank {r} accumulated")

"""GPU parity of small bf16 calls whose key ranges are cut into chunks: each
chunk of a segment is a partial (O_s, LSE_s) in the workspace, merged by
log-sum-exp into the caller's rows.  Causal with implicit positions and a
cached prefix, explicit key positions (a ring pair), GQA, all three head
shapes, bf16 and fp32 output, non-causal, and rows that no segment covers
left as they were."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
from oracle import attn_oracle as ao
from oracle import index_oracle as ix
from gpu_helpers import compare, f64, oracle_segments, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _tensors(n_q, n_kv, hq, hkv, dqk, dv, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = torch.randn((n_q, hq, dqk), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((n_kv, hkv, dqk), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((n_kv, hkv, dv), generator=g, device=DEV).to(torch.bfloat16)
    return q, k, v


def _split_used(q, k, v, segs, o, lse, kv_pos=None, causal=True):
    """The call was planned as a split one: its workspace holds the partials
    (flags alone are 4 bytes per workgroup)."""
    a, keep = cp._lib.attn_args(q, k, v, segs, 0.1, o, lse, causal, kv_pos)
    need = cp.attn_workspace_size(a)
    del keep
    return need > 2 * o.numel() * o.element_size()


@pytest.mark.parametrize("dqk,dv,odt", [(192, 128, torch.bfloat16), (128, 128, torch.float32),
                                        (64, 64, torch.bfloat16)])
def test_split_zigzag_prefix(dqk, dv, odt):
    """Rank 0 of a zigzag CP=2 shard of 1400 new tokens after a 4000-token
    prefix (700 rows against 5400 keys), GQA 8/2."""
    lens, pre, C, r, hq, hkv = [1400], [4000], 2, 0, 8, 2
    n_kv = pre[0] + lens[0]
    q, k, v = _tensors(lens[0], n_kv, hq, hkv, dqk, dv, seed=dqk + dv)
    scale = 1.0 / np.sqrt(dqk)
    plan = cp.shard_plan("zigzag", C, r, lens, pre)
    gidx = torch.from_numpy(plan.global_idx.astype(np.int64)).to(DEV)
    q_loc = q.index_select(0, gidx)
    o = torch.empty((plan.num_local, hq, dv), device=DEV, dtype=odt)
    lse = torch.empty((plan.num_local, hq), device=DEV, dtype=torch.float32)
    assert _split_used(q_loc, k, v, plan, o, lse)
    say(f"split zigzag prefix d={dqk}/{dv} out={odt}")
    cp.attn_fwd(q_loc, k, v, plan, scale, o=o, lse=lse)
    torch.cuda.synchronize()
    toks = ix.rank_tokens("zigzag", C, r, lens, pre)
    segs = oracle_segments("zigzag", C, r, lens, pre)
    ro, rl = ao.shard_attention(f64(q)[[t.g for t in toks]], f64(k), f64(v), segs, hq, hkv, scale)
    compare(f64(o), f64(lse), ro, rl, range(plan.num_local), "bf16", "split")


def test_split_ring_pair_key_positions():
    """Rank 0's queries of a zigzag CP=4 shard of 8192 tokens against rank
    2's KV pair (4096 keys with explicit positions), 4 heads."""
    C, T, H, dqk, dv = 4, 8192, 4, 128, 128
    q, k, v = _tensors(T, T, H, H, dqk, dv, seed=11)
    scale = 1.0 / np.sqrt(dqk)
    plan = cp.shard_plan("zigzag", C, 0, [T], [0])
    mine = plan.global_idx.astype(np.int64)
    q_loc = q.index_select(0, torch.from_numpy(mine).to(DEV))
    rows_j = cp.shard_plan("zigzag", C, 2, [T], [0]).global_idx.astype(np.int64)
    idx = torch.from_numpy(rows_j).to(DEV)
    kj, vj, kv_pos = k.index_select(0, idx), v.index_select(0, idx), idx.to(torch.int32)
    segs = [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, len(rows_j))
            for s in plan.segments]
    o = torch.empty((len(mine), H, dv), device=DEV, dtype=torch.bfloat16)
    lse = torch.empty((len(mine), H), device=DEV, dtype=torch.float32)
    assert _split_used(q_loc, kj, vj, segs, o, lse, kv_pos)
    say("split ring pair with key positions")
    cp.attn_fwd(q_loc, kj, vj, segs, scale, kv_pos=kv_pos, o=o, lse=lse)
    torch.cuda.synchronize()
    osegs = [ix.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, len(rows_j))
             for s in oracle_segments("zigzag", C, 0, [T], [0])]
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.integers(0, len(mine), 300), [0, len(mine) - 1]]))
    ro, rl = ao.shard_attention(f64(q_loc), f64(kj), f64(vj), osegs, H, H, scale, kv_pos=rows_j,
                                rows=rows)
    compare(f64(o), f64(lse), ro, rl, rows, "bf16", "split ring pair")


def test_split_noncausal_and_untouched_rows():
    """A non-causal segment of 500 rows against 3000 keys inside an output
    of 640 rows: rows 500..639 keep what they held."""
    H, dqk, dv, n_q, n_kv = 4, 128, 128, 640, 3000
    q, k, v = _tensors(n_q, n_kv, H, H, dqk, dv, seed=21)
    segs = [cp.Segment(0, 0, 500, 0, 1, 0, n_kv)]
    o = torch.full((n_q, H, dv), 7.0, device=DEV, dtype=torch.bfloat16)
    lse = torch.full((n_q, H), 3.0, device=DEV, dtype=torch.float32)
    assert _split_used(q, k, v, segs, o, lse, causal=False)
    say("split non-causal, untouched rows")
    cp.attn_fwd(q, k, v, segs, 0.05, causal=False, o=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = ao.shard_attention(f64(q), f64(k), f64(v), [ix.Segment(0, 0, 500, 0, 1, 0, n_kv)],
                                H, H, 0.05, causal=False)
    compare(f64(o), f64(lse), ro, rl, range(500), "bf16", "non-causal")
    assert torch.all(o[500:] == 7.0) and torch.all(lse[500:] == 3.0)


def test_split_repeatable_bitwise():
    H, dqk, dv = 4, 192, 128
    q, k, v = _tensors(300, 4000, H, H, dqk, dv, seed=31)
    segs = [cp.Segment(0, 0, 300, 3700, 1, 0, 4000)]
    o1, l1 = cp.attn_fwd(q, k, v, segs, 0.07)
    o2, l2 = cp.attn_fwd(q, k, v, segs, 0.07)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_segments_at_offsets():
    """Two requests' segments at rows [100, 400) and [500, 800) of a 900-row
    output, each against its own keys (2400 and 3000, after cached
    prefixes): the partials use compact rows, the merge writes the
    segments' rows, and the gaps keep what they held."""
    H, hkv, dqk, dv, n_q = 8, 2, 128, 128, 900
    n_kv = 2400 + 3000
    q, k, v = _tensors(n_q, n_kv, H, hkv, dqk, dv, seed=41)
    segs = [cp.Segment(0, 100, 400, 2100, 1, 0, 2400),        # positions 2100..2399
            cp.Segment(1, 500, 800, 2700, 1, 2400, 5400)]     # positions 2700..2999
    o = torch.full((n_q, H, dv), -5.0, device=DEV, dtype=torch.float32)
    lse = torch.full((n_q, H), 9.0, device=DEV, dtype=torch.float32)
    assert _split_used(q, k, v, segs, o, lse)
    say("split segments at row offsets")
    cp.attn_fwd(q, k, v, segs, 0.09, o=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = ao.shard_attention(f64(q), f64(k), f64(v), [ix.Segment(*s.astuple()) for s in segs],
                                H, hkv, 0.09)
    rows = list(range(100, 400)) + list(range(500, 800))
    compare(f64(o), f64(lse), ro, rl, rows, "bf16", "segments at offsets")
    gap = torch.cat([torch.arange(0, 100), torch.arange(400, 500), torch.arange(800, 900)]).to(DEV)
    assert torch.all(o[gap] == -5.0) and torch.all(lse[gap] == 9.0)

"""GPU parity on seeded random configurations: strategy, CP size and rank,
request lengths and cached prefixes, GQA ratio, head dims, input and output
dtype, and (zigzag) one ring pair with explicit key positions; every row of
the rank against the oracle.  Shapes stay small enough for the fp64 oracle
to finish in seconds."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
from oracle import attn_oracle as ao
from oracle import index_oracle as ix
from gpu_helpers import compare, f64, oracle_segments, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _config(seed):
    rng = np.random.default_rng(1000 + seed)
    strategy = ("zigzag", "interleave")[int(rng.integers(0, 2))]
    C = int(rng.choice([1, 2, 3, 4, 5, 8]))
    B = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(1, 700, size=B)]
    pre = [int(x) if rng.random() < 0.6 else 0 for x in rng.integers(0, 300, size=B)]
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    dims = [(64, 64), (128, 128)] if dtype == "f32" else [(64, 64), (128, 128), (192, 128)]
    dqk, dv = dims[int(rng.integers(0, len(dims)))]
    hkv = int((1, 2, 4)[int(rng.integers(0, 3))])
    hq = hkv * int((1, 2, 4)[int(rng.integers(0, 3))])
    r = int(rng.integers(0, C))
    out_f32 = dtype == "bf16" and rng.random() < 0.3
    ring = strategy == "zigzag" and C > 1 and rng.random() < 0.5
    j = int(rng.integers(0, C))
    return strategy, C, lens, pre, hq, hkv, dqk, dv, dtype, r, out_f32, ring, j


@pytest.mark.parametrize("seed", range(32))
def test_random_config(seed):
    strategy, C, lens, pre, hq, hkv, dqk, dv, dtype, r, out_f32, ring, j = _config(seed)
    say(f"random {seed}: {strategy} C={C} r={r} lens={lens} pre={pre} heads={hq}/{hkv} "
        f"d={dqk}/{dv} {dtype} out_f32={out_f32} ring={ring and j}")
    n_new = sum(lens)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn((n_new, hq, dqk), generator=g, device=DEV).to(td)
    scale = 1.0 / np.sqrt(dqk)
    plan = cp.shard_plan(strategy, C, r, lens, pre)
    if plan.num_local == 0:
        return
    gidx = plan.global_idx.astype(np.int64)
    q_loc = q.index_select(0, torch.from_numpy(gidx).to(DEV))
    odt = torch.float32 if out_f32 else None
    if not ring:
        n_kv = sum(p + t for p, t in zip(pre, lens))
        k = torch.randn((n_kv, hkv, dqk), generator=g, device=DEV).to(td)
        v = torch.randn((n_kv, hkv, dv), generator=g, device=DEV).to(td)
        o, lse = cp.attn_fwd(q_loc, k, v, plan, scale, o_dtype=odt)
        torch.cuda.synchronize()
        toks = ix.rank_tokens(strategy, C, r, lens, pre)
        segs = oracle_segments(strategy, C, r, lens, pre)
        ro, rl = ao.shard_attention(f64(q)[[t.g for t in toks]], f64(k), f64(v), segs, hq, hkv, scale)
    else:
        # one request without prefix: rank j's zigzag pair as the KV buffer
        T = lens[0]
        plan = cp.shard_plan("zigzag", C, r, [T], [0])
        if plan.num_local == 0:
            return
        gidx = plan.global_idx.astype(np.int64)
        q_loc = q.index_select(0, torch.from_numpy(gidx).to(DEV))
        k = torch.randn((T, hkv, dqk), generator=g, device=DEV).to(td)
        v = torch.randn((T, hkv, dv), generator=g, device=DEV).to(td)
        rows_j = cp.shard_plan("zigzag", C, j, [T], [0]).global_idx.astype(np.int64)
        idx = torch.from_numpy(rows_j).to(DEV)
        segs_j = [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, len(rows_j))
                  for s in plan.segments]
        o, lse = cp.attn_fwd(q_loc, k.index_select(0, idx), v.index_select(0, idx), segs_j, scale,
                             kv_pos=idx.to(torch.int32), o_dtype=odt)
        torch.cuda.synchronize()
        osegs = [ix.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, len(rows_j))
                 for s in oracle_segments("zigzag", C, r, [T], [0])]
        ro, rl = ao.shard_attention(f64(q)[gidx], f64(k)[rows_j], f64(v)[rows_j], osegs, hq, hkv,
                                    scale, kv_pos=rows_j)
    compare(f64(o), f64(lse), ro, rl, range(plan.num_local), dtype, f"seed {seed}")

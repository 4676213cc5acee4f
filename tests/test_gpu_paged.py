"""GPU parity of the decode shard over a paged KV cache with the block-level
interleave (token i on rank (i // block) mod W): every rank's logical rows
are scattered over a randomly allocated pool of blocks, the rest of the pool
holds NaN.  The paged call must equal, bit for bit, the same call on the
rank's rows laid out contiguously, match the oracle per rank, and merge over
the ranks into full attention."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
import workloads
from oracle import attn_oracle as ao
from gpu_helpers import compare, f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
DQK, DV = 576, 512


def _rank_keys(ctx, W, j, bs):
    i = np.arange(ctx)
    return i[(i // bs) % W == j]


class _Paged:
    """Rank j's shard of kv [B, ctx, 576] in a paged pool, plus the same rows
    laid out contiguously (request after request)."""

    def __init__(self, kv, W, j, bs, spare=5, seed=0):
        B, ctx, _ = kv.shape
        self.keys = _rank_keys(ctx, W, j, bs)
        n = len(self.keys)
        self.n, self.bs = n, bs
        table, pool_row, nblocks = workloads.paged_layout([n] * B, bs, spare, seed)
        self.table = torch.from_numpy(table).to(DEV)
        stride = table.shape[1]
        pool = torch.full((nblocks * bs, DQK), float("nan"), device=DEV, dtype=kv.dtype)
        src = torch.from_numpy((np.arange(B)[:, None] * ctx + self.keys[None, :]).reshape(-1)).to(DEV)
        dst = torch.from_numpy(pool_row[:, :n].reshape(-1)).to(DEV)
        flat = kv.reshape(B * ctx, DQK)
        pool[dst] = flat[src]
        self.k = pool.view(nblocks * bs, 1, DQK)
        pos = np.full((B, stride * bs), 1 << 30, dtype=np.int32)
        pos[:, :n] = self.keys
        self.pos = torch.from_numpy(pos.reshape(-1)).to(DEV)
        self.kc = flat[src].view(B * n, 1, DQK)
        self.pos_c = torch.from_numpy(np.tile(self.keys, B).astype(np.int32)).to(DEV)

    def run(self, q, q_pos, scale, kv_lo=0, o=None, lse=None, accumulate=False,
            o_dtype=torch.float32):
        B = q.shape[0]
        segs = [cp.Segment(b, b, b + 1, int(q_pos[b]), 1, kv_lo, self.n) for b in range(B)]
        return cp.attn_fwd(q, self.k, self.k[:, :, :DV], segs, scale, kv_pos=self.pos,
                           o=o, lse=lse, accumulate=accumulate, o_dtype=o_dtype,
                           block_table=self.table, block_size=self.bs)

    def run_contiguous(self, q, q_pos, scale, kv_lo=0):
        B = q.shape[0]
        segs = [cp.Segment(b, b, b + 1, int(q_pos[b]), 1, b * self.n + kv_lo, (b + 1) * self.n)
                for b in range(B)]
        return cp.attn_fwd(q, self.kc, self.kc[:, :, :DV], segs, scale, kv_pos=self.pos_c,
                           o_dtype=torch.float32)


def _inputs(B, ctx, hq, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = torch.randn((B, hq, DQK), generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn((B, ctx, DQK), generator=g, device=DEV).to(torch.bfloat16)
    return q, kv


@pytest.mark.parametrize("B,ctx,W,bs,hq", [(3, 1000, 4, 128, 128), (2, 1500, 2, 32, 16),
                                           (1, 5000, 1, 256, 160), (2, 777, 3, 64, 128)])
def test_paged_block_interleave(B, ctx, W, bs, hq):
    say(f"paged decode B={B} ctx={ctx} W={W} block={bs} hq={hq}")
    q, kv = _inputs(B, ctx, hq, ctx + bs)
    scale = 1.0 / np.sqrt(DQK)
    # the first request decodes the next token; the others sit earlier in
    # the context, so the causal mask cuts into the shard
    q_pos = [ctx] + [ctx - 1 - 211 * b for b in range(1, B)]
    q64, kv64 = f64(q), f64(kv)
    outs = []
    for j in range(W):
        pg = _Paged(kv, W, j, bs, seed=j)
        o, l = pg.run(q, q_pos, scale)
        oc, lc = pg.run_contiguous(q, q_pos, scale)
        torch.cuda.synchronize()
        assert torch.equal(o, oc) and torch.equal(l, lc), f"rank {j}: paged != contiguous"
        for b in range(B):
            ro, rl = ao.attend(q64[b], kv64[b, pg.keys], kv64[b, pg.keys, :DV], [q_pos[b]] * hq,
                               pg.keys, scale)
            compare(f64(o[b]), f64(l[b]), ro, rl, range(hq), "bf16", f"rank {j} req {b}")
        outs.append((o, l))
    mo, ml = cp.lse_merge(torch.stack([o for o, _ in outs]), torch.stack([l for _, l in outs]))
    torch.cuda.synchronize()
    for b in range(B):
        keys = np.arange(ctx)
        ro, rl = ao.attend(q64[b], kv64[b], kv64[b, :, :DV], [q_pos[b]] * hq, keys, scale)
        compare(f64(mo[b]), f64(ml[b]), ro, rl, range(hq), "bf16", f"merged req {b}")


def test_paged_kv_offset_and_accumulate():
    """Segments that start inside the request's logical rows (kv_begin = 64),
    and the ranks' partials accumulated in place into one running (O, LSE)."""
    B, ctx, W, bs, hq = 2, 2000, 4, 64, 128
    q, kv = _inputs(B, ctx, hq, 77)
    scale = 1.0 / np.sqrt(DQK)
    q_pos = [ctx, ctx]
    q64, kv64 = f64(q), f64(kv)
    say("paged decode kv_begin=64")
    pg = _Paged(kv, W, 1, bs, seed=3)
    o, l = pg.run(q, q_pos, scale, kv_lo=64)
    oc, lc = pg.run_contiguous(q, q_pos, scale, kv_lo=64)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(l, lc)
    keys = pg.keys[64:]
    for b in range(B):
        ro, rl = ao.attend(q64[b], kv64[b, keys], kv64[b, keys, :DV], [ctx] * hq, keys, scale)
        compare(f64(o[b]), f64(l[b]), ro, rl, range(hq), "bf16", f"offset req {b}")
    say("paged decode accumulate over ranks")
    o = torch.zeros((B, hq, DV), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((B, hq), -np.inf, device=DEV, dtype=torch.float32)
    for j in range(W):
        _Paged(kv, W, j, bs, seed=10 + j).run(q, q_pos, scale, o=o, lse=lse, accumulate=True)
    torch.cuda.synchronize()
    for b in range(B):
        ro, rl = ao.attend(q64[b], kv64[b], kv64[b, :, :DV], [ctx] * hq, np.arange(ctx), scale)
        compare(f64(o[b]), f64(lse[b]), ro, rl, range(hq), "bf16", f"accumulated req {b}")


def test_paged_decode_mla_b64_block128():
    """The 64-request x 131072-context decode workload with the cache
    interleaved over 8 ranks in blocks of 128 tokens: ranks 0 and 7 paged vs
    contiguous (bit for bit) and two requests per rank against the oracle."""
    w = workloads.get("decode_mla_b64")
    q, kv = workloads.decode_tensors(w, DEV)
    W, bs, ctx = w.cp_size, 128, w.ctx_len
    q_pos = [ctx] * w.num_reqs
    for j in (0, W - 1):
        say(f"paged decode_mla_b64 rank {j}")
        pg = _Paged(kv, W, j, bs, spare=64, seed=100 + j)
        o, l = pg.run(q, q_pos, w.scale)
        oc, lc = pg.run_contiguous(q, q_pos, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, oc) and torch.equal(l, lc), f"rank {j}: paged != contiguous"
        for b in (0, w.num_reqs - 1):
            qb, kb = f64(q[b]), f64(kv[b, pg.keys])
            ro, rl = ao.attend(qb, kb, kb[:, :DV], [ctx] * w.hq, pg.keys, w.scale)
            compare(f64(o[b]), f64(l[b]), ro, rl, range(w.hq), "bf16", f"rank {j} req {b}")
        del pg
        torch.cuda.empty_cache()


def test_paged_gqa_empty_and_invisible():
    """Two latent KV heads (64 query heads each) in one paged pool, an empty
    segment, and a query that sits before every key of the rank: the empty
    and the invisible rows get O = 0, LSE = -inf; the others match the
    oracle and the same call on contiguous rows bit for bit."""
    B, ctx, W, j, bs, hq, hkv = 3, 1200, 2, 1, 64, 128, 2
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    q = torch.randn((B, hq, DQK), generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn((B, ctx, hkv, DQK), generator=g, device=DEV).to(torch.bfloat16)
    scale = 1.0 / np.sqrt(DQK)
    keys = _rank_keys(ctx, W, j, bs)          # rank 1 of 2: blocks 1, 3, 5, ...
    n = len(keys)
    table, pool_row, nblocks = workloads.paged_layout([n] * B, bs, 3, 5)
    stride = table.shape[1]
    pool = torch.full((nblocks * bs, hkv, DQK), float("nan"), device=DEV, dtype=kv.dtype)
    src = torch.from_numpy((np.arange(B)[:, None] * ctx + keys[None, :]).reshape(-1)).to(DEV)
    flat = kv.reshape(B * ctx, hkv, DQK)
    pool[torch.from_numpy(pool_row[:, :n].reshape(-1)).to(DEV)] = flat[src]
    pos = np.full((B, stride * bs), 1 << 30, dtype=np.int32)
    pos[:, :n] = keys
    pos_t = torch.from_numpy(pos.reshape(-1)).to(DEV)
    # request 0: whole shard; request 1: empty range; request 2: query at
    # position 10, before the rank's first key (64)
    q_pos = [ctx, ctx, 10]
    segs = [cp.Segment(0, 0, 1, q_pos[0], 1, 0, n), cp.Segment(1, 1, 2, q_pos[1], 1, 64, 64),
            cp.Segment(2, 2, 3, q_pos[2], 1, 0, n)]
    say("paged decode GQA 2 KV heads, empty and invisible rows")
    o, l = cp.attn_fwd(q, pool, pool[:, :, :DV], segs, scale, kv_pos=pos_t, o_dtype=torch.float32,
                       block_table=torch.from_numpy(table).to(DEV), block_size=bs)
    kc = flat[src].view(B * n, hkv, DQK)
    segs_c = [cp.Segment(0, 0, 1, q_pos[0], 1, 0, n), cp.Segment(1, 1, 2, q_pos[1], 1, n + 64, n + 64),
              cp.Segment(2, 2, 3, q_pos[2], 1, 2 * n, 3 * n)]
    oc, lc = cp.attn_fwd(q, kc, kc[:, :, :DV], segs_c, scale,
                         kv_pos=torch.from_numpy(np.tile(keys, B).astype(np.int32)).to(DEV),
                         o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(l, lc)
    q64, kv64 = f64(q), f64(kv)
    G = hq // hkv
    for kvh in range(hkv):
        hs = slice(kvh * G, (kvh + 1) * G)
        ro, rl = ao.attend(q64[0, hs], kv64[0, keys, kvh], kv64[0, keys, kvh, :DV], [ctx] * G, keys,
                           scale)
        compare(f64(o[0, hs]), f64(l[0, hs]), ro, rl, range(G), "bf16", f"req 0 kv head {kvh}")
    for b in (1, 2):
        lb = f64(l[b])
        assert np.all(lb == -np.inf) and np.all(f64(o[b]) == 0), f"req {b}: not empty"


def test_paged_repeatable():
    """The same paged and contiguous shard calls, repeated: every repeat is
    bitwise equal to the first (a run-to-run difference would mean a race
    between the waves of a workgroup)."""
    B, ctx, W, bs, hq = 3, 1000, 4, 128, 128
    say("paged decode repeatability")
    q, kv = _inputs(B, ctx, hq, ctx + bs)
    scale = 1.0 / np.sqrt(DQK)
    q_pos = [ctx] + [ctx - 1 - 211 * b for b in range(1, B)]
    pg = _Paged(kv, W, 0, bs, seed=0)
    for run in (pg.run, pg.run_contiguous):
        o0, l0 = run(q, q_pos, scale)
        for rep in range(6):
            o, l = run(q, q_pos, scale)
            torch.cuda.synchronize()
            assert torch.equal(o, o0) and torch.equal(l, l0), f"{run.__name__}: repeat {rep} differs"

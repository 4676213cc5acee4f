"""GPU parity of the decode-CP shard path (MLA-absorbed latent, V = first
512 columns of K) against the oracle: small ragged shapes, partial head
blocks, several KV heads, causal masking by key position, and the full
64-request x 131072-context workload on its 8 interleaved shards + merge."""
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


def _run_shards(q, kv, W, scale, q_pos=None, causal=True):
    """Every shard j of the token-interleaved cache (token i on shard i % W):
    partial attention of each request's query over its shard.  Returns the
    list of (o_j, lse_j) and the shard key positions."""
    B, ctx, _ = kv.shape
    hq = q.shape[1]
    outs = []
    for j in range(W):
        shard = kv[:, j::W].contiguous()                 # [B, n_j, 576]
        n_j = shard.shape[1]
        k = shard.view(B * n_j, 1, DQK)
        v = k[:, :, :DV]                                 # V aliases K
        pos = torch.arange(j, ctx, W, device=DEV, dtype=torch.int32).repeat(B)
        segs = [cp.Segment(b, b, b + 1, ctx if q_pos is None else int(q_pos[b]), 1,
                           b * n_j, (b + 1) * n_j) for b in range(B)]
        o, l = cp.attn_fwd(q, k, v, segs, scale, causal=causal, kv_pos=pos,
                           o_dtype=torch.float32)
        outs.append((o, l))
    return outs


def _oracle_shard(q64, kv64, b, j, W, scale, q_pos, causal=True):
    keys = np.arange(j, kv64.shape[1], W)
    # all heads share the one latent KV head and the one query position, so
    # the heads are the rows of a single attention call
    return ao.attend(q64[b], kv64[b, keys], kv64[b, keys, :DV], [q_pos] * q64.shape[1],
                     keys, scale, causal)


# head counts that end inside a score wave's 32 heads or inside one of its
# 16-head blocks (8, 40, 100) as well as whole ones
@pytest.mark.parametrize("B,ctx,W,hq", [(3, 1000, 4, 128), (2, 777, 2, 16), (1, 4100, 1, 160),
                                        (2, 600, 1, 8), (2, 900, 2, 40), (1, 1300, 3, 100)])
def test_decode_shards_small(B, ctx, W, hq):
    say(f"decode small B={B} ctx={ctx} W={W} hq={hq}")
    g = torch.Generator(device=DEV)
    g.manual_seed(ctx + hq)
    q = torch.randn((B, hq, DQK), generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn((B, ctx, DQK), generator=g, device=DEV).to(torch.bfloat16)
    scale = 1.0 / np.sqrt(DQK)
    outs = _run_shards(q, kv, W, scale)
    torch.cuda.synchronize()
    q64, kv64 = f64(q), f64(kv)
    for j, (o, l) in enumerate(outs):
        for b in range(B):
            ro, rl = _oracle_shard(q64, kv64, b, j, W, scale, ctx)
            compare(f64(o[b]), f64(l[b]), ro, rl, range(hq), "bf16", f"shard {j} req {b}")
    mo, ml = cp.lse_merge(torch.stack([o for o, _ in outs]), torch.stack([l for _, l in outs]))
    torch.cuda.synchronize()
    for b in range(B):
        ro, rl = ao.attend(q64[b], kv64[b], kv64[b, :, :DV], [ctx] * hq, np.arange(ctx), scale)
        compare(f64(mo[b]), f64(ml[b]), ro, rl, range(hq), "bf16", f"merged req {b}")


def test_decode_causal_mask_and_gqa():
    """Queries in the middle of the context (keys after them are masked) and
    two KV heads sharing 32 query heads each."""
    B, ctx, hkv, G = 2, 1500, 2, 32
    hq = hkv * G
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    q = torch.randn((B, hq, DQK), generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn((B * ctx, hkv, DQK), generator=g, device=DEV).to(torch.bfloat16)
    v = kv[:, :, :DV]
    q_pos = [731, 1499]
    segs = [cp.Segment(b, b, b + 1, q_pos[b], 1, b * ctx, (b + 1) * ctx) for b in range(B)]
    scale = 0.05
    say("decode causal mask + 2 KV heads")
    o, l = cp.attn_fwd(q, kv, v, segs, scale, o_dtype=torch.float32)
    torch.cuda.synchronize()
    q64, kv64 = f64(q), f64(kv)
    for b in range(B):
        for kh in range(hkv):
            rows = kv64[b * ctx:(b + 1) * ctx, kh]
            ro, rl = ao.attend(q64[b, kh * G:(kh + 1) * G], rows, rows[:, :DV], [q_pos[b]] * G,
                               np.arange(ctx), scale)
            compare(f64(o[b, kh * G:(kh + 1) * G]), f64(l[b, kh * G:(kh + 1) * G]), ro, rl,
                    range(G), "bf16", f"req {b} kv head {kh}")


def test_decode_requires_v_alias():
    q = torch.zeros((1, 128, DQK), device=DEV, dtype=torch.bfloat16)
    k = torch.zeros((64, 1, DQK), device=DEV, dtype=torch.bfloat16)
    v = torch.zeros((64, 1, DV), device=DEV, dtype=torch.bfloat16)   # separate buffer
    with pytest.raises(cp.CpError) as e:
        cp.attn_fwd(q, k, v, [cp.Segment(0, 0, 1, 64, 1, 0, 64)], 0.1)
    assert e.value.status == 2


def test_decode_mla_b64_workload():
    w = workloads.get("decode_mla_b64")
    say(f"workload {w.name}")
    q, kv = workloads.decode_tensors(w, DEV)
    W = w.cp_size
    outs = _run_shards(q, kv, W, w.scale)
    mo, ml = cp.lse_merge(torch.stack([o for o, _ in outs]), torch.stack([l for _, l in outs]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    reqs = sorted(int(x) for x in rng.choice(w.num_reqs, size=4, replace=False))
    q64 = f64(q[reqs])
    for i, b in enumerate(reqs):
        kvb = f64(kv[b])[None]
        for j, (o, l) in enumerate(outs):
            ro, rl = _oracle_shard(q64[i:i + 1], kvb, 0, j, W, w.scale, w.ctx_len)
            compare(f64(o[b]), f64(l[b]), ro, rl, range(w.hq), "bf16", f"req {b} shard {j}")
        ro, rl = ao.attend(q64[i], kvb[0], kvb[0, :, :DV], [w.ctx_len] * w.hq,
                           np.arange(w.ctx_len), w.scale)
        compare(f64(mo[b]), f64(ml[b]), ro, rl, range(w.hq), "bf16", f"req {b} merged")
    # q = 0 closed form on every request and shard: LSE = ln(16384)
    qz = torch.zeros_like(q)
    for j, (o, l) in enumerate(_run_shards(qz, kv, W, w.scale)):
        torch.cuda.synchronize()
        err = float((l - np.log(w.ctx_len // W)).abs().max())
        say(f"  q=0 closed form shard {j}: max|dLSE|={err:.2e}")
        assert err < 1e-3


@pytest.mark.parametrize("val", [0.05, 0.25])
def test_decode_reference_growth(val):
    """One key far above every other score, after the first tile: 0.05 lifts
    the row max by about 2^41 (log2 units) over the first tile's, 0.25 by
    about 2^207 (beyond the fp32 range of exp without a moved reference).
    The kernel's softmax reference handling must still give the plain
    definition's result."""
    B, ctx, hq = 2, 3000, 128
    q = torch.ones((B, hq, DQK), device=DEV, dtype=torch.bfloat16)
    kv = torch.zeros((B, ctx, DQK), device=DEV, dtype=torch.bfloat16)
    kv[0, 2000] = val
    kv[1, 37] = val
    kv[1, 2999] = -val
    say(f"decode reference growth val={val}")
    outs = _run_shards(q, kv, 1, 1.0)
    torch.cuda.synchronize()
    q64, kv64 = f64(q), f64(kv)
    o, l = outs[0]
    for b in range(B):
        ro, rl = _oracle_shard(q64, kv64, b, 0, 1, 1.0, ctx)
        compare(f64(o[b]), f64(l[b]), ro, rl, range(hq), "bf16", f"req {b}")


def test_decode_huge_values_overflow_guard():
    """A key whose score is 2^59.9 above the first tile's (q is zero on the
    512 latent columns and one on the 64 rope columns, so the score comes
    from the rope part alone) while its latent columns -- its V row -- are
    near 2^70: the main pass's numerator times V leaves the fp32 range
    although the exact output is finite.  The slice must be flagged and
    recomputed; O is compared after scaling by 2^-70 (linear in V)."""
    B, ctx, hq, big = 2, 3000, 128, 2.0 ** 70
    g = torch.Generator(device=DEV)
    g.manual_seed(777)
    q = torch.zeros((B, hq, DQK), device=DEV, dtype=torch.bfloat16)
    q[:, :, DV:] = 1.0
    kv = torch.randn((B, ctx, DQK), generator=g, device=DEV)
    kv[:, :, DV:] = 0.0
    kv[0, 2000, DV:] = 0.6484375          # 64 x 0.6484375 x log2(e) = 59.87
    kv[0, 2000, :DV] *= big
    kv[1, 40, DV:] = 0.6484375
    kv[1, 40, :DV] *= big
    kv = kv.to(torch.bfloat16)
    say("decode huge values")
    outs = _run_shards(q, kv, 1, 1.0)
    torch.cuda.synchronize()
    o, l = outs[0]
    assert bool(torch.isfinite(o.float()).all()), "non-finite O"
    q64, kv64 = f64(q), f64(kv)
    for b in range(B):
        ro, rl = _oracle_shard(q64, kv64, b, 0, 1, 1.0, ctx)
        compare(f64(o[b]) / big, f64(l[b]), ro / big, rl, range(hq), "bf16", f"req {b} (O / 2^70)")


def test_decode_accumulate_in_place():
    """The W shard partials merged into a running (O, LSE) by the decode
    combine (accumulate=1) instead of a separate merge."""
    B, ctx, W, hq = 2, 2000, 4, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(4242)
    q = torch.randn((B, hq, DQK), generator=g, device=DEV).to(torch.bfloat16)
    kv = torch.randn((B, ctx, DQK), generator=g, device=DEV).to(torch.bfloat16)
    scale = 1.0 / np.sqrt(DQK)
    o = torch.zeros((B, hq, DV), device=DEV, dtype=torch.float32)
    lse = torch.full((B, hq), -np.inf, device=DEV, dtype=torch.float32)
    for j in range(W):
        say(f"decode accumulate shard {j}")
        shard = kv[:, j::W].contiguous()
        n_j = shard.shape[1]
        k = shard.view(B * n_j, 1, DQK)
        pos = torch.arange(j, ctx, W, device=DEV, dtype=torch.int32).repeat(B)
        segs = [cp.Segment(b, b, b + 1, ctx, 1, b * n_j, (b + 1) * n_j) for b in range(B)]
        cp.attn_fwd(q, k, k[:, :, :DV], segs, scale, kv_pos=pos, o=o, lse=lse, accumulate=True)
    torch.cuda.synchronize()
    q64, kv64 = f64(q), f64(kv)
    for b in range(B):
        ro, rl = ao.attend(q64[b], kv64[b], kv64[b, :, :DV], [ctx] * hq, np.arange(ctx), scale)
        compare(f64(o[b]), f64(lse[b]), ro, rl, range(hq), "bf16", f"req {b} accumulated")

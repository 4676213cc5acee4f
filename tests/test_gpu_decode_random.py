"""GPU parity of the decode shard (MLA-absorbed latent, 576/512, V = the
first 512 columns of K) on seeded random configurations: request count and
per-request context lengths, CP size and rank, one or two latent KV heads
with 16..160 query heads each (partial and several head tiles), one or two
query rows per request at the next position or inside the context (the
causal cut falls in the shard), and the rank's keys either contiguous
(token interleave) or in a randomly allocated paged pool (block interleave,
unused pool rows NaN).  Every request and KV head against the oracle."""
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


def _config(seed):
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.integers(1, 6))
    ctx = [int(x) for x in rng.integers(1, 3001, size=B)]
    W = int(rng.choice([1, 2, 4, 8]))
    j = int(rng.integers(0, W))
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([16, 64, 128, 160]))
    q_len = int(rng.choice([1, 2]))
    # query position of each request's first row: the next token, or inside
    qp = [c if rng.random() < 0.6 else int(rng.integers(0, c)) for c in ctx]
    paged = rng.random() < 0.5
    bs = int(rng.choice([32, 64, 128]))
    return B, ctx, W, j, hkv, G, q_len, qp, paged, bs


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_config(seed):
    B, ctx, W, j, hkv, G, q_len, qp, paged, bs = _config(seed)
    hq = G * hkv
    say(f"decode random {seed}: B={B} ctx={ctx} W={W} j={j} heads={hq}/{hkv} q_len={q_len} "
        f"qpos={qp} paged={paged and bs}")
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = torch.randn((B * q_len, hq, DQK), generator=g, device=DEV).to(torch.bfloat16)
    kv = [torch.randn((c, hkv, DQK), generator=g, device=DEV).to(torch.bfloat16) for c in ctx]
    # this rank's keys of every request (absolute positions, increasing)
    if paged:
        keys = [np.arange(c)[(np.arange(c) // bs) % W == j] for c in ctx]
    else:
        keys = [np.arange(c)[np.arange(c) % W == j] for c in ctx]
    n = [len(x) for x in keys]
    scale = 1.0 / np.sqrt(DQK)
    if paged:
        table, pool_row, nblocks = workloads.paged_layout(n, bs, 3, seed)
        stride = table.shape[1]
        pool = torch.full((max(nblocks, 1) * bs, hkv, DQK), float("nan"), device=DEV,
                          dtype=torch.bfloat16)
        pos = np.full((B, stride * bs), 1 << 30, dtype=np.int32)
        for b in range(B):
            if n[b]:
                pool[torch.from_numpy(pool_row[b, :n[b]]).to(DEV)] = kv[b][torch.from_numpy(keys[b]).to(DEV)]
                pos[b, :n[b]] = keys[b]
        segs = [cp.Segment(b, b * q_len, (b + 1) * q_len, qp[b], 1, 0, n[b]) for b in range(B)]
        o, lse = cp.attn_fwd(q, pool, pool[:, :, :DV], segs, scale,
                             kv_pos=torch.from_numpy(pos.reshape(-1)).to(DEV), o_dtype=torch.float32,
                             block_table=torch.from_numpy(table).to(DEV), block_size=bs)
    else:
        rows = [kv[b][torch.from_numpy(keys[b]).to(DEV)] for b in range(B)]
        kc = torch.cat(rows) if sum(n) else torch.zeros((1, hkv, DQK), device=DEV, dtype=torch.bfloat16)
        off = np.concatenate([[0], np.cumsum(n)]).astype(int)
        segs = [cp.Segment(b, b * q_len, (b + 1) * q_len, qp[b], 1, int(off[b]), int(off[b + 1]))
                for b in range(B)]
        pos = np.concatenate(keys).astype(np.int32) if sum(n) else np.zeros(1, np.int32)
        o, lse = cp.attn_fwd(q, kc, kc[:, :, :DV], segs, scale, kv_pos=torch.from_numpy(pos).to(DEV),
                             o_dtype=torch.float32)
    torch.cuda.synchronize()
    q64 = f64(q)
    for b in range(B):
        kb = f64(kv[b])[keys[b]] if n[b] else np.zeros((0, hkv, DQK))
        for kh in range(hkv):
            hs = slice(kh * G, (kh + 1) * G)
            qrows = q64[b * q_len:(b + 1) * q_len, hs].reshape(q_len * G, DQK)
            qpos = np.repeat(np.arange(q_len) + qp[b], G)
            ro, rl = ao.attend(qrows, kb[:, kh], kb[:, kh, :DV], qpos, keys[b], scale)
            compare(f64(o[b * q_len:(b + 1) * q_len, hs]).reshape(q_len * G, DV),
                    f64(lse[b * q_len:(b + 1) * q_len, hs]).reshape(q_len * G),
                    ro, rl, range(q_len * G), "bf16", f"req {b} kv head {kh}")

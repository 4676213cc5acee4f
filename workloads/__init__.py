"""Seeded synthetic workloads for context-parallel causal attention.

This module only draws numbers: request lengths, cached-prefix lengths and
N(0, 1) tensors from fixed seeds.  It holds none of the method's arithmetic
(no sharding, no masking, no softmax), so that both the HIP path and the CPU
oracle can take their inputs from it without sharing any logic.

The five workloads follow the shapes the pages use for this problem:

* ``zigzag_t256``: zigzag layout, CP=4, one request of 256 new tokens, no
  prefix, 4 q heads = 4 KV heads, head dim 64, fp32.
* ``zigzag_t8192_p1024``: zigzag, CP=8, 8192 new tokens after a 1024-token
  cached prefix, GQA 32 q / 8 KV heads, head dim 128, bf16, scale 1/sqrt(128).
* ``interleave_b12``: interleave, CP=4, 12 requests of lengths 5, 3 and ten
  lengths uniform in [1024, 16384]; prefixes uniform in [0, 4096]; GQA 32/8,
  head dim 128, bf16.
* ``zigzag_t131072_mla``: zigzag, CP=8, 131072 new tokens, MLA-prefill shape
  (128 heads, qk dim 192 = 128 + 64 rope, v dim 128), bf16; ring partials
  against each rank's KV pair, then the LSE merge.
* ``decode_mla_b64``: decode shard, 64 requests x 1 query token over a
  131072-token context whose KV is interleaved token i -> rank i mod 8,
  MLA-absorbed 128 q heads vs 1 latent KV head (576 = 512 latent + 64 rope,
  V = the first 512 latent columns), bf16.

Tensors are drawn as fp32 N(0, 1) from a seeded ``torch.Generator`` in the
order Q, K, V, then rounded to bf16 (round-to-nearest-even) where the
workload says bf16.  Integer draws use ``numpy.random.default_rng(seed)``
with inclusive bounds.  ``paged_layout`` draws a random page allocation
(a permutation of pool blocks) for the paged-KV decode layout.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get",
    "small",
    "prefill_tensors",
    "decode_tensors",
    "paged_layout",
    "rand_tensor",
]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                      # "prefill" or "decode"
    strategy: Optional[str]        # "zigzag" | "interleave" | None (decode)
    cp_size: int
    new_lens: Tuple[int, ...]
    prefix_lens: Tuple[int, ...]
    hq: int
    hkv: int
    dqk: int
    dv: int
    dtype: str                     # "f32" | "bf16"
    seed: int
    scale: float
    # decode only: each request has ``ctx_len`` cached keys spread over
    # ``cp_size`` shards and one new query token at position ``ctx_len``.
    ctx_len: int = 0
    v_aliases_k: bool = False
    # ring partials: run one partial per rank-owned KV pair, then merge
    ring: bool = False
    notes: str = field(default="", compare=False)

    @property
    def num_reqs(self) -> int:
        return len(self.new_lens)

    @property
    def total_new(self) -> int:
        return int(sum(self.new_lens))

    @property
    def total_kv(self) -> int:
        return int(sum(p + t for p, t in zip(self.prefix_lens, self.new_lens)))

    @property
    def group(self) -> int:
        return self.hq // self.hkv


def _interleave_b12_lens(seed: int) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    rng = np.random.default_rng(seed)
    tail = rng.integers(1024, 16384 + 1, size=10)
    prefixes = rng.integers(0, 4096 + 1, size=12)
    lens = (5, 3) + tuple(int(x) for x in tail)
    return lens, tuple(int(x) for x in prefixes)


_IL_LENS, _IL_PREFIX = _interleave_b12_lens(3)

WORKLOADS = {
    "zigzag_t256": Workload(
        name="zigzag_t256", kind="prefill", strategy="zigzag", cp_size=4,
        new_lens=(256,), prefix_lens=(0,), hq=4, hkv=4, dqk=64, dv=64,
        dtype="f32", seed=1, scale=1.0 / 8.0),
    "zigzag_t8192_p1024": Workload(
        name="zigzag_t8192_p1024", kind="prefill", strategy="zigzag", cp_size=8,
        new_lens=(8192,), prefix_lens=(1024,), hq=32, hkv=8, dqk=128, dv=128,
        dtype="bf16", seed=2, scale=1.0 / math.sqrt(128.0)),
    "interleave_b12": Workload(
        name="interleave_b12", kind="prefill", strategy="interleave", cp_size=4,
        new_lens=_IL_LENS, prefix_lens=_IL_PREFIX, hq=32, hkv=8, dqk=128, dv=128,
        dtype="bf16", seed=3, scale=1.0 / math.sqrt(128.0)),
    "zigzag_t131072_mla": Workload(
        name="zigzag_t131072_mla", kind="prefill", strategy="zigzag", cp_size=8,
        new_lens=(131072,), prefix_lens=(0,), hq=128, hkv=128, dqk=192, dv=128,
        dtype="bf16", seed=4, scale=1.0 / math.sqrt(192.0), ring=True),
    "decode_mla_b64": Workload(
        name="decode_mla_b64", kind="decode", strategy=None, cp_size=8,
        new_lens=(1,) * 64, prefix_lens=(131072,) * 64, hq=128, hkv=1,
        dqk=576, dv=512, dtype="bf16", seed=5, scale=1.0 / math.sqrt(576.0),
        ctx_len=131072, v_aliases_k=True),
}

_ORDER = ["zigzag_t256", "zigzag_t8192_p1024", "interleave_b12",
          "zigzag_t131072_mla", "decode_mla_b64"]


def get(name: str) -> Workload:
    return WORKLOADS[name]


def ordered() -> list:
    return [WORKLOADS[n] for n in _ORDER]


def small(w: Workload, **overrides) -> Workload:
    """A copy of ``w`` with some fields replaced (for scaled-down test cases)."""
    return replace(w, **overrides)


def _torch():
    import torch  # imported lazily: the oracle tests do not need a GPU
    return torch


def rand_tensor(shape: Sequence[int], gen, device, dtype: str):
    """fp32 N(0,1) from ``gen``, then rounded to ``dtype`` (RNE for bf16)."""
    torch = _torch()
    t = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype}")
    return t


def _randn_chunked(shape, gen, device, dtype, chunk_rows=8192):
    """Same draws as ``rand_tensor`` for one big tensor, but converted to
    bf16 in row chunks so a 131072-row tensor never exists in fp32.

    The Generator is advanced chunk by chunk, so the values differ from a
    single ``randn`` call of the full shape; every consumer goes through this
    function, so the stream is still fixed by the seed."""
    torch = _torch()
    out_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty(tuple(shape), device=device, dtype=out_dtype)
    n = shape[0]
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=gen,
                               device=device, dtype=torch.float32).to(out_dtype)
    return out


def prefill_tensors(w: Workload, device="cpu"):
    """Q for every new token of the batch (flattened batch order) and the
    full K, V buffers (per request: cached prefix then new tokens, requests
    packed back to back).

    Returns (q [sum T, hq, dqk], k [sum (P+T), hkv, dqk], v [sum (P+T), hkv, dv]).
    """
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    q = _randn_chunked((w.total_new, w.hq, w.dqk), gen, device, w.dtype)
    k = _randn_chunked((w.total_kv, w.hkv, w.dqk), gen, device, w.dtype)
    v = _randn_chunked((w.total_kv, w.hkv, w.dv), gen, device, w.dtype)
    return q, k, v


def decode_tensors(w: Workload, device="cpu", num_reqs: Optional[int] = None,
                   ctx_len: Optional[int] = None):
    """Decode workload: q [B, hq, dqk] for the one new token of each request
    and the full latent cache kv [B, ctx, dqk] in position order (V is the
    first ``dv`` columns of the same rows)."""
    torch = _torch()
    b = w.num_reqs if num_reqs is None else num_reqs
    ctx = w.ctx_len if ctx_len is None else ctx_len
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    q = _randn_chunked((b, w.hq, w.dqk), gen, device, w.dtype)
    kv = _randn_chunked((b * ctx, w.dqk), gen, device, w.dtype).view(b, ctx, w.dqk)
    return q, kv


def paged_layout(rows_per_req: Sequence[int], block_size: int, spare_blocks: int, seed: int):
    """A random page allocation for a paged KV cache: request b's logical
    rows [0, rows_per_req[b]) are cut into blocks of ``block_size`` rows and
    every block gets a distinct pool block, drawn as a random permutation of
    ``sum(blocks) + spare_blocks`` pool blocks (the spare ones stay unused).

    Returns (block_table int32 [B, max blocks] (unused entries -1),
    pool_row int64 [B, max blocks * block_size] (pool row of every logical
    row, -1 past the request's end), pool_blocks)."""
    nblk = [(int(n) + block_size - 1) // block_size for n in rows_per_req]
    total = sum(nblk) + int(spare_blocks)
    perm = np.random.default_rng(seed).permutation(total).astype(np.int32)
    stride = max(1, max(nblk, default=1))
    table = np.full((len(nblk), stride), -1, dtype=np.int32)
    pool_row = np.full((len(nblk), stride * block_size), -1, dtype=np.int64)
    at = 0
    for b, (n, nb) in enumerate(zip(rows_per_req, nblk)):
        table[b, :nb] = perm[at:at + nb]
        at += nb
        x = np.arange(int(n))
        pool_row[b, :n] = table[b, x // block_size].astype(np.int64) * block_size + x % block_size
    return table, pool_row, total

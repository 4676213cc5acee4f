"""cp_attn_fwd_noalloc (scratch in the library's static per-GPU array)
against cp_attn_fwd (caller workspace) through the C ABI: the same kernels
on the same inputs, so the results must be bitwise equal.  Two calls in a
row per path, the second smaller than the first (the shared scratch keeps
the first call's contents): the bf16 kernel's per-workgroup flags, a small
call whose keys are split into partials, the pass-Q accumulator, and the
MLA decode shard's slice partials."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand(shape, g):
    return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)


def _same(a, b, what):
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), f"{what}: outputs differ"


def _both(q, k, v, segs, scale, out_shape, odt=torch.bfloat16, **kw):
    o1 = torch.empty(out_shape, device=DEV, dtype=odt)
    l1 = torch.empty(out_shape[:2], device=DEV, dtype=torch.float32)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    if kw.get("accumulate"):
        for o, l in ((o1, l1), (o2, l2)):
            o.fill_(0.25)
            l.fill_(3.0)
    ref = cp.attn_fwd(q, k, v, segs, scale, o=o1, lse=l1, **kw)
    got = cp.attn_fwd_noalloc(q, k, v, segs, scale, o2, l2, **kw)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("split", [False, True], ids=["flags", "split-keys"])
def test_noalloc_prefill(split):
    g = torch.Generator(device=DEV)
    g.manual_seed(71)
    d = 128
    # split: few enough workgroups that the keys are cut into partials;
    # otherwise enough of them (>= 512 of 128 rows) for the flags alone
    calls = ((4096, 512, 2), (1536, 100, 2)) if split else ((4096, 512, 64), (2048, 100, 64))
    for T, P, hh in calls:                       # the second call is smaller
        C = 2
        plan = cp.shard_plan("zigzag", C, 1, [T], [P])
        q = _rand((plan.num_local, hh, d), g)
        k, v = _rand((P + T, hh, d), g), _rand((P + T, hh, d), g)
        say(f"noalloc prefill split={split} T={T} P={P} heads={hh}")
        a, _ = cp._lib.attn_args(q, k, v, plan, 0.088,
                                 torch.empty((plan.num_local, hh, d), device=DEV,
                                             dtype=torch.bfloat16),
                                 torch.empty((plan.num_local, hh), device=DEV))
        ws = cp.attn_workspace_size(a)
        parts = ws > 4 * plan.num_local * hh        # more than the flags alone
        assert parts == split, (ws, split)
        ref, got = _both(q, k, v, plan, 0.088, (plan.num_local, hh, d))
        _same(ref, got, f"T={T}")


def test_noalloc_accumulate():
    g = torch.Generator(device=DEV)
    g.manual_seed(72)
    H, d = 4, 192
    for T in (3000, 700):
        q = _rand((T, H, d), g)
        k, v = _rand((T, H, d), g), _rand((T, H, 128), g)
        segs = [cp.Segment(0, 0, T, 0, 1, 0, T)]
        say(f"noalloc accumulate T={T}")
        ref, got = _both(q, k, v, segs, 0.07, (T, H, 128), odt=torch.float32, accumulate=True)
        _same(ref, got, f"accumulate T={T}")


def test_noalloc_decode():
    g = torch.Generator(device=DEV)
    g.manual_seed(73)
    for B, n in ((16, 8192), (5, 3000)):
        q = _rand((B, 128, 576), g)
        kv = _rand((B * n, 1, 576), g)
        segs = [cp.Segment(b, b, b + 1, 10 ** 6, 1, b * n, (b + 1) * n) for b in range(B)]
        pos = torch.arange(n, device=DEV, dtype=torch.int32).repeat(B) * 8
        say(f"noalloc decode B={B} n={n}")
        ref, got = _both(q, kv, kv[:, :, :512], segs, 576 ** -0.5, (B, 128, 512),
                         odt=torch.float32, kv_pos=pos)
        _same(ref, got, f"decode B={B}")


def test_noalloc_too_large_is_refused():
    # 7168 rows x 4 heads against 2^20 keys: 112 workgroups of 256 rows, so the
    # keys are cut into 16 chunks, whose fp32 partials (235 MB) are more than
    # the static scratch; nothing may be enqueued or written
    q = torch.zeros((7168, 4, 128), device=DEV, dtype=torch.bfloat16)
    k = torch.zeros((1 << 20, 4, 128), device=DEV, dtype=torch.bfloat16)
    o = torch.full((7168, 4, 128), 5.0, device=DEV)
    lse = torch.full((7168, 4), 5.0, device=DEV)
    segs = [cp.Segment(0, 0, 7168, (1 << 20) - 7168, 1, 0, 1 << 20)]
    with pytest.raises(cp.CpError) as e:
        cp.attn_fwd_noalloc(q, k, k, segs, 0.1, o, lse)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((o == 5.0).all()) and bool((lse == 5.0).all())

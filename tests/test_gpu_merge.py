"""GPU parity of cp_lse_merge against the oracle's merge."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
from oracle import attn_oracle as ao
from gpu_helpers import f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _parts(P, rows, heads, dv, dtype, seed, empty_frac=0.2):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    o = torch.randn((P, rows, heads, dv), generator=g, device=DEV, dtype=torch.float32).to(dtype)
    lse = torch.randn((P, rows, heads), generator=g, device=DEV, dtype=torch.float32) * 4
    drop = torch.rand((P, rows, heads), generator=g, device=DEV) < empty_frac
    lse[drop] = -float("inf")
    o[drop] = 0
    return o, lse


@pytest.mark.parametrize("P,rows,heads,dv,pdt,odt", [
    (8, 300, 16, 128, torch.bfloat16, torch.bfloat16),
    (8, 64, 128, 512, torch.float32, torch.bfloat16),
    (3, 77, 5, 64, torch.float32, torch.float32),
    (11, 50, 4, 128, torch.bfloat16, torch.float32),   # more partials than one load batch
    (2, 1, 1, 8, torch.float32, torch.float32),
])
def test_merge_matches_oracle(P, rows, heads, dv, pdt, odt):
    say(f"merge P={P} rows={rows} heads={heads} dv={dv} {pdt}->{odt}")
    o, lse = _parts(P, rows, heads, dv, pdt, seed=P * 1000 + dv)
    # make some (row, head) empty in every partial
    lse[:, 0, 0] = -float("inf")
    o[:, 0, 0] = 0
    mo, ml = cp.lse_merge(o, lse, out_dtype=odt)
    torch.cuda.synchronize()
    ro, rl = ao.lse_merge(f64(o), f64(lse))
    tol = 2e-2 if odt == torch.bfloat16 else 1e-5
    assert np.max(np.abs(f64(mo) - ro)) <= tol
    fin = np.isfinite(rl)
    got = f64(ml)
    assert np.array_equal(np.isfinite(got), fin)
    if fin.any():
        err = float(np.max(np.abs(got[fin] - rl[fin])))
        say(f"  max|dO|={np.max(np.abs(f64(mo) - ro)):.3e} max|dLSE|={err:.3e}")
        assert err <= 1e-5
    assert np.all(f64(mo)[~fin] == 0)


def test_merge_identities_bit_exact():
    say("merge identities")
    o, lse = _parts(1, 200, 8, 128, torch.bfloat16, seed=7, empty_frac=0.0)
    mo, ml = cp.lse_merge(o, lse)
    assert torch.equal(mo, o[0]) and torch.equal(ml, lse[0])
    # a second, empty partial changes nothing
    o2 = torch.cat([o, torch.zeros_like(o)])
    l2 = torch.cat([lse, torch.full_like(lse, -float("inf"))])
    mo2, ml2 = cp.lse_merge(o2, l2)
    assert torch.equal(mo2, o[0]) and torch.equal(ml2, lse[0])
    # two identical partials: O unchanged, L + ln 2
    of = o.float()
    mo3, ml3 = cp.lse_merge(torch.cat([of, of]), torch.cat([lse, lse]), out_dtype=torch.float32)
    assert torch.allclose(mo3, of[0], atol=1e-6, rtol=0)
    assert torch.allclose(ml3, lse[0] + np.log(2.0), atol=1e-6, rtol=0)
    torch.cuda.synchronize()


def test_merge_repeatable():
    o, lse = _parts(8, 128, 16, 128, torch.bfloat16, seed=9)
    a = cp.lse_merge(o, lse)
    b = cp.lse_merge(o, lse)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("seed", range(16))
def test_merge_random_config(seed):
    """Seeded random shapes: 1..16 partials, ragged rows and heads, every
    allowed dv (8 x a power of two up to 2048), mixed part / output dtypes,
    0..60 % empty partials."""
    rng = np.random.default_rng(3000 + seed)
    P = int(rng.integers(1, 17))
    rows, heads = int(rng.integers(1, 300)), int(rng.integers(1, 24))
    dv = int(8 * 2 ** rng.integers(0, 9))
    pdt = (torch.bfloat16, torch.float32)[int(rng.integers(0, 2))]
    odt = (torch.bfloat16, torch.float32)[int(rng.integers(0, 2))]
    empty = float(rng.uniform(0.0, 0.6))
    say(f"merge random {seed}: P={P} rows={rows} heads={heads} dv={dv} {pdt}->{odt} empty={empty:.2f}")
    o, lse = _parts(P, rows, heads, dv, pdt, seed=4000 + seed, empty_frac=empty)
    mo, ml = cp.lse_merge(o, lse, out_dtype=odt)
    torch.cuda.synchronize()
    ro, rl = ao.lse_merge(f64(o), f64(lse))
    tol = 2e-2 if odt == torch.bfloat16 else 1e-5
    fin = np.isfinite(rl)
    got = f64(ml)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.max(np.abs(f64(mo) - ro)) <= tol
    if fin.any():
        assert float(np.max(np.abs(got[fin] - rl[fin]))) <= 1e-5
    assert np.all(f64(mo)[~fin] == 0)

"""GPU checks of the two measurement probes the benchmark reports beside the
published peaks: the matrix-core loop's sums are exact (8 chains x 16 per
bf16 32x32x16 product of ones, per round) and the streamed copy reproduces
its source, including a size that ends inside a one-wave piece."""
import pytest
import torch

import context_causal_attention_cp_amd as cp
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wgs,iters", [(1, 1), (7, 33), (512, 256)])
def test_calib_mfma_sums(wgs, iters):
    say(f"calib mfma wgs={wgs} iters={iters}")
    out = torch.full((wgs * 4,), -1.0, device="cuda", dtype=torch.float32)
    cp.calib_mfma(wgs, iters, out)
    torch.cuda.synchronize()
    assert bool((out == 8.0 * 16 * iters).all()), out[:8]


@pytest.mark.parametrize("nbytes", [16, 1024, 1040, (64 << 20) + 48])
def test_calib_copy(nbytes):
    say(f"calib copy {nbytes} B")
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), generator=g, device="cuda", dtype=torch.uint8)
    dst = torch.zeros_like(src)
    cp.calib_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_calib_refuses_bad_arguments():
    out = torch.empty(4, device="cuda", dtype=torch.float32)
    with pytest.raises(cp.CpError):
        cp.calib_mfma(0, 1, out)
    with pytest.raises(cp.CpError):
        cp.calib_mfma(1, (1 << 17) + 1, out)
    src = torch.empty(24, device="cuda", dtype=torch.uint8)
    with pytest.raises(cp.CpError):
        cp.calib_copy(src, torch.empty_like(src))

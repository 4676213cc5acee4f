"""GPU parity of cp_restore_apply (the device gather by the restore index)
against the oracle's gather, bit-exact: rows of 16 B to 48 KiB, strided
source and destination, out-of-range entries (zero rows), the zigzag and
interleave restore of real plans, and an empty call."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
from oracle import index_oracle as ix
from oracle import select_oracle as so
from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("rows,row_elems", [(37, 8), (300, 24), (1000, 136), (50, 400), (129, 2072),
                                           (65, 24576)])
def test_restore_apply_random(rows, row_elems):
    say(f"restore apply rows={rows} row_bytes={row_elems * 2}")
    g = torch.Generator(device=DEV)
    g.manual_seed(rows)
    src = torch.randint(-30000, 30000, (rows, row_elems), generator=g, device=DEV,
                        dtype=torch.int16)
    rng = np.random.default_rng(rows)
    idx = rng.integers(-3, rows + 3, size=rows + 11).astype(np.int32)   # some out of range
    out = cp.restore_apply(torch.from_numpy(idx).to(DEV), src)
    torch.cuda.synchronize()
    want = so.restore_apply(idx, src.cpu().numpy())
    assert np.array_equal(out.cpu().numpy(), want)


def test_restore_apply_strided():
    say("restore apply strided rows")
    src_full = torch.arange(50 * 64, device=DEV, dtype=torch.float32).view(50, 64)
    src = src_full[:, :32]                       # rows of 128 B, 256 B apart
    dst_full = torch.full((20, 48), -1.0, device=DEV)
    idx = torch.tensor(list(range(49, 29, -1)), device=DEV, dtype=torch.int32)
    cp.restore_apply(idx, src, out=dst_full[:, :32])
    torch.cuda.synchronize()
    want = so.restore_apply(idx.cpu().numpy(), src.cpu().numpy())
    assert np.array_equal(dst_full[:, :32].cpu().numpy(), want)
    assert bool((dst_full[:, 32:] == -1).all())  # outside the rows: untouched


@pytest.mark.parametrize("strategy,C,lens", [("zigzag", 8, [8192]), ("interleave", 4, [5, 3, 1000, 777])])
def test_restore_apply_plan(strategy, C, lens):
    say(f"restore apply {strategy} C={C} lens={lens}")
    restore, pad = cp.restore_index(strategy, C, lens)
    gathered = np.array(ix.gathered_global_idx(strategy, C, lens), dtype=np.int64)
    # rank-major K rows of 8 heads x 128 dims bf16 (stand-in: row g holds g)
    src = torch.from_numpy(gathered).to(DEV).view(-1, 1).repeat(1, 1024).to(torch.int16)
    out = cp.restore_apply(torch.from_numpy(restore.astype(np.int32)).to(DEV), src)
    torch.cuda.synchronize()
    want = so.restore_apply(restore, src.cpu().numpy())
    assert np.array_equal(out.cpu().numpy(), want)
    assert np.array_equal(out[:, 0].cpu().numpy(), np.arange(sum(lens)).astype(np.int16))


def test_restore_apply_empty():
    src = torch.zeros((4, 8), device=DEV)
    out = cp.restore_apply(torch.zeros((0,), device=DEV, dtype=torch.int32), src)
    assert out.shape == (0, 8)


@pytest.mark.parametrize("seed", range(12))
def test_restore_apply_random_plan(seed):
    """Seeded random plans: strategy, CP size, 1..6 requests of 1..3000
    tokens; the rank-major gathered rows (int32 rows of 16 B .. 12 KiB whose
    first element is the token's global index) restored to causal order."""
    rng = np.random.default_rng(5000 + seed)
    strategy = ("zigzag", "interleave")[int(rng.integers(0, 2))]
    C = int(rng.choice([1, 2, 3, 4, 5, 8]))
    lens = [int(x) for x in rng.integers(1, 3001, size=int(rng.integers(1, 7)))]
    row_elems = 4 * int(rng.integers(1, 769))
    say(f"restore random {seed}: {strategy} C={C} lens={lens} row_bytes={4 * row_elems}")
    restore, pad = cp.restore_index(strategy, C, lens)
    gathered = np.array(ix.gathered_global_idx(strategy, C, lens), dtype=np.int64)
    assert np.array_equal(restore, np.array(ix.restore_index(strategy, C, lens)[0], dtype=np.int32))
    src = torch.from_numpy(gathered.astype(np.int32)).to(DEV).view(-1, 1).repeat(1, row_elems)
    src[:, 1:] += torch.arange(1, row_elems, device=DEV, dtype=torch.int32)
    out = cp.restore_apply(torch.from_numpy(restore.astype(np.int32)).to(DEV), src)
    torch.cuda.synchronize()
    want = so.restore_apply(restore, src.cpu().numpy())
    assert np.array_equal(out.cpu().numpy(), want)
    assert np.array_equal(out[:, 0].cpu().numpy(), np.arange(sum(lens), dtype=np.int32))

"""Helpers shared by the GPU parity tests (not collected: no test_ prefix)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import attn_oracle as ao
from oracle import index_oracle as ix

TOL_F32 = 1e-5      # fp32 inputs, fp32 math: max abs error on O and LSE
TOL_BF16_O = 2e-2   # bf16 inputs, fp32 accumulation: max abs error on O
TOL_BF16_LSE = 1e-3  # ... and on LSE


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t) -> np.ndarray:
    """Exact upcast of a device tensor (bf16 or fp32) to a float64 array."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def tols(dtype: str):
    if dtype == "f32":
        return TOL_F32, TOL_F32
    return TOL_BF16_O, TOL_BF16_LSE


def compare(o_gpu, lse_gpu, o_ref, lse_ref, rows, dtype, what=""):
    """Element-wise check on ``rows`` (all heads, all dims)."""
    tol_o, tol_l = tols(dtype)
    rows = np.asarray(rows, dtype=np.int64)
    og = o_gpu[rows]
    lg = lse_gpu[rows]
    orf = o_ref[rows]
    lrf = lse_ref[rows]
    fin_g, fin_r = np.isfinite(lg), np.isfinite(lrf)
    assert np.array_equal(fin_g, fin_r), f"{what}: -inf pattern of LSE differs"
    assert np.all(lg[~fin_g] == -np.inf) and np.all(og[~fin_g] == 0), f"{what}: empty rows"
    err_o = float(np.max(np.abs(og - orf))) if og.size else 0.0
    err_l = float(np.max(np.abs(lg[fin_g] - lrf[fin_r]))) if fin_g.any() else 0.0
    say(f"  {what}: rows={len(rows)} max|dO|={err_o:.3e} (tol {tol_o}) "
        f"max|dLSE|={err_l:.3e} (tol {tol_l})")
    assert err_o <= tol_o, f"{what}: O error {err_o}"
    assert err_l <= tol_l, f"{what}: LSE error {err_l}"
    return err_o, err_l


def sample_rows(segs, n_per_seg, seed):
    """Seeded rows per segment plus every segment's first and last row."""
    rng = np.random.default_rng(seed)
    rows = set()
    for s in segs:
        b, e = s.q_begin, s.q_end
        if e <= b:
            continue
        rows.update((b, e - 1))
        k = min(n_per_seg, e - b)
        rows.update(int(x) for x in rng.choice(np.arange(b, e), size=k, replace=False))
    return sorted(rows)


def oracle_segments(strategy, C, r, lens, pre):
    return ix.segments(strategy, C, r, list(lens), list(pre))


def oracle_attention(q_loc64, k64, v64, segs, hq, hkv, scale, rows=None, kv_pos=None,
                     causal=True):
    return ao.shard_attention(q_loc64, k64, v64, segs, hq, hkv, scale, kv_pos=kv_pos,
                              rows=rows, causal=causal)


def par_map(fn, items, workers=None):
    """fn over items in a thread pool (NumPy's kernels release the GIL), with
    one BLAS thread per worker; results in the order of items.  The oracle's
    arithmetic is unchanged: the work items are independent heads or row
    blocks of the same definition."""
    from threadpoolctl import threadpool_limits
    items = list(items)
    if workers is None:
        workers = int(os.environ.get("CPATTN_ORACLE_THREADS", "0")) or \
            min(16, len(os.sched_getaffinity(0)))
    with threadpool_limits(limits=1), ThreadPoolExecutor(max(1, workers)) as ex:
        return list(ex.map(fn, items))


def chunks(xs, n):
    xs = list(xs)
    return [xs[i:i + n] for i in range(0, len(xs), n)]


def bf16_host(t) -> np.ndarray:
    """A bf16 tensor's bit patterns on the host (uint16 array, same shape)."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_bits_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (a bf16 is the upper half
    of the fp32 with the same bits)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

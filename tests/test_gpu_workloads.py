"""GPU parity on the full-size workloads, through the C ABI, in the launch
configuration the bench times.  Rows the oracle can afford are compared
element by element (all rows for the small workloads, seeded samples plus
every segment's first and last row for the large ones); the closed form
LSE = ln(#visible keys) for q = 0 checks the mask on every row."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
import workloads
from oracle import attn_oracle as ao
from oracle import index_oracle as ix
from gpu_helpers import compare, f64, oracle_segments, sample_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _local_q(q, plan):
    return q.index_select(0, torch.from_numpy(plan.global_idx.astype(np.int64)).to(DEV))


def _zero_q_check(w, k, v, ranks):
    for r in ranks:
        plan = cp.shard_plan(w.strategy, w.cp_size, r, list(w.new_lens), list(w.prefix_lens))
        q0 = torch.zeros((plan.num_local, w.hq, w.dqk), device=DEV, dtype=k.dtype)
        _, l = cp.attn_fwd(q0, k, v, plan, w.scale)
        torch.cuda.synchronize()
        want = np.log(plan.positions.astype(np.float64) + 1.0)
        err = float(np.max(np.abs(f64(l) - want[:, None])))
        say(f"  q=0 closed form rank {r}: rows={plan.num_local} max|dLSE|={err:.2e}")
        assert err < 1e-3


def test_zigzag_t256_all_ranks_restore_vs_dense():
    w = workloads.get("zigzag_t256")
    say(f"workload {w.name}")
    q, k, v = workloads.prefill_tensors(w, DEV)
    q64, k64, v64 = f64(q), f64(k), f64(v)
    lens, pre = list(w.new_lens), list(w.prefix_lens)
    dense_o, dense_l = ao.shard_attention(q64, k64, v64, ix.segments("zigzag", 1, 0, lens, pre),
                                          w.hq, w.hkv, w.scale)
    restore, pad = cp.restore_index(w.strategy, w.cp_size, lens)
    gathered_o = torch.zeros((w.cp_size * pad, w.hq, w.dv), device=DEV, dtype=q.dtype)
    gathered_l = torch.zeros((w.cp_size * pad, w.hq), device=DEV, dtype=torch.float32)
    for r in range(w.cp_size):
        plan = cp.shard_plan(w.strategy, w.cp_size, r, lens, pre)
        o, l = cp.attn_fwd(_local_q(q, plan), k, v, plan, w.scale)
        gathered_o[r * pad:r * pad + plan.num_local] = o
        gathered_l[r * pad:r * pad + plan.num_local] = l
        toks = ix.rank_tokens("zigzag", w.cp_size, r, lens, pre)
        ro, rl = ao.shard_attention(q64[[t.g for t in toks]], k64, v64,
                                    oracle_segments("zigzag", w.cp_size, r, lens, pre),
                                    w.hq, w.hkv, w.scale)
        torch.cuda.synchronize()
        compare(f64(o), f64(l), ro, rl, range(plan.num_local), "f32", f"rank {r}")
    idx = torch.from_numpy(restore.astype(np.int64)).to(DEV)
    compare(f64(gathered_o.index_select(0, idx)), f64(gathered_l.index_select(0, idx)),
            dense_o, dense_l, range(w.total_new), "f32", "restored vs dense")


def test_zigzag_t8192_p1024():
    w = workloads.get("zigzag_t8192_p1024")
    say(f"workload {w.name}")
    q, k, v = workloads.prefill_tensors(w, DEV)
    q64, k64, v64 = f64(q), f64(k), f64(v)
    lens, pre = list(w.new_lens), list(w.prefix_lens)
    for r in range(w.cp_size):
        plan = cp.shard_plan(w.strategy, w.cp_size, r, lens, pre)
        o, l = cp.attn_fwd(_local_q(q, plan), k, v, plan, w.scale)
        torch.cuda.synchronize()
        segs = oracle_segments("zigzag", w.cp_size, r, lens, pre)
        rows = range(plan.num_local) if r == 0 else sample_rows(segs, 48, seed=r)
        toks = ix.rank_tokens("zigzag", w.cp_size, r, lens, pre)
        ro, rl = ao.shard_attention(q64[[t.g for t in toks]], k64, v64, segs, w.hq, w.hkv,
                                    w.scale, rows=rows)
        compare(f64(o), f64(l), ro, rl, rows, "bf16", f"rank {r}")
    _zero_q_check(w, k, v, range(w.cp_size))


def test_interleave_b12():
    w = workloads.get("interleave_b12")
    say(f"workload {w.name} lens={w.new_lens} prefix={w.prefix_lens}")
    q, k, v = workloads.prefill_tensors(w, DEV)
    q64, k64, v64 = f64(q), f64(k), f64(v)
    lens, pre = list(w.new_lens), list(w.prefix_lens)
    for r in range(w.cp_size):
        plan = cp.shard_plan(w.strategy, w.cp_size, r, lens, pre)
        o, l = cp.attn_fwd(_local_q(q, plan), k, v, plan, w.scale)
        torch.cuda.synchronize()
        segs = oracle_segments("interleave", w.cp_size, r, lens, pre)
        rows = set(sample_rows(segs, 24, seed=10 + r))
        for s in segs:                      # the two short requests: every row
            if s.req < 2:
                rows.update(range(s.q_begin, s.q_end))
        rows = sorted(rows)
        toks = ix.rank_tokens("interleave", w.cp_size, r, lens, pre)
        ro, rl = ao.shard_attention(q64[[t.g for t in toks]], k64, v64, segs, w.hq, w.hkv,
                                    w.scale, rows=rows)
        compare(f64(o), f64(l), ro, rl, rows, "bf16", f"rank {r}")
    _zero_q_check(w, k, v, range(w.cp_size))


def _mla_rank(w, q, k, v, r, heads, n_rows):
    lens, pre = list(w.new_lens), list(w.prefix_lens)
    C = w.cp_size
    plan = cp.shard_plan("zigzag", C, r, lens, pre)
    q_loc = _local_q(q, plan)
    n = plan.num_local
    segs_o = oracle_segments("zigzag", C, r, lens, pre)
    rows = sample_rows(segs_o, n_rows, seed=40 + r)
    mine = plan.global_idx.astype(np.int64)
    hsel = torch.tensor(heads, device=DEV)
    q_s = f64(q_loc[torch.tensor(rows, device=DEV)][:, hsel])        # [rows, nh, dqk]
    # ring partials: KV_j = rank j's zigzag pair, masked by absolute positions
    o_parts = torch.empty((C, n, w.hq, w.dv), device=DEV, dtype=torch.bfloat16)
    l_parts = torch.empty((C, n, w.hq), device=DEV, dtype=torch.float32)
    for j in range(C):
        say(f"  rank {r} ring partial {j}")
        rows_j = cp.shard_plan("zigzag", C, j, lens, pre).global_idx.astype(np.int64)
        idx = torch.from_numpy(rows_j).to(DEV)
        kj, vj = k.index_select(0, idx), v.index_select(0, idx)
        segs = [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, len(rows_j))
                for s in plan.segments]
        cp.attn_fwd(q_loc, kj, vj, segs, w.scale, kv_pos=idx.to(torch.int32),
                    o=o_parts[j], lse=l_parts[j])
        torch.cuda.synchronize()
        osegs = [ix.Segment(s.req, s.q_begin - 0, s.q_end, s.pos_begin, s.pos_stride, 0,
                            len(rows_j)) for s in segs_o]
        # oracle on the sampled rows / heads (row indices remapped to the sample)
        sub_segs = _remap(osegs, rows)
        ko, vo = f64(kj[:, hsel]), f64(vj[:, hsel])
        ro, rl = ao.shard_attention(q_s, ko, vo, sub_segs, len(heads), len(heads), w.scale,
                                    kv_pos=rows_j)
        compare(f64(o_parts[j][torch.tensor(rows, device=DEV)][:, hsel]),
                f64(l_parts[j][torch.tensor(rows, device=DEV)][:, hsel]),
                ro, rl, range(len(rows)), "bf16", f"partial {j}")
        del kj, vj
    mo, ml = cp.lse_merge(o_parts, l_parts)
    say(f"  rank {r} direct call over the full KV")
    do, dl = cp.attn_fwd(q_loc, k, v, plan, w.scale)
    torch.cuda.synchronize()
    # merged vs direct on every row (both GPU)
    err_o = float((mo.float() - do.float()).abs().max())
    err_l = float((ml - dl).abs().max())
    say(f"  merged vs direct, all rows: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= 2e-2 and err_l <= 1e-3
    ko, vo = f64(k[:, hsel]), f64(v[:, hsel])
    ro, rl = ao.shard_attention(q_s, ko, vo, _remap(segs_o, rows), len(heads), len(heads),
                                w.scale)
    sel = torch.tensor(rows, device=DEV)
    compare(f64(mo[sel][:, hsel]), f64(ml[sel][:, hsel]), ro, rl, range(len(rows)), "bf16",
            "merged vs dense oracle")
    compare(f64(do[sel][:, hsel]), f64(dl[sel][:, hsel]), ro, rl, range(len(rows)), "bf16",
            "direct vs dense oracle")
    del o_parts, l_parts


def _remap(segs, rows):
    """Segments restricted to the sampled rows, renumbered 0..len(rows)-1.
    Each sampled row becomes a one-row segment with its own position."""
    out = []
    for i, r in enumerate(rows):
        for s in segs:
            if s.q_begin <= r < s.q_end:
                pos = s.pos_begin + (r - s.q_begin) * s.pos_stride
                out.append(ix.Segment(s.req, i, i + 1, pos, 1, s.kv_begin, s.kv_end))
                break
    assert len(out) == len(rows)
    return out


def test_zigzag_t131072_mla_ring_and_direct():
    w = workloads.get("zigzag_t131072_mla")
    say(f"workload {w.name}")
    q, k, v = workloads.prefill_tensors(w, DEV)
    # every 4th head and the last; 24 seeded rows per segment plus its first
    # and last row (the fp64 oracle over 131072 keys bounds the sample)
    heads = list(range(0, 128, 4)) + [127]
    for r in (0, 7):
        _mla_rank(w, q, k, v, r, heads, n_rows=24)
    _zero_q_check(w, k, v, [0, 5])

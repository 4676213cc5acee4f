"""GPU parity on the full-size workloads, through the C ABI, in the launch
configuration the bench times.  Rows are compared element by element with
the fp64 oracle, all heads:

* 256 tokens (fp32) and 8192 tokens after a 1024-token prefix: every row of
  every rank;
* the 12-request interleave batch: every row of requests 0 and 1 and of the
  two longest requests, 256 seeded rows of each other segment plus its
  first and last row, every rank;
* 131072 tokens (MLA prefill), ranks 0, 3 and 7: 256 seeded rows per zigzag
  block plus its first and last row, for each of the 8 ring partials, their
  LSE merge, the direct call over the full KV and (rank 0) the 8 partials
  accumulated in place.

The closed form LSE = ln(#visible keys) for q = 0 checks the mask on every
row.  The oracle runs heads (and row blocks) in a thread pool."""
import numpy as np
import pytest
import torch

import context_causal_attention_cp_amd as cp
import workloads
from oracle import attn_oracle as ao
from oracle import index_oracle as ix
from gpu_helpers import (bf16_bits_f64, bf16_host, chunks, compare, f64, oracle_segments, par_map,
                         sample_rows, say)

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


def _oracle_rows(q_loc64_h, k_h, v_h, segs, scale, rows, kv_pos=None, block=1024):
    """Oracle (O, LSE) of one head for the local rows ``rows`` (q_loc64_h:
    [N, dqk] fp64 of that head; k_h / v_h: [Lkv, d] fp64)."""
    out_o = np.zeros((q_loc64_h.shape[0], 1, v_h.shape[1]))
    out_l = np.full((q_loc64_h.shape[0], 1), -np.inf)
    for blk in chunks(rows, block):
        o, l = ao.shard_attention(q_loc64_h[:, None], k_h[:, None], v_h[:, None], segs, 1, 1,
                                  scale, kv_pos=kv_pos, rows=blk)
        out_o[blk] = o[blk]
        out_l[blk] = l[blk]
    return out_o[:, 0], out_l[:, 0]


def _gqa_prefill_all(w, rows_of):
    """One prefill workload, every rank: the GPU output against the oracle on
    rows_of(rank, oracle segments), all heads (heads x row blocks in a thread
    pool)."""
    q, k, v = workloads.prefill_tensors(w, DEV)
    lens, pre = list(w.new_lens), list(w.prefix_lens)
    G = w.hq // w.hkv
    k64, v64 = f64(k), f64(v)
    kh64 = [np.ascontiguousarray(k64[:, h]) for h in range(w.hkv)]
    vh64 = [np.ascontiguousarray(v64[:, h]) for h in range(w.hkv)]
    del k64, v64
    for r in range(w.cp_size):
        plan = cp.shard_plan(w.strategy, w.cp_size, r, lens, pre)
        q_loc = _local_q(q, plan)
        o, l = cp.attn_fwd(q_loc, k, v, plan, w.scale)
        torch.cuda.synchronize()
        segs = oracle_segments(w.strategy, w.cp_size, r, lens, pre)
        rows = rows_of(r, segs)
        q64 = f64(q_loc)
        say(f"  rank {r}: {len(rows)} rows x {w.hq} heads, oracle ...")
        tasks = [(h, blk) for h in range(w.hq) for blk in chunks(rows, 512)]
        res = par_map(lambda t: _oracle_rows(q64[:, t[0]], kh64[t[0] // G], vh64[t[0] // G],
                                             segs, w.scale, t[1]), tasks)
        ro = np.zeros((plan.num_local, w.hq, w.dv))
        rl = np.full((plan.num_local, w.hq), -np.inf)
        for (h, blk), (oo, ll) in zip(tasks, res):
            ro[blk, h] = oo[blk]
            rl[blk, h] = ll[blk]
        compare(f64(o), f64(l), ro, rl, rows, "bf16", f"rank {r}")
    _zero_q_check(w, k, v, range(w.cp_size))


def test_zigzag_t8192_p1024():
    w = workloads.get("zigzag_t8192_p1024")
    say(f"workload {w.name}: every row of every rank")
    _gqa_prefill_all(w, lambda r, segs: [i for s in segs for i in range(s.q_begin, s.q_end)])


def test_interleave_b12():
    w = workloads.get("interleave_b12")
    say(f"workload {w.name} lens={w.new_lens} prefix={w.prefix_lens}")
    order = sorted(range(w.num_reqs), key=lambda b: -w.new_lens[b])
    whole = {0, 1, order[0], order[1]}       # the two short and the two longest requests
    say(f"  every row of requests {sorted(whole)}")

    def rows_of(r, segs):
        rows = set(sample_rows(segs, 256, seed=10 + r))
        for s in segs:
            if s.req in whole:
                rows.update(range(s.q_begin, s.q_end))
        return sorted(rows)
    _gqa_prefill_all(w, rows_of)


@pytest.fixture(scope="module")
def mla_inputs():
    w = workloads.get("zigzag_t131072_mla")
    q, k, v = workloads.prefill_tensors(w, DEV)
    return w, q, k, v, bf16_host(k), bf16_host(v)


def _pair_segments(plan, n_keys):
    return [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0, n_keys)
            for s in plan.segments]


@pytest.mark.parametrize("r", [0, 3, 7])
def test_zigzag_t131072_mla(mla_inputs, r):
    """Rank r of the 131072-token MLA prefill: the 8 ring partials (KV_j =
    rank j's zigzag pair, masked by absolute key positions), their LSE
    merge, the direct call over the full KV and, for rank 0, the 8 partials
    accumulated in place (pass-Q accumulator, as the bench times it): every
    one against the oracle on 256 seeded rows per block plus the block's
    first and last row, all 128 heads."""
    w, q, k, v, k_cpu, v_cpu = mla_inputs
    lens, pre, C = list(w.new_lens), list(w.prefix_lens), w.cp_size
    plan = cp.shard_plan("zigzag", C, r, lens, pre)
    q_loc = _local_q(q, plan)
    n = plan.num_local
    segs_o = oracle_segments("zigzag", C, r, lens, pre)
    rows = sample_rows(segs_o, 256, seed=40 + r)
    sel = torch.tensor(rows, device=DEV)
    say(f"workload {w.name} rank {r}: {len(rows)} rows x {w.hq} heads")
    pairs = [cp.shard_plan("zigzag", C, j, lens, pre).global_idx.astype(np.int64)
             for j in range(C)]
    o_parts = torch.empty((C, n, w.hq, w.dv), device=DEV, dtype=torch.bfloat16)
    l_parts = torch.empty((C, n, w.hq), device=DEV, dtype=torch.float32)
    acc_o = torch.full((n, w.hq, w.dv), 7.0, device=DEV, dtype=torch.bfloat16)
    acc_l = torch.full((n, w.hq), -np.inf, device=DEV, dtype=torch.float32)
    for j in range(C):
        idx = torch.from_numpy(pairs[j]).to(DEV)
        kj, vj, pj = k.index_select(0, idx), v.index_select(0, idx), idx.to(torch.int32)
        segs = _pair_segments(plan, len(pairs[j]))
        cp.attn_fwd(q_loc, kj, vj, segs, w.scale, kv_pos=pj, o=o_parts[j], lse=l_parts[j])
        if r == 0:
            cp.attn_fwd(q_loc, kj, vj, segs, w.scale, kv_pos=pj, o=acc_o, lse=acc_l,
                        accumulate=True)
        del kj, vj
    mo, ml = cp.lse_merge(o_parts, l_parts)
    do, dl = cp.attn_fwd(q_loc, k, v, plan, w.scale)
    torch.cuda.synchronize()
    g_parts = (f64(o_parts[:, sel]), f64(l_parts[:, sel]))
    got = {"merged": (f64(mo[sel]), f64(ml[sel])), "direct": (f64(do[sel]), f64(dl[sel]))}
    if r == 0:
        got["accumulated in place"] = (f64(acc_o[sel]), f64(acc_l[sel]))
    del o_parts, l_parts, acc_o, acc_l, mo, ml, do, dl
    q_s = f64(q_loc[sel])                                    # [rows, hq, dqk]
    q_pos = plan.positions[rows].astype(np.int64)
    # the sampled rows of each zigzag block: one oracle call per block, over
    # the keys up to the block's last sampled position (later keys are
    # invisible to all of them); one request, no prefix, so a key's position
    # is its row in the full KV and its flattened index in a pair
    blocks = []
    for sg in segs_o:
        ii = np.array([i for i, row in enumerate(rows) if sg.q_begin <= row < sg.q_end])
        if len(ii):
            blocks.append((ii, int(q_pos[ii].max()) + 1))
    ro_d = np.zeros((len(rows), w.hq, w.dv))
    rl_d = np.full((len(rows), w.hq), -np.inf)
    ro_p = np.zeros((C, len(rows), w.hq, w.dv))
    rl_p = np.full((C, len(rows), w.hq), -np.inf)

    def head(h):
        kh, vh = bf16_bits_f64(k_cpu[:, h]), bf16_bits_f64(v_cpu[:, h])
        od = np.zeros((len(rows), w.dv))
        ld = np.full(len(rows), -np.inf)
        op = np.zeros((C, len(rows), w.dv))
        lp = np.full((C, len(rows)), -np.inf)
        for ii, kmax in blocks:
            od[ii], ld[ii] = ao.attend(q_s[ii, h], kh[:kmax], vh[:kmax], q_pos[ii],
                                       np.arange(kmax), w.scale)
            for j in range(C):
                kj = pairs[j][pairs[j] < kmax]
                op[j, ii], lp[j, ii] = ao.attend(q_s[ii, h], kh[kj], vh[kj], q_pos[ii], kj,
                                                 w.scale)
        return od, ld, op, lp
    for h, (od, ld, op, lp) in enumerate(par_map(head, range(w.hq))):
        ro_d[:, h], rl_d[:, h] = od, ld
        ro_p[:, :, h], rl_p[:, :, h] = op, lp
    allr = range(len(rows))
    for j in range(C):
        compare(g_parts[0][j], g_parts[1][j], ro_p[j], rl_p[j], allr, "bf16", f"partial {j}")
    for name, (go, gl) in got.items():
        compare(go, gl, ro_d, rl_d, allr, "bf16", f"{name} vs dense oracle")


def test_zigzag_t131072_mla_zero_query(mla_inputs):
    w, q, k, v, _, _ = mla_inputs
    _zero_q_check(w, k, v, [0, 5])

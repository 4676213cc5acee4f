"""Benchmark: one CP rank's share of context-parallel causal attention.

One step = rank 0's share of the 131072-token zigzag workload (CP=8,
MLA-prefill shape: 128 heads, qk 192, v 128, bf16) on the ring (pass-KV)
path: the shard plan, eight partial attention launches against each rank's
zigzag KV pair (masked by absolute key positions), and the LSE merge of the
eight partials.  Inputs are seeded synthetic N(0,1) tensors already resident
in HBM; the KV pairs a ring would receive are built before timing.

Prints ONE JSON line.  ``value`` is useful causal TFLOP/s of the step
(visible (q,k) pairs x heads x 2 x (192 + 128) / step time).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "causal attn TFLOP/s per CP-rank shard + % bf16 MFMA peak; merge GB/s % HBM"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--rank", type=int, default=0, help="CP rank whose share is timed")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="only the headline step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--only", choices=["decode", "decode_paged", "restore", "zigzag_t8192_p1024",
                                       "interleave_b12", "peaks"],
                    help="only this measurement of the extra section (for profiling)")
    return ap.parse_args()


def _copy_calibration(steps):
    """A copy of known size: 1 GiB read + 1 GiB written per launch.  Its
    FETCH_SIZE / WRITE_SIZE counters give the factor between counter KiB
    and bytes moved."""
    import torch
    src = torch.ones(1 << 28, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4,
                      "copy_calibration_bytes_written": dst.numel() * 4,
                      "launches": steps}), flush=True)


def _profiled_traffic(kernel: str, source: str):
    """HBM bytes per launch (read + write) that rocprofv3 counters measured
    for ``kernel``, from the summaries under profiles/; None when no summary
    was taken with the kernel's current source."""
    import hashlib
    src = os.path.join(ROOT, "context_causal_attention_cp_amd", "csrc", source)
    with open(src, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()[:16]
    pdir = os.path.join(ROOT, "profiles")
    for fn in sorted(os.listdir(pdir)) if os.path.isdir(pdir) else []:
        with open(os.path.join(pdir, fn)) as f:
            for line in f:
                if not line.startswith("TRAFFIC "):
                    continue
                kv = dict(x.split("=", 1) for x in line.split()[1:])
                if kv.get("kernel") == kernel and kv.get("sha256_16") == h:
                    return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


def _useful_flops(pairs_per_head, hq, dqk, dv):
    return float(pairs_per_head) * hq * 2.0 * (dqk + dv)


def _rank_pairs(plan):
    return int(sum(int(p) + 1 for p in plan.positions))


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: every CP rank's share is a separate launch on "
              f"that GPU, so --gpus {a.gpus} is not a configuration it measures.",
              file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        _copy_calibration(a.steps)
        return
    import numpy as np
    import torch

    import context_causal_attention_cp_amd as cp
    if a.only:
        _only(cp, a.only)
        return
    import workloads

    dev = "cuda"
    w = workloads.get("zigzag_t131072_mla")
    C, r = w.cp_size, a.rank
    lens, pre = list(w.new_lens), list(w.prefix_lens)
    q, k, v = workloads.prefill_tensors(w, dev)
    plan = cp.shard_plan("zigzag", C, r, lens, pre)
    q_loc = q.index_select(0, torch.from_numpy(plan.global_idx.astype(np.int64)).to(dev))
    kv = []
    for j in range(C):
        idx = torch.from_numpy(cp.shard_plan("zigzag", C, j, lens, pre).global_idx
                               .astype(np.int64)).to(dev)
        kv.append((k.index_select(0, idx), v.index_select(0, idx), idx.to(torch.int32)))
    n = plan.num_local
    o_parts = torch.empty((C, n, w.hq, w.dv), device=dev, dtype=torch.bfloat16)
    l_parts = torch.empty((C, n, w.hq), device=dev, dtype=torch.float32)
    o_out = torch.empty((n, w.hq, w.dv), device=dev, dtype=torch.bfloat16)
    l_out = torch.empty((n, w.hq), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * C + 2)] for _ in range(a.steps)]

    def step(events=None):
        pl = cp.shard_plan("zigzag", C, r, lens, pre)
        for j in range(C):
            kj, vj, pj = kv[j]
            segs = [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0,
                               kj.shape[0]) for s in pl.segments]
            if events:
                events[2 * j].record(stream)
            cp.attn_fwd(q_loc, kj, vj, segs, w.scale, kv_pos=pj, o=o_parts[j], lse=l_parts[j])
            if events:
                events[2 * j + 1].record(stream)
        if events:
            events[2 * C].record(stream)
        cp.lse_merge(o_parts, l_parts, o_out=o_out, lse_out=l_out)
        if events:
            events[2 * C + 1].record(stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / a.steps

    pairs = _rank_pairs(plan)
    flops = _useful_flops(pairs, w.hq, w.dqk, w.dv)
    attn_ms = [sum(ev[i][2 * j].elapsed_time(ev[i][2 * j + 1]) for j in range(C))
               for i in range(a.steps)]
    merge_ms = [ev[i][2 * C].elapsed_time(ev[i][2 * C + 1]) for i in range(a.steps)]
    attn_ms_avg = float(np.mean(attn_ms))
    merge_ms_avg = float(np.mean(merge_ms))
    attn_launch_ms = attn_ms_avg / C
    achieved_tflops = flops / (attn_ms_avg * 1e-3) / 1e12

    # attention algorithmic bytes per launch: Q, K_j, V_j, kv_pos read once,
    # O and LSE written once
    kj0 = kv[0][0]
    attn_bytes = (q_loc.numel() * 2 + kj0.numel() * 2 + kv[0][1].numel() * 2 + kv[0][2].numel() * 4
                  + n * w.hq * (w.dv * 2 + 4))
    # merge algorithmic bytes: live partial rows' O (bf16) + every LSE + outputs
    lp = l_parts.isfinite()
    live_rows = int(lp.sum().item())                   # (row, head, part) triples
    merge_bytes = (live_rows * w.dv * 2 + C * n * w.hq * 4 + n * w.hq * (w.dv * 2 + 4))
    merge_gbs = merge_bytes / (merge_ms_avg * 1e-3) / 1e9
    # the same merge with the Infinity Cache flushed first (a 512 MB scratch
    # write before each run): the partials written just before are evicted,
    # so every byte comes from HBM
    merge_cold_ms = _time_cold_ms(
        lambda: cp.lse_merge(o_parts, l_parts, o_out=o_out, lse_out=l_out), reps=10)
    merge_cold_gbs = merge_bytes / (merge_cold_ms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 Q/K/V",
        "config": {
            "workload": "zigzag_t131072_mla rank %d: plan + 8 ring partials + LSE merge" % r,
            "strategy": "zigzag", "cp_size": C, "cp_rank": r, "new_tokens": w.total_new,
            "local_rows": n, "heads_q": w.hq, "heads_kv": w.hkv, "dqk": w.dqk, "dv": w.dv,
            "visible_pairs_per_head": pairs, "useful_tflop_per_step": round(flops / 1e12, 3),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_bf16_split_kernel<192,128> + exact pass attn_fwd_bf16_kernel<192,128,2,true>",
            "achieved": round(achieved_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": _profiled_traffic("attn_fwd_bf16_split_kernel<192,128>", "attn_fwd_bf16.hip"),
            "algorithmic_bytes": attn_bytes,
            "avg_launch_ms": round(attn_launch_ms, 4),
        },
        "merge": {
            "kernel": "lse_merge_kernel<16,bf16,bf16>",
            "ms": round(merge_cold_ms, 4),
            "algorithmic_bytes": merge_bytes,
            "GB/s": round(merge_cold_gbs, 1),
            "frac_hbm": round(merge_cold_gbs / PEAK_HBM_GBS, 4),
            "timing": "median of 10, each after a 512 MB scratch write that evicts the partials "
                      "from the 256 MB Infinity Cache",
            "in_step_ms": round(merge_ms_avg, 4),
            "in_step_GB/s": round(merge_gbs, 1),
            "in_step_note": "the merge inside the timed steps, right after the partials are "
                            "written (part of its reads may hit the Infinity Cache)",
            "traffic": _profiled_traffic("lse_merge_kernel<16,bf16,bf16>", "lse_merge.hip"),
        },
    }
    acc = None
    if not a.no_extra:
        acc = _ring_accumulate(cp, w, q_loc, kv, lens, pre, r, flops)
    del kv, o_parts, l_parts
    torch.cuda.empty_cache()
    if not a.no_extra:
        out["extra"] = {"zigzag_t131072_mla_ring_accumulate": acc,
                        "zigzag_t131072_mla_direct": _direct(cp, w, q_loc, k, v, plan),
                        "restore_apply_k_t131072": _restore(cp, w, k)}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(w, q, k, v, plan, a.cpu_baseline_seconds)
    del q, k, v, q_loc
    torch.cuda.empty_cache()
    if not a.no_extra:
        out["extra"]["zigzag_t8192_p1024"] = _prefill_ranks(cp, workloads.get("zigzag_t8192_p1024"))
        out["extra"]["interleave_b12"] = _prefill_ranks(cp, workloads.get("interleave_b12"))
        out["extra"]["decode_mla_b64"] = _decode(cp, workloads.get("decode_mla_b64"))
        out["extra"]["decode_mla_b64_paged_block128"] = _decode_paged(
            cp, workloads.get("decode_mla_b64"), 128)
        mp = _measured_peaks(cp)
        out["measured_peaks"] = mp
        out["roofline"]["frac_of_measured_mfma_loop"] = round(
            out["roofline"]["achieved"] / mp["mfma_loop_TFLOP/s"], 4)
        out["roofline"]["frac_of_measured_gemm"] = round(
            out["roofline"]["achieved"] / mp["bf16_gemm_TFLOP/s"], 4)
        out["merge"]["frac_of_measured_copy"] = round(out["merge"]["GB/s"] / mp["copy_GB/s"], 4)
        dec = out["extra"]["decode_mla_b64"]
        dec["frac_of_measured_copy"] = round(dec["GB/s"] / mp["copy_GB/s"], 4)
    print(json.dumps(out), flush=True)


def _only(cp, name):
    """One measurement of the extra section on its own, as a JSON line."""
    import workloads
    if name == "decode":
        out = _decode(cp, workloads.get("decode_mla_b64"))
    elif name in ("zigzag_t8192_p1024", "interleave_b12"):
        out = _prefill_ranks(cp, workloads.get(name))
    elif name == "decode_paged":
        out = _decode_paged(cp, workloads.get("decode_mla_b64"), 128)
    elif name == "peaks":
        out = _measured_peaks(cp)
    else:
        w = workloads.get("zigzag_t131072_mla")
        _, k, _ = workloads.prefill_tensors(w, "cuda")
        out = _restore(cp, w, k)
    print(json.dumps({"only": name, **out}), flush=True)


def _time_cold_ms(fn, reps=10):
    """Median time of ``fn`` with the Infinity Cache flushed before each run
    (a 512 MB scratch write between the runs, outside the timed region)."""
    import numpy as np
    import torch
    scratch = torch.empty(512 << 20, device="cuda", dtype=torch.uint8)
    fn()
    times = []
    for _ in range(reps):
        scratch.fill_(1)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    del scratch
    return float(np.median(times))


def _measured_peaks(cp):
    """Sustained rates measured on this GPU in the same run, as references
    beside the published peaks (the fractions in "roofline", "merge" and the
    extras stay against the published ones): the library's matrix-core loop
    (independent bf16 32x32x16 products on register operands, at the clock
    the chip holds under that load), its streamed device copy, and a large
    bf16 GEMM through torch (hipBLASLt)."""
    import numpy as np
    import torch
    # matrix-core loop: 2 workgroups of 4 waves per compute unit
    wgs, iters = 2 * torch.cuda.get_device_properties(0).multi_processor_count, 16384
    out = torch.empty(wgs * 4, device="cuda", dtype=torch.float32)
    mfma_ms = _time_ms(lambda: cp.calib_mfma(wgs, iters, out), reps=5, warm=2)
    torch.cuda.synchronize()
    if not bool((out == 8.0 * 16 * iters).all()):
        raise RuntimeError("matrix-core loop returned wrong sums")
    mfma_flops = wgs * 4 * iters * 8 * 2.0 * 32 * 32 * 16
    # streamed copy of 4 GiB
    nbytes = 4 << 30
    src = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
    src.fill_(7)
    dst = torch.empty_like(src)
    copy_ms = _time_ms(lambda: cp.calib_copy(src, dst), reps=5, warm=2)
    del src, dst
    torch.cuda.empty_cache()
    n = 8192
    a = torch.randn((n, n), device="cuda", dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda", dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    gemm_ms = _time_ms(lambda: torch.mm(a, b, out=c), reps=10, warm=3)
    del a, b, c
    torch.cuda.empty_cache()
    return {"mfma_loop_TFLOP/s": round(mfma_flops / mfma_ms / 1e9, 1),
            "mfma_loop_what": "cp_calib_mfma: %d workgroups x 4 waves x %d rounds of 8 independent "
                              "bf16 32x32x16 products, mean of 5" % (wgs, iters),
            "copy_GB/s": round(2.0 * nbytes / copy_ms / 1e6, 1),
            "copy_what": "cp_calib_copy of 4 GiB (read + write bytes), mean of 5",
            "bf16_gemm_TFLOP/s": round(2.0 * n ** 3 / gemm_ms / 1e9, 1),
            "bf16_gemm_what": "torch.mm bf16 8192 x 8192 x 8192 (hipBLASLt), mean of 10"}


def _time_ms(fn, reps=5, warm=1):
    """Average time of ``fn`` (HIP events on the current stream)."""
    import torch
    for _ in range(warm):
        fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def _ring_accumulate(cp, w, q_loc, kv, lens, pre, r, flops):
    """The same 8 ring partials merged in the attention epilogue into one
    running bf16 (O, LSE) (accumulate=1, the pass-Q accumulator) instead of
    8 partial outputs and a separate merge."""
    import torch
    C, n = w.cp_size, q_loc.shape[0]
    o = torch.empty((n, w.hq, w.dv), device=q_loc.device, dtype=torch.bfloat16)
    lse = torch.empty((n, w.hq), device=q_loc.device, dtype=torch.float32)
    pl = cp.shard_plan("zigzag", C, r, lens, pre)

    def run():
        lse.fill_(float("-inf"))
        for j in range(C):
            kj, vj, pj = kv[j]
            segs = [cp.Segment(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, 0,
                               kj.shape[0]) for s in pl.segments]
            cp.attn_fwd(q_loc, kj, vj, segs, w.scale, kv_pos=pj, o=o, lse=lse, accumulate=True)
    ms = _time_ms(run, reps=2)
    del o, lse
    return {"ms": round(ms, 3), "TFLOP/s": round(flops / ms / 1e9, 1),
            "frac_bf16_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "note": "8 accumulating launches, no partial buffers and no merge kernel"}


def _restore(cp, w, k):
    """cp_restore_apply on the all-gathered K rows of the 131072-token MLA
    prefill (rank-major zigzag order -> causal order; 131072 rows of
    128 x 192 bf16 = 48 KiB).  HBM-bound: algorithmic bytes = rows read +
    rows written + the index."""
    import numpy as np
    import torch
    restore, _ = cp.restore_index("zigzag", w.cp_size, list(w.new_lens))
    idx = torch.from_numpy(restore.astype(np.int32)).to(k.device)
    dst = torch.empty_like(k)
    ms = _time_ms(lambda: cp.restore_apply(idx, k, out=dst), reps=5)
    by = 2 * k.numel() * k.element_size() + idx.numel() * 4
    del dst
    torch.cuda.empty_cache()
    return {"ms": round(ms, 4), "algorithmic_bytes": by, "GB/s": round(by / ms / 1e6, 1),
            "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4),
            "traffic": _profiled_traffic("restore_apply_long_kernel", "restore_apply.hip")}


def _direct(cp, w, q_loc, k, v, plan):
    """The same shard as one call over the full (gathered) KV."""
    import torch
    o = torch.empty((q_loc.shape[0], w.hq, w.dv), device=q_loc.device, dtype=torch.bfloat16)
    lse = torch.empty((q_loc.shape[0], w.hq), device=q_loc.device, dtype=torch.float32)
    ms = _time_ms(lambda: cp.attn_fwd(q_loc, k, v, plan, w.scale, o=o, lse=lse), reps=3)
    fl = _useful_flops(_rank_pairs(plan), w.hq, w.dqk, w.dv)
    return {"ms": round(ms, 3), "TFLOP/s": round(fl / ms / 1e9, 1),
            "frac_bf16_peak": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}


def _prefill_ranks(cp, w):
    """Each rank's shard of a prefill workload against the gathered KV:
    per-rank time and useful TFLOP/s, and all ranks back to back."""
    import numpy as np
    import torch
    import workloads
    q, k, v = workloads.prefill_tensors(w, "cuda")
    lens, pre = list(w.new_lens), list(w.prefix_lens)
    ranks = []
    total_fl, total_ms = 0.0, 0.0
    for r in range(w.cp_size):
        plan = cp.shard_plan(w.strategy, w.cp_size, r, lens, pre)
        q_loc = q.index_select(0, torch.from_numpy(plan.global_idx.astype(np.int64)).cuda())
        o = torch.empty((plan.num_local, w.hq, w.dv), device="cuda", dtype=q.dtype)
        lse = torch.empty((plan.num_local, w.hq), device="cuda", dtype=torch.float32)
        ms = _time_ms(lambda: cp.attn_fwd(q_loc, k, v, plan, w.scale, o=o, lse=lse), reps=10)
        fl = _useful_flops(_rank_pairs(plan), w.hq, w.dqk, w.dv)
        total_fl += fl
        total_ms += ms
        ranks.append({"rank": r, "ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1)})
    return {"ranks": ranks, "all_ranks_ms": round(total_ms, 4),
            "all_ranks_TFLOP/s": round(total_fl / total_ms / 1e9, 1),
            "frac_bf16_peak": round(total_fl / total_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}


def _decode(cp, w):
    """Decode-CP: each of the W token-interleaved KV shards (fp32 partials),
    then the LSE merge.  HBM-bound: algorithmic bytes = the shard's latent
    rows + q + the fp32 partial output and its LSE."""
    import numpy as np
    import torch
    import workloads
    q, kv = workloads.decode_tensors(w, "cuda")
    W, B, ctx = w.cp_size, w.num_reqs, w.ctx_len
    shards = [kv[:, j::W].contiguous() for j in range(W)]
    del kv
    torch.cuda.empty_cache()
    n_j = ctx // W
    o_parts = torch.empty((W, B, w.hq, w.dv), device="cuda", dtype=torch.float32)
    l_parts = torch.empty((W, B, w.hq), device="cuda", dtype=torch.float32)
    segs = [cp.Segment(b, b, b + 1, ctx, 1, b * n_j, (b + 1) * n_j) for b in range(B)]
    ws = None
    res = []
    for j, sh in enumerate(shards):
        k = sh.view(B * n_j, 1, w.dqk)
        vv = k[:, :, :w.dv]
        pos = torch.arange(j, ctx, W, device="cuda", dtype=torch.int32).repeat(B)
        if ws is None:
            a, keep = cp._lib.attn_args(q, k, vv, segs, w.scale, o_parts[j], l_parts[j],
                                        kv_pos=pos)
            ws = torch.empty(cp.attn_workspace_size(a), device="cuda", dtype=torch.uint8)
        ms = _time_ms(lambda: cp.attn_fwd(q, k, vv, segs, w.scale, kv_pos=pos, o=o_parts[j],
                                          lse=l_parts[j], workspace=ws), reps=10)
        res.append(ms)
    by = B * n_j * w.dqk * 2 + q.numel() * 2 + B * w.hq * (w.dv * 4 + 4)
    o_out = torch.empty((B, w.hq, w.dv), device="cuda", dtype=torch.bfloat16)
    l_out = torch.empty((B, w.hq), device="cuda", dtype=torch.float32)
    # the partials (134 MB) fit the 256 MB Infinity Cache: each timed merge
    # follows a 512 MB scratch write that evicts them (HBM rate), and the
    # back-to-back rate (cache-resident partials) is reported beside it
    mms_warm = _time_ms(lambda: cp.lse_merge(o_parts, l_parts, o_out=o_out, lse_out=l_out),
                        reps=10)
    mms = _time_cold_ms(lambda: cp.lse_merge(o_parts, l_parts, o_out=o_out, lse_out=l_out),
                        reps=10)
    mby = W * B * w.hq * (w.dv * 4 + 4) + B * w.hq * (w.dv * 2 + 4)
    ms = float(np.mean(res))
    fl = 2.0 * B * w.hq * n_j * (w.dqk + w.dv)
    return {"shard_ms": round(ms, 4), "algorithmic_bytes_per_shard": by,
            "GB/s": round(by / ms / 1e6, 1), "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4),
            "TFLOP/s": round(fl / ms / 1e9, 1), "workspace_bytes": int(ws.numel()),
            "traffic": _profiled_traffic("attn_decode_rs_kernel", "attn_decode_mla.hip"),
            "merge_ms": round(mms, 4), "merge_GB/s": round(mby / mms / 1e6, 1),
            "merge_frac_hbm": round(mby / mms / 1e6 / PEAK_HBM_GBS, 4),
            "merge_cache_resident_ms": round(mms_warm, 4),
            "merge_note": "merge_ms: median of 10, each after a 512 MB scratch write (partials "
                          "evicted from the 256 MB Infinity Cache)"}


def _decode_paged(cp, w, bs):
    """Decode-CP rank 0 with the cache interleaved over the ranks in blocks
    of ``bs`` tokens (token i on rank (i // bs) mod W), its blocks scattered
    over a randomly allocated pool and read through a block table; the same
    rows laid out contiguously are timed beside it, in alternating rounds."""
    import numpy as np
    import torch
    import workloads
    q, kv = workloads.decode_tensors(w, "cuda")
    W, B, ctx = w.cp_size, w.num_reqs, w.ctx_len
    i = np.arange(ctx)
    keys = i[(i // bs) % W == 0]
    n = len(keys)
    table, pool_row, nblocks = workloads.paged_layout([n] * B, bs, 64, 2024)
    src = torch.from_numpy((np.arange(B)[:, None] * ctx + keys[None, :]).reshape(-1)).cuda()
    flat = kv.view(B * ctx, w.dqk)
    pool = torch.zeros((nblocks * bs, 1, w.dqk), device="cuda", dtype=kv.dtype)
    pool[torch.from_numpy(pool_row[:, :n].reshape(-1)).cuda(), 0] = flat[src]
    kc = flat[src].view(B * n, 1, w.dqk)
    del kv, flat
    torch.cuda.empty_cache()
    stride = table.shape[1]
    pos = np.zeros((B, stride * bs), dtype=np.int32)
    pos[:, :n] = keys
    pos = torch.from_numpy(pos.reshape(-1)).cuda()
    pos_c = torch.from_numpy(np.tile(keys, B).astype(np.int32)).cuda()
    bt = torch.from_numpy(table).cuda()
    o = torch.empty((B, w.hq, w.dv), device="cuda", dtype=torch.float32)
    lse = torch.empty((B, w.hq), device="cuda", dtype=torch.float32)
    segs_p = [cp.Segment(b, b, b + 1, ctx, 1, 0, n) for b in range(B)]
    segs_c = [cp.Segment(b, b, b + 1, ctx, 1, b * n, (b + 1) * n) for b in range(B)]
    a, keep = cp._lib.attn_args(q, pool, pool[:, :, :w.dv], segs_p, w.scale, o, lse, kv_pos=pos,
                                block_table=bt, block_size=bs)
    ws = torch.empty(cp.attn_workspace_size(a), device="cuda", dtype=torch.uint8)
    fp = lambda: cp.attn_fwd(q, pool, pool[:, :, :w.dv], segs_p, w.scale, kv_pos=pos, o=o,
                             lse=lse, workspace=ws, block_table=bt, block_size=bs)
    fc = lambda: cp.attn_fwd(q, kc, kc[:, :, :w.dv], segs_c, w.scale, kv_pos=pos_c, o=o, lse=lse,
                             workspace=ws)
    # the two alternate in rounds (the GPU's clock drifts over a run, so two
    # back-to-back blocks of calls would not compare like with like); the
    # median round of each after two warm-up rounds
    tp, tc = [], []
    for r in range(7):
        tp.append(_time_ms(fp, reps=4, warm=1 if r == 0 else 0))
        tc.append(_time_ms(fc, reps=4, warm=1 if r == 0 else 0))
    paged, cont = float(np.median(tp[2:])), float(np.median(tc[2:]))
    by = B * n * w.dqk * 2 + q.numel() * 2 + B * w.hq * (w.dv * 4 + 4)
    return {"block_size": bs, "rank_rows_per_request": n, "paged_ms": round(paged, 4),
            "contiguous_ms": round(cont, 4), "algorithmic_bytes": by,
            "paged_GB/s": round(by / paged / 1e6, 1),
            "paged_frac_hbm": round(by / paged / 1e6 / PEAK_HBM_GBS, 4),
            "paged_over_contiguous": round(paged / cont, 4),
            "traffic_contiguous": _profiled_traffic("attn_decode_rs_kernel", "attn_decode_mla.hip")}


def _cpu_baseline(w, q, k, v, plan, budget_s):
    """The oracle as it stands, timed on the host: dense attention of a
    sample of rank 0's rows for as many heads as fit the time budget;
    reported as useful TFLOP/s of the rows it computed."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import attn_oracle as ao
    from oracle import index_oracle as ix
    threads = len(os.sched_getaffinity(0))   # the cores this process may run on
    segs = ix.segments("zigzag", w.cp_size, 0, list(w.new_lens), list(w.prefix_lens))
    rng = np.random.default_rng(99)
    rows = sorted(set(int(x) for x in rng.choice(plan.num_local, size=16, replace=False)))
    q_loc = q.index_select(0, torch.from_numpy(plan.global_idx.astype(np.int64)).to(q.device))
    q_rows = q_loc[torch.tensor(rows, device=q.device)]
    pos = plan.positions[rows].astype(np.int64)
    pairs_per_head = int(np.sum(pos + 1))
    done_heads = 0
    t_compute = 0.0
    t_start = time.perf_counter()
    with threadpool_limits(limits=threads):
        for h in range(w.hq):
            qh = q_rows[:, h].float().cpu().numpy()
            kh = k[:, h].float().cpu().numpy()
            vh = v[:, h].float().cpu().numpy()
            sub = [ix.Segment(0, i, i + 1, int(pos[i]), 1, 0, int(pos[i]) + 1)
                   for i in range(len(rows))]
            t0 = time.perf_counter()
            ao.shard_attention(qh[:, None], kh[:, None], vh[:, None], sub, 1, 1, w.scale)
            t_compute += time.perf_counter() - t0
            done_heads += 1
            if time.perf_counter() - t_start > budget_s:
                break
    flops = _useful_flops(pairs_per_head, done_heads, w.dqk, w.dv)
    return {
        "value": round(flops / t_compute / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(rows)} seeded rows of rank 0 x {done_heads} of {w.hq} heads, dense "
                  f"causal fp64 over up to {int(pos.max()) + 1} keys "
                  f"({flops / 1e9:.1f} GFLOP in {t_compute:.1f} s; BLAS threads = cores)",
        "scalar_oracle": _scalar_oracle_cfg1(),
    }


def _scalar_oracle_cfg1():
    """The pure-Python scalar oracle (triple loop, one thread) on the whole
    256-token fp32 workload's rank 0: its 64 rows x 4 heads over their
    causal keys (d = 64)."""
    import numpy as np
    import workloads
    from oracle import index_oracle as ix
    from oracle import scalar_oracle as so
    w = workloads.get("zigzag_t256")
    q, k, v = workloads.prefill_tensors(w, "cuda")
    toks = ix.rank_tokens("zigzag", w.cp_size, 0, list(w.new_lens), list(w.prefix_lens))
    q64 = q.double().cpu().numpy()[[t.g for t in toks]]
    k64, v64 = k.double().cpu().numpy(), v.double().cpu().numpy()
    pairs = 0
    t0 = time.perf_counter()
    for i, t in enumerate(toks):
        keys = list(range(t.pos + 1))   # no prefix: the request's keys 0 .. pos
        for h in range(w.hq):
            so.attend_row(q64[i, h].tolist(), k64[keys, h].tolist(), v64[keys, h].tolist(),
                          t.pos, keys, w.scale)
        pairs += t.pos + 1
    dt = time.perf_counter() - t0
    flops = _useful_flops(pairs, w.hq, w.dqk, w.dv)
    return {"value": round(flops / dt / 1e9, 4), "unit": "GFLOP/s", "cores": 1,
            "rows_per_s": round(len(toks) * w.hq / dt, 1),
            "sample": f"zigzag_t256 rank 0: all {len(toks)} rows x {w.hq} heads, "
                      f"{pairs} visible pairs per head, {dt:.2f} s"}


if __name__ == "__main__":
    main()

"""CPU tests of the C ABI: exported symbols, the planner and restore index
bit-exact against the index oracle, and every host-side error path."""
import ctypes
import random
import re

import numpy as np
import pytest

import context_causal_attention_cp_amd as cp
from context_causal_attention_cp_amd import _lib
from oracle import index_oracle as ix
import workloads


def _header_functions():
    import os
    from conftest import ROOT
    src = open(os.path.join(ROOT, "include", "cp_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z_0-9]+)\s*\(", src)))


def test_exports_match_header():
    names = _header_functions()
    assert set(names) == set(_lib.EXPORTS)
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert cp.version().count(".") == 2
    assert cp.status_str(0) == "CP_OK"


def _cmp_plan(strategy, C, lens, pre):
    for r in range(C):
        got = cp.shard_plan(strategy, C, r, lens, pre)
        toks = ix.rank_tokens(strategy, C, r, lens, pre)
        segs = ix.segments(strategy, C, r, lens, pre)
        assert got.num_local == len(toks)
        assert got.padded_local == ix.padded_local(strategy, C, lens, pre)
        assert got.positions.tolist() == [t.pos for t in toks]
        assert got.global_idx.tolist() == [t.g for t in toks]
        assert [s.astuple() for s in got.segments] == \
            [(s.req, s.q_begin, s.q_end, s.pos_begin, s.pos_stride, s.kv_begin, s.kv_end)
             for s in segs]
    restore, pad = cp.restore_index(strategy, C, lens)
    want, wpad = ix.restore_index(strategy, C, lens)
    assert restore.tolist() == want and pad == wpad


@pytest.mark.parametrize("strategy", ["zigzag", "interleave"])
def test_planner_matches_oracle_random(strategy):
    rnd = random.Random(42 if strategy == "zigzag" else 43)
    for _ in range(250):
        C = rnd.randint(1, 8)
        B = rnd.randint(0, 5)
        lens = [rnd.randint(0, 70) for _ in range(B)]
        pre = [rnd.randint(0, 50) if rnd.random() < 0.5 else 0 for _ in range(B)]
        _cmp_plan(strategy, C, lens, pre)


@pytest.mark.parametrize("name", ["zigzag_t256", "zigzag_t8192_p1024", "interleave_b12"])
def test_planner_matches_oracle_workloads(name):
    w = workloads.get(name)
    _cmp_plan(w.strategy, w.cp_size, list(w.new_lens), list(w.prefix_lens))


def test_planner_mla_131072_all_ranks():
    # the long-context zigzag workload: every rank owns 2 blocks of 8192
    for r in range(8):
        p = cp.shard_plan("zigzag", 8, r, [131072], [0])
        assert [s.astuple() for s in p.segments] == [
            (0, 0, 8192, 8192 * r, 1, 0, 8192 * (r + 1)),
            (0, 8192, 16384, 8192 * (15 - r), 1, 0, 8192 * (16 - r))]
        assert p.num_local == p.padded_local == 16384


def test_planner_null_prefix_and_empty_batch():
    a = cp.shard_plan("interleave", 3, 1, [4, 5])
    b = cp.shard_plan("interleave", 3, 1, [4, 5], [0, 0])
    assert [s.astuple() for s in a.segments] == [s.astuple() for s in b.segments]
    e = cp.shard_plan("zigzag", 4, 2, [])
    assert e.num_local == 0 and e.segments == [] and e.padded_local == 0


def _raw_plan(strategy, C, r, lens, pre, seg_cap, tok_cap, want_arrays=True):
    L = _lib._lib
    tl = np.asarray(lens, dtype=np.int32)
    pl = np.asarray(pre, dtype=np.int32)
    P32 = ctypes.POINTER(ctypes.c_int32)
    segs = (_lib.Segment * max(1, seg_cap))()
    pos = np.zeros(max(1, tok_cap), dtype=np.int32)
    nseg, nloc, pad = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = L.cp_shard_plan(strategy, C, r, len(lens), tl.ctypes.data_as(P32), pl.ctypes.data_as(P32),
                         segs if want_arrays else None, seg_cap, ctypes.byref(nseg),
                         pos.ctypes.data_as(P32) if want_arrays else None, None, tok_cap,
                         ctypes.byref(nloc), ctypes.byref(pad))
    return st, nseg.value, nloc.value, pad.value


def test_plan_error_paths():
    ok = _raw_plan(0, 4, 1, [16], [0], 8, 64)
    assert ok == (_lib.CP_OK, 2, 4, 4)
    assert _raw_plan(2, 4, 1, [16], [0], 8, 64)[0] == _lib.CP_ERR_ARG      # strategy
    assert _raw_plan(0, 0, 0, [16], [0], 8, 64)[0] == _lib.CP_ERR_ARG      # C = 0
    assert _raw_plan(0, 4, 4, [16], [0], 8, 64)[0] == _lib.CP_ERR_ARG      # rank = C
    assert _raw_plan(0, 4, -1, [16], [0], 8, 64)[0] == _lib.CP_ERR_ARG
    assert _raw_plan(0, 4, 0, [-3], [0], 8, 64)[0] == _lib.CP_ERR_ARG      # negative length
    assert _raw_plan(1, 4, 0, [3], [-1], 8, 64)[0] == _lib.CP_ERR_ARG      # negative prefix
    assert _raw_plan(0, 2, 0, [2**30, 2**30], [0, 0], 8, 64)[0] == _lib.CP_ERR_ARG  # overflow
    # too small: sizes are still reported
    st, nseg, nloc, pad = _raw_plan(0, 4, 1, [16], [0], 1, 64)
    assert (st, nseg, nloc, pad) == (_lib.CP_ERR_SMALL_BUFFER, 2, 4, 4)
    st, nseg, nloc, pad = _raw_plan(0, 4, 1, [16], [0], 8, 3)
    assert (st, nseg, nloc, pad) == (_lib.CP_ERR_SMALL_BUFFER, 2, 4, 4)
    # size query with NULL arrays
    assert _raw_plan(0, 4, 1, [16], [0], 0, 0, want_arrays=False) == (_lib.CP_OK, 2, 4, 4)


def test_restore_error_paths():
    L = _lib._lib
    P32 = ctypes.POINTER(ctypes.c_int32)
    tl = np.asarray([5, 3], dtype=np.int32)
    out = np.zeros(8, dtype=np.int32)
    pad = ctypes.c_int32(-1)
    assert L.cp_restore_index(1, 4, 2, tl.ctypes.data_as(P32), out.ctypes.data_as(P32), 7,
                              ctypes.byref(pad)) == _lib.CP_ERR_SMALL_BUFFER
    assert pad.value == 2
    assert L.cp_restore_index(1, 4, 2, tl.ctypes.data_as(P32), None, 0,
                              ctypes.byref(pad)) == _lib.CP_OK
    assert L.cp_restore_index(1, 0, 2, tl.ctypes.data_as(P32), out.ctypes.data_as(P32), 8,
                              ctypes.byref(pad)) == _lib.CP_ERR_ARG
    assert L.cp_restore_index(1, 4, 2, tl.ctypes.data_as(P32), out.ctypes.data_as(P32), 8,
                              ctypes.byref(pad)) == _lib.CP_OK
    assert out.tolist() == ix.restore_index("interleave", 4, [5, 3])[0]


# ---------------------------------------------------------------- attn / merge argument checks
# Every case below must fail validation before anything touches a device, so
# the fake, never-dereferenced device addresses are safe on a CPU-only host.

FAKE = 0x10000


def _args(**kw):
    a = _lib.AttnArgs()
    segs = (_lib.Segment * 2)(_lib.Segment(0, 0, 4, 0, 1, 0, 4), _lib.Segment(0, 4, 8, 12, 1, 0, 16))
    base = dict(dtype=_lib.CP_BF16, o_dtype=_lib.CP_BF16, num_q_rows=8, num_kv_rows=16, hq=4,
                hkv=2, dqk=128, dv=128, scale=0.1, causal=1,
                q=FAKE, q_row_stride=512, q_head_stride=128,
                k=FAKE, k_row_stride=256, k_head_stride=128,
                v=FAKE, v_row_stride=256, v_head_stride=128,
                o=FAKE, o_row_stride=512, o_head_stride=128,
                lse=FAKE, lse_row_stride=4, num_segs=2)
    base.update(kw)
    for k_, v_ in base.items():
        setattr(a, k_, v_)
    a.segs = kw.get("segs", segs)
    return a, segs


def _fwd(**kw):
    a, keep = _args(**kw)
    st = _lib._lib.cp_attn_fwd(ctypes.byref(a), None)
    del keep
    return st


def _ws(**kw):
    a, keep = _args(**kw)
    n = ctypes.c_size_t(123)
    st = _lib._lib.cp_attn_workspace_size(ctypes.byref(a), ctypes.byref(n))
    del keep
    return st, n.value


@pytest.mark.parametrize("kw,want", [
    (dict(hq=3), _lib.CP_ERR_ARG),                     # hq % hkv
    (dict(hkv=0), _lib.CP_ERR_ARG),
    (dict(dqk=96), _lib.CP_ERR_UNSUPPORTED),
    (dict(dv=64), _lib.CP_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.CP_ERR_UNSUPPORTED),
    (dict(o_dtype=9), _lib.CP_ERR_UNSUPPORTED),
    (dict(dtype=_lib.CP_F32, dqk=192, dv=128), _lib.CP_ERR_UNSUPPORTED),
    (dict(num_q_rows=7), _lib.CP_ERR_ARG),             # segment beyond the q rows
    (dict(num_kv_rows=15), _lib.CP_ERR_ARG),           # segment beyond the kv rows
    (dict(num_q_rows=-1), _lib.CP_ERR_ARG),
    (dict(scale=float("nan")), _lib.CP_ERR_ARG),
    (dict(q=0), _lib.CP_ERR_ARG),                      # NULL
    (dict(lse=0), _lib.CP_ERR_ARG),
    (dict(q=FAKE + 8), _lib.CP_ERR_ARG),               # misaligned
    (dict(k_row_stride=250), _lib.CP_ERR_ARG),         # stride not a multiple of 8
    (dict(o_head_stride=130), _lib.CP_ERR_ARG),
    (dict(accumulate=2), _lib.CP_ERR_ARG),
])
def test_attn_arg_errors(kw, want):
    assert _fwd(**kw) == want
    # the allocation-free entry point checks its arguments the same way,
    # before it looks up any device scratch
    a, keep = _args(**kw)
    assert _lib._lib.cp_attn_fwd_noalloc(ctypes.byref(a), None) == want
    del keep


def test_noalloc_rejects_calls_beyond_its_scratch():
    # one long segment, 4 heads: 112 workgroups of 256 rows, so the 2^20 keys
    # are cut into 16 chunks (7 rounds of workgroups); fp32 partials of
    # 16 x 7168 rows x 4 heads x 128 need more than the static scratch; the
    # call must say so and enqueue nothing (no device is touched)
    segs = (_lib.Segment * 1)(_lib.Segment(0, 0, 7168, (1 << 20) - 7168, 1, 0, 1 << 20))
    kw = dict(num_q_rows=7168, num_kv_rows=1 << 20, hq=4, hkv=4, o_dtype=_lib.CP_F32,
              k_row_stride=512, v_row_stride=512, num_segs=1, segs=segs)
    st, need = _ws(**kw)
    assert st == _lib.CP_OK and need > _lib.NOALLOC_SCRATCH_BYTES
    a, keep = _args(**kw)
    assert _lib._lib.cp_attn_fwd_noalloc(ctypes.byref(a), None) == _lib.CP_ERR_SMALL_BUFFER
    msg = _lib.last_error()
    assert str(need) in msg and str(_lib.NOALLOC_SCRATCH_BYTES) in msg, msg
    del keep


def test_attn_segment_errors():
    bad = [
        _lib.Segment(0, 5, 4, 0, 1, 0, 4),       # q_end < q_begin
        _lib.Segment(0, -1, 4, 0, 1, 0, 4),
        _lib.Segment(0, 0, 4, 0, -1, 0, 4),      # negative stride
        _lib.Segment(0, 0, 4, 0, 1, 3, 2),       # kv_end < kv_begin
        _lib.Segment(0, 0, 4, 2**30, 1, 0, 4),   # positions out of range
    ]
    for s in bad:
        arr = (_lib.Segment * 1)(s)
        assert _fwd(segs=arr, num_segs=1) == _lib.CP_ERR_ARG, s
    assert _fwd(segs=None, num_segs=1) == _lib.CP_ERR_ARG


def test_workspace_size_query():
    # bf16: one int32 flag per workgroup; 2 segments of 4 rows x 4 heads = 8
    assert _ws() == (_lib.CP_OK, 32)
    # 8 query heads over 2 KV heads: GQA packing puts the 4 query heads of a
    # KV head in one workgroup, so 2 segments x 2 head groups = 4 flags
    assert _ws(hq=8, hkv=2, q_row_stride=1024, o_row_stride=1024, lse_row_stride=8) == (_lib.CP_OK, 16)
    # 12 over 4 (3 per KV head): no packing, 2 x 12 flags
    assert _ws(hq=12, hkv=4, q_row_stride=1536, o_row_stride=1536, lse_row_stride=12) == (_lib.CP_OK, 96)
    assert _ws(dtype=_lib.CP_F32, o_dtype=_lib.CP_F32) == (_lib.CP_OK, 0)
    assert _ws(hq=3)[0] == _lib.CP_ERR_ARG


def test_split_workspace_size():
    # one 512-row causal segment against 8192 keys, 32 heads over 8 KV heads,
    # bf16 out: 4 x 32 128-row workgroups (< 512), so the keys are split.  With
    # GQA packing a workgroup takes 64 rows x 4 heads: 8 x 8 per chunk, and the
    # launch model picks 4 chunks of 2048 keys (256 workgroups, one round):
    # flags 4 x 64 x 4 B + partial O 4 x 512 x 32 x 128 x 2 B + LSE 4 x 512 x 32 x 4 B
    segs = (_lib.Segment * 1)(_lib.Segment(0, 0, 512, 7680, 1, 0, 8192))
    kw = dict(num_q_rows=512, num_kv_rows=8192, hq=32, hkv=8, q_row_stride=32 * 128,
              k_row_stride=8 * 128, v_row_stride=8 * 128, o_row_stride=32 * 128,
              lse_row_stride=32, segs=segs, num_segs=1)
    split_bytes = 1024 + 4 * 512 * 32 * 128 * 2 + 4 * 512 * 32 * 4
    assert _ws(**kw) == (_lib.CP_OK, split_bytes)
    # partial rows cover only the segments' rows, not the whole output buffer
    assert _ws(**dict(kw, num_q_rows=100000)) == (_lib.CP_OK, split_bytes)
    # non-dense output rows: no split, flags of the 4 x 32 128-row workgroups only
    assert _ws(**dict(kw, o_row_stride=32 * 128 + 8)) == (_lib.CP_OK, 512)
    # 1000 keys: 4 chunks of 256 (8 tiles each, against 32 unsplit)
    k1000 = (_lib.Segment * 1)(_lib.Segment(0, 0, 512, 488, 1, 0, 1000))
    assert _ws(**dict(kw, segs=k1000)) == (
        _lib.CP_OK, 1024 + 4 * 512 * 32 * 128 * 2 + 4 * 512 * 32 * 4)
    # short keys (under two chunks of the 256-key minimum): nothing to split
    short = (_lib.Segment * 1)(_lib.Segment(0, 0, 512, 0, 1, 0, 400))
    assert _ws(**dict(kw, segs=short)) == (_lib.CP_OK, 512)
    # accumulate mode never splits
    assert _ws(**dict(kw, accumulate=1)) == (_lib.CP_OK, 512)


def test_attn_workspace_required():
    # the bf16 path needs its flag workspace: refused before any launch
    assert _fwd() == _lib.CP_ERR_SMALL_BUFFER
    assert _fwd(workspace=FAKE, workspace_bytes=16) == _lib.CP_ERR_SMALL_BUFFER
    assert _fwd(workspace=FAKE + 4, workspace_bytes=64) == _lib.CP_ERR_ARG   # misaligned


def _paged(segs, **kw):
    # MLA decode shape over a paged pool of 4 blocks of 64 rows
    arr = (_lib.Segment * len(segs))(*segs)
    base = dict(hq=128, hkv=1, dqk=576, dv=512, num_q_rows=2, num_kv_rows=256,
                q_row_stride=128 * 576, q_head_stride=576, k_row_stride=576, k_head_stride=576,
                v_row_stride=576, v_head_stride=576, o_row_stride=128 * 512, o_head_stride=512,
                lse_row_stride=128, block_table=FAKE, block_table_stride=8, block_size=64,
                segs=arr, num_segs=len(segs))
    base.update(kw)
    return base


def test_paged_kv_arg_errors():
    S = _lib.Segment
    ok = [S(0, 0, 1, 600, 1, 0, 512), S(1, 1, 2, 100, 1, 64, 96)]
    # logical rows may exceed the pool (512 > 256 rows): only the workspace query
    st, n = _ws(**_paged(ok))
    assert st == _lib.CP_OK and n > 0
    bad = [
        (_paged(ok, block_size=48), _lib.CP_ERR_ARG),        # not a multiple of 32
        (_paged(ok, block_size=0), _lib.CP_ERR_ARG),
        (_paged(ok, block_table_stride=0), _lib.CP_ERR_ARG),
        (_paged(ok, num_kv_rows=32), _lib.CP_ERR_ARG),       # pool smaller than a block
        (_paged([S(0, 0, 1, 600, 1, 16, 512)]), _lib.CP_ERR_ARG),   # kv_begin off a tile
        (_paged([S(0, 0, 1, 600, 1, 0, 513)]), _lib.CP_ERR_ARG),    # past the request's table
        (_paged([S(-1, 0, 1, 600, 1, 0, 64)]), _lib.CP_ERR_ARG),    # no table row
        (dict(block_table=FAKE, block_table_stride=8, block_size=64), _lib.CP_ERR_UNSUPPORTED),
    ]
    for kw, want in bad:
        assert _ws(**kw)[0] == want, kw
        assert _fwd(**kw) == want, kw


def test_merge_arg_errors():
    L = _lib._lib
    def m(parts=2, rows=4, heads=2, dv=128, op=FAKE, pdt=1, ops=1024, lp=FAKE, lps=8,
          oo=FAKE, odt=1, lo=FAKE):
        return L.cp_lse_merge(parts, rows, heads, dv, op, pdt, ops, lp, lps, oo, odt, lo, None)
    assert m(parts=0) == _lib.CP_ERR_ARG
    assert m(rows=-1) == _lib.CP_ERR_ARG
    assert m(dv=12) == _lib.CP_ERR_ARG
    assert m(dv=192) == _lib.CP_ERR_ARG          # 24 lanes do not tile a workgroup
    assert m(pdt=5) == _lib.CP_ERR_UNSUPPORTED
    assert m(odt=5) == _lib.CP_ERR_UNSUPPORTED
    assert m(op=0) == _lib.CP_ERR_ARG
    assert m(op=FAKE + 4) == _lib.CP_ERR_ARG
    assert m(ops=1000) == _lib.CP_ERR_ARG        # parts overlap
    assert m(lps=7) == _lib.CP_ERR_ARG
    assert m(rows=0) == _lib.CP_OK               # nothing to do, nothing enqueued


# ---------------------------------------------------------------- pass selection, ring padding,
# restore gather argument checks
from oracle import select_oracle as so  # noqa: E402


def test_choose_pass_matches_oracle():
    rng = np.random.default_rng(11)
    cases = [(1, 131071, 128, 8), (16384, 114688, 128, 8), (16385, 114687, 128, 8),
             (131072, 0, 128, 8), (131072, 0, 8, 8), (7, 0, 32, 8), (100, 1 << 40, 64, 1)]
    cases += [(int(rng.integers(1, 1 << 20)), int(rng.integers(0, 1 << 22)),
               int(h), int(k)) for h, k in [(128, 8), (32, 8), (64, 4), (16, 16)] * 25]
    for T, P, nh, nkv in cases:
        p, m, h = cp.choose_pass(T, P, nh, nkv)
        assert p == so.choose_pass(T, P, nh, nkv), (T, P, nh, nkv)
        assert m == float(so.miss_rate(T, P))
        assert abs(h - so.h_score(T, P)) <= 1e-9 * max(1.0, abs(h))


def test_choose_pass_errors():
    L = _lib._lib
    p = ctypes.c_int32()
    for args in [(0, 5, 8, 8), (1, -1, 8, 8), (1, 0, 0, 1), (1, 0, 8, 0), (1, 0, 4, 8), (1 << 50, 0, 8, 8)]:
        assert L.cp_choose_pass(*args, ctypes.byref(p), None, None) == _lib.CP_ERR_ARG, args
    assert L.cp_choose_pass(5, 0, 8, 8, None, None, None) == _lib.CP_OK


def test_ring_pad_len_matches_oracle():
    assert cp.ring_pad_len(3, [100, 300, 200], 10) == so.ring_pad_len([100, 300, 200], 10) == 304
    rng = np.random.default_rng(5)
    for _ in range(50):
        N = int(rng.integers(1, 17))
        Ps = [int(x) for x in rng.integers(0, 1 << 30, size=N)]
        T = int(rng.integers(0, 1 << 30))
        assert cp.ring_pad_len(N, Ps, T) == so.ring_pad_len(Ps, T)
    L = _lib._lib
    out = ctypes.c_int64()
    arr = (ctypes.c_int64 * 2)(1, -1)
    assert L.cp_ring_pad_len(2, arr, 3, ctypes.byref(out)) == _lib.CP_ERR_ARG
    assert L.cp_ring_pad_len(0, arr, 3, ctypes.byref(out)) == _lib.CP_ERR_ARG
    assert L.cp_ring_pad_len(2, None, 3, ctypes.byref(out)) == _lib.CP_ERR_ARG


def test_restore_apply_arg_errors():
    L = _lib._lib
    def ra(idx=FAKE, n=4, src=FAKE, rows=8, ss=64, dst=FAKE, ds=64, rb=64):
        return L.cp_restore_apply(idx, n, src, rows, ss, dst, ds, rb, None)
    assert ra(n=-1) == _lib.CP_ERR_ARG
    assert ra(idx=0) == _lib.CP_ERR_ARG
    assert ra(dst=0) == _lib.CP_ERR_ARG
    assert ra(rb=24) == _lib.CP_ERR_ARG          # not a multiple of 16
    assert ra(ss=48) == _lib.CP_ERR_ARG          # stride below the row
    assert ra(ds=72) == _lib.CP_ERR_ARG
    assert ra(dst=FAKE + 8) == _lib.CP_ERR_ARG   # misaligned
    assert ra(n=0) == _lib.CP_OK                 # nothing to do, nothing enqueued
    assert ra(rb=0) == _lib.CP_OK

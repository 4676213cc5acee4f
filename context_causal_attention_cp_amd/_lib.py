"""ctypes binding of libcpattn (include/cp_attn.h).

Argument marshalling only: every step of the path runs in the library.
PyTorch supplies device memory and the current HIP stream.  If the shared
library is missing the import fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcpattn.so")

CP_OK, CP_ERR_ARG, CP_ERR_UNSUPPORTED, CP_ERR_SMALL_BUFFER, CP_ERR_DEVICE = range(5)
CP_ZIGZAG, CP_INTERLEAVE = 0, 1
CP_F32, CP_BF16 = 0, 1

EXPORTS = ("cp_shard_plan", "cp_restore_index", "cp_restore_apply", "cp_choose_pass",
           "cp_ring_pad_len", "cp_attn_workspace_size", "cp_attn_fwd", "cp_attn_fwd_noalloc",
           "cp_lse_merge", "cp_status_str", "cp_last_error", "cp_version", "cp_calib_mfma",
           "cp_calib_copy")
NOALLOC_SCRATCH_BYTES = 128 << 20   # CP_NOALLOC_SCRATCH_BYTES

_STRATEGY = {"zigzag": CP_ZIGZAG, "interleave": CP_INTERLEAVE}


class CpError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = last_error() if status in (CP_ERR_DEVICE, CP_ERR_SMALL_BUFFER) else ""
        super().__init__(f"{what}: {status_str(status)} ({status}) {detail}".rstrip())


class Segment(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("req", "q_begin", "q_end", "pos_begin", "pos_stride", "kv_begin", "kv_end")]

    def astuple(self):
        return (self.req, self.q_begin, self.q_end, self.pos_begin, self.pos_stride,
                self.kv_begin, self.kv_end)

    def __repr__(self):
        return "Segment(%d, %d, %d, %d, %d, %d, %d)" % self.astuple()


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
        ("num_q_rows", ctypes.c_int32), ("num_kv_rows", ctypes.c_int32),
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("dqk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("k_row_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
        ("v", ctypes.c_void_p), ("v_row_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
        ("o", ctypes.c_void_p), ("o_row_stride", ctypes.c_int64), ("o_head_stride", ctypes.c_int64),
        ("lse", ctypes.c_void_p), ("lse_row_stride", ctypes.c_int64),
        ("segs", ctypes.POINTER(Segment)), ("num_segs", ctypes.c_int32),
        ("kv_pos", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("accumulate", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
    ]


def _load():
    # PyTorch brings its own HIP runtime (same soname, libamdhip64.so.7).  It
    # must be loaded before libcpattn so that the library's dependency
    # resolves to that one runtime: the streams and device memory the
    # library is handed belong to it.  Loading the library first would map a
    # second runtime into the process, and torch's stream handles would be
    # foreign to it.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python context_causal_attention_cp_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.cp_shard_plan.restype = i32
    lib.cp_shard_plan.argtypes = [i32, i32, i32, i32, pi32, pi32, ctypes.POINTER(Segment), i32,
                                  pi32, pi32, pi32, i32, pi32, pi32]
    lib.cp_restore_index.restype = i32
    lib.cp_restore_index.argtypes = [i32, i32, i32, pi32, pi32, i32, pi32]
    lib.cp_restore_apply.restype = i32
    lib.cp_restore_apply.argtypes = [vp, i64, vp, i64, i64, vp, i64, i64, vp]
    lib.cp_choose_pass.restype = i32
    lib.cp_choose_pass.argtypes = [i64, i64, i32, i32, pi32, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_double)]
    lib.cp_ring_pad_len.restype = i32
    lib.cp_ring_pad_len.argtypes = [i32, ctypes.POINTER(ctypes.c_int64), i64,
                                    ctypes.POINTER(ctypes.c_int64)]
    lib.cp_calib_mfma.restype = i32
    lib.cp_calib_mfma.argtypes = [i32, i32, vp, vp]
    lib.cp_calib_copy.restype = i32
    lib.cp_calib_copy.argtypes = [vp, vp, i64, vp]
    lib.cp_attn_workspace_size.restype = i32
    lib.cp_attn_workspace_size.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.cp_attn_fwd.restype = i32
    lib.cp_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), vp]
    lib.cp_attn_fwd_noalloc.restype = i32
    lib.cp_attn_fwd_noalloc.argtypes = [ctypes.POINTER(AttnArgs), vp]
    lib.cp_lse_merge.restype = i32
    lib.cp_lse_merge.argtypes = [i32, i32, i32, i32, vp, i32, i64, vp, i64, vp, i32, vp, vp]
    lib.cp_status_str.restype = ctypes.c_char_p
    lib.cp_status_str.argtypes = [i32]
    lib.cp_last_error.restype = ctypes.c_char_p
    lib.cp_last_error.argtypes = []
    lib.cp_version.restype = ctypes.c_char_p
    lib.cp_version.argtypes = []
    return lib


_lib = _load()


def status_str(status: int) -> str:
    return _lib.cp_status_str(int(status)).decode()


def last_error() -> str:
    return _lib.cp_last_error().decode()


def version() -> str:
    return _lib.cp_version().decode()


def _i32_array(xs: Sequence[int]):
    arr = np.ascontiguousarray(np.asarray(list(xs), dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _strategy(s) -> int:
    if isinstance(s, str):
        if s not in _STRATEGY:
            raise ValueError(f"unknown strategy {s!r}")
        return _STRATEGY[s]
    return int(s)


@dataclass
class ShardPlan:
    segments: List[Segment]
    positions: np.ndarray     # int32 [num_local]
    global_idx: np.ndarray    # int32 [num_local]
    num_local: int
    padded_local: int

    def segment_array(self):
        arr = (Segment * max(1, len(self.segments)))()
        for i, s in enumerate(self.segments):
            arr[i] = s
        return arr


def shard_plan(strategy, cp_size: int, cp_rank: int, new_lens: Sequence[int],
               prefix_lens: Optional[Sequence[int]] = None) -> ShardPlan:
    """cp_shard_plan: this rank's segments, positions and flattened indices."""
    st = _strategy(strategy)
    B = len(new_lens)
    tl, tp = _i32_array(new_lens)
    if prefix_lens is None:
        pl, pp = None, None
    else:
        if len(prefix_lens) != B:
            raise ValueError("prefix_lens length differs from new_lens")
        pl, pp = _i32_array(prefix_lens)
    nseg, nloc, pad = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    s = _lib.cp_shard_plan(st, cp_size, cp_rank, B, tp, pp, None, 0, ctypes.byref(nseg),
                           None, None, 0, ctypes.byref(nloc), ctypes.byref(pad))
    if s != CP_OK:
        raise CpError(s, "cp_shard_plan")
    segs = (Segment * max(1, nseg.value))()
    pos = np.zeros(max(1, nloc.value), dtype=np.int32)
    gidx = np.zeros(max(1, nloc.value), dtype=np.int32)
    s = _lib.cp_shard_plan(st, cp_size, cp_rank, B, tp, pp, segs, nseg.value, ctypes.byref(nseg),
                           pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                           gidx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), nloc.value,
                           ctypes.byref(nloc), ctypes.byref(pad))
    if s != CP_OK:
        raise CpError(s, "cp_shard_plan")
    del tl, pl
    return ShardPlan([segs[i] for i in range(nseg.value)], pos[:nloc.value].copy(),
                     gidx[:nloc.value].copy(), nloc.value, pad.value)


def restore_index(strategy, cp_size: int, new_lens: Sequence[int]):
    """cp_restore_index: (restore int32 [sum T], padded_local)."""
    st = _strategy(strategy)
    tl, tp = _i32_array(new_lens)
    total = int(sum(new_lens))
    out = np.zeros(max(1, total), dtype=np.int32)
    pad = ctypes.c_int32()
    s = _lib.cp_restore_index(st, cp_size, len(new_lens), tp,
                              out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), total,
                              ctypes.byref(pad))
    if s != CP_OK:
        raise CpError(s, "cp_restore_index")
    del tl
    return out[:total].copy(), pad.value


# ---------------------------------------------------------------- GPU calls

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CP_BF16
    if t.dtype == torch.float32:
        return CP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    return _torch().cuda.current_stream() if stream is None else stream


def _stream_handle(stream) -> int:
    return int(_stream(stream).cuda_stream)


def _segments_arg(segs):
    if isinstance(segs, ShardPlan):
        segs = segs.segments
    arr = (Segment * max(1, len(segs)))()
    for i, s in enumerate(segs):
        arr[i] = s if isinstance(s, Segment) else Segment(*[int(x) for x in s])
    return arr, len(segs)


def _check_3d(name, t, rows_dim=None):
    if t.dim() != 3:
        raise ValueError(f"{name} must be [rows, heads, dim]")
    if t.stride(2) != 1:
        raise ValueError(f"{name} must be contiguous in its last dim")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def attn_args(q, k, v, segs, scale: float, o, lse, causal: bool = True, kv_pos=None,
              workspace=None, accumulate: bool = False, block_table=None, block_size: int = 0):
    """Fill an AttnArgs from tensors (no call).

    Paged KV: block_table int32 [requests, blocks per request] (rows
    contiguous), k / v the pool of blocks of block_size rows; kv_pos, if
    given, is int32 [requests * blocks per request * block_size] by logical
    row."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_3d(name, t)
    if k.shape[0] != v.shape[0] or k.shape[1] != v.shape[1] or q.shape[2] != k.shape[2]:
        raise ValueError("q/k/v shapes disagree")
    if o.shape[0] != q.shape[0] or o.shape[1] != q.shape[1] or o.shape[2] != v.shape[2]:
        raise ValueError("o has the wrong shape")
    if lse.dim() != 2 or lse.shape[0] != q.shape[0] or lse.shape[1] != q.shape[1] or \
            lse.stride(1) != 1 or lse.dtype != _torch().float32:
        raise ValueError("lse must be fp32 [rows, hq] with contiguous heads")
    kv_rows = k.shape[0]
    if block_table is not None:
        if block_table.dtype != _torch().int32 or block_table.dim() != 2 or \
                block_table.stride(1) != 1:
            raise ValueError("block_table must be int32 [requests, blocks] with contiguous rows")
        kv_rows = block_table.shape[0] * block_table.stride(0) * int(block_size)
    if kv_pos is not None:
        if kv_pos.dtype != _torch().int32 or kv_pos.dim() != 1 or kv_pos.shape[0] != kv_rows \
                or not kv_pos.is_contiguous():
            raise ValueError("kv_pos must be int32 [kv rows], contiguous")
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share a dtype")
    seg_arr, nseg = _segments_arg(segs)
    a = AttnArgs()
    a.dtype, a.o_dtype = dt, _dtype_code(o)
    a.num_q_rows, a.num_kv_rows = q.shape[0], k.shape[0]
    a.hq, a.hkv, a.dqk, a.dv = q.shape[1], k.shape[1], q.shape[2], v.shape[2]
    a.scale, a.causal = float(scale), 1 if causal else 0
    a.q, a.q_row_stride, a.q_head_stride = q.data_ptr(), q.stride(0), q.stride(1)
    a.k, a.k_row_stride, a.k_head_stride = k.data_ptr(), k.stride(0), k.stride(1)
    a.v, a.v_row_stride, a.v_head_stride = v.data_ptr(), v.stride(0), v.stride(1)
    a.o, a.o_row_stride, a.o_head_stride = o.data_ptr(), o.stride(0), o.stride(1)
    a.lse, a.lse_row_stride = lse.data_ptr(), lse.stride(0)
    a.segs, a.num_segs = seg_arr, nseg
    a.kv_pos = kv_pos.data_ptr() if kv_pos is not None else None
    a.accumulate = 1 if accumulate else 0
    if block_table is not None:
        a.block_table = block_table.data_ptr()
        a.block_table_stride, a.block_size = block_table.stride(0), int(block_size)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a, seg_arr


def attn_workspace_size(a: AttnArgs) -> int:
    n = ctypes.c_size_t()
    s = _lib.cp_attn_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if s != CP_OK:
        raise CpError(s, "cp_attn_workspace_size")
    return n.value


def attn_fwd(q, k, v, segs, scale: float, causal: bool = True, kv_pos=None, o=None,
             lse=None, o_dtype=None, workspace=None, stream=None, accumulate: bool = False,
             block_table=None, block_size: int = 0):
    """cp_attn_fwd.  Returns (o [rows, hq, dv], lse fp32 [rows, hq]).

    Outputs are allocated with torch.empty when not given (rows that no
    segment covers are left as allocated).  accumulate=True merges each row's
    new partial into the (o, lse) given (lse = -inf: empty accumulator).
    block_table / block_size: paged KV (see attn_args)."""
    if accumulate and (o is None or lse is None):
        raise ValueError("accumulate needs the running o and lse")
    torch = _torch()
    stream = _stream(stream)
    # buffers allocated here belong to the stream the kernels run on: the
    # caching allocator then hands a freed block to other work only in that
    # stream's order, never while these kernels may still use it
    with torch.cuda.stream(stream):
        if o is None:
            o = torch.empty((q.shape[0], q.shape[1], v.shape[2]), device=q.device,
                            dtype=o_dtype if o_dtype is not None else q.dtype)
        if lse is None:
            lse = torch.empty((q.shape[0], q.shape[1]), device=q.device, dtype=torch.float32)
        a, keep = attn_args(q, k, v, segs, scale, o, lse, causal, kv_pos, workspace, accumulate,
                            block_table, block_size)
        need = attn_workspace_size(a)
        if need and (workspace is None or a.workspace_bytes < need):
            workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
            a.workspace, a.workspace_bytes = workspace.data_ptr(), need
    s = _lib.cp_attn_fwd(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream)))
    del keep
    if s != CP_OK:
        raise CpError(s, "cp_attn_fwd")
    return o, lse


def attn_fwd_noalloc(q, k, v, segs, scale: float, o, lse, causal: bool = True, kv_pos=None,
                     stream=None, accumulate: bool = False, block_table=None,
                     block_size: int = 0):
    """cp_attn_fwd_noalloc: as attn_fwd with caller-given outputs, the
    scratch taken from the library's static per-GPU array (no allocation
    here or in the library).  Returns (o, lse)."""
    a, keep = attn_args(q, k, v, segs, scale, o, lse, causal, kv_pos, None, accumulate,
                        block_table, block_size)
    s = _lib.cp_attn_fwd_noalloc(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream)))
    del keep
    if s != CP_OK:
        raise CpError(s, "cp_attn_fwd_noalloc")
    return o, lse


def lse_merge(o_parts, lse_parts, out_dtype=None, o_out=None, lse_out=None, stream=None):
    """cp_lse_merge over the leading dim: o_parts [P, rows, heads, dv],
    lse_parts [P, rows, heads] (each part contiguous).  Returns (o, lse)."""
    torch = _torch()
    if o_parts.dim() != 4 or lse_parts.dim() != 3:
        raise ValueError("o_parts must be [P, rows, heads, dv], lse_parts [P, rows, heads]")
    P, rows, heads, dv = o_parts.shape
    if tuple(lse_parts.shape) != (P, rows, heads) or lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be fp32 [P, rows, heads]")
    if not (o_parts[0].is_contiguous() and lse_parts[0].is_contiguous()):
        raise ValueError("each partial must be contiguous")
    stream = _stream(stream)
    with torch.cuda.stream(stream):   # outputs made here belong to the kernel's stream
        if o_out is None:
            o_out = torch.empty((rows, heads, dv), device=o_parts.device,
                                dtype=out_dtype if out_dtype is not None else o_parts.dtype)
        if lse_out is None:
            lse_out = torch.empty((rows, heads), device=o_parts.device, dtype=torch.float32)
    if not o_out.is_contiguous() or not lse_out.is_contiguous():
        raise ValueError("outputs must be contiguous")
    s = _lib.cp_lse_merge(P, rows, heads, dv, o_parts.data_ptr(), _dtype_code(o_parts),
                          o_parts.stride(0), lse_parts.data_ptr(), lse_parts.stride(0),
                          o_out.data_ptr(), _dtype_code(o_out), lse_out.data_ptr(),
                          ctypes.c_void_p(_stream_handle(stream)))
    if s != CP_OK:
        raise CpError(s, "cp_lse_merge")
    return o_out, lse_out

def restore_apply(index, src, out=None, stream=None):
    """cp_restore_apply: out[i] = src[index[i]] row-wise on the GPU.  ``index``
    int32 [n] on the device; ``src`` [rows, ...] with contiguous rows."""
    torch = _torch()
    if index.dtype != torch.int32 or index.dim() != 1 or not index.is_contiguous():
        raise ValueError("index must be a contiguous int32 vector")
    if src.dim() < 1 or not src[0:1].is_contiguous():
        raise ValueError("src rows must be contiguous")
    n = index.shape[0]
    stream = _stream(stream)
    if out is None:
        with torch.cuda.stream(stream):   # belongs to the kernel's stream
            out = torch.empty((n,) + tuple(src.shape[1:]), device=src.device, dtype=src.dtype)
    row_bytes = src[0:1].numel() * src.element_size() if src.shape[0] else 0
    s = _lib.cp_restore_apply(index.data_ptr(), n, src.data_ptr(), src.shape[0],
                              src.stride(0) * src.element_size(), out.data_ptr(),
                              out.stride(0) * out.element_size(), row_bytes,
                              ctypes.c_void_p(_stream_handle(stream)))
    if s != CP_OK:
        raise CpError(s, "cp_restore_apply")
    return out


def calib_mfma(workgroups: int, iters: int, out, stream=None):
    """cp_calib_mfma: the matrix-core loop; ``out`` fp32 [workgroups * 4] on
    the device receives 8 * 16 * iters per wave."""
    stream = _stream(stream)
    s = _lib.cp_calib_mfma(workgroups, iters, out.data_ptr(), ctypes.c_void_p(_stream_handle(stream)))
    if s != CP_OK:
        raise CpError(s, "cp_calib_mfma")
    return out


def calib_copy(src, dst, stream=None):
    """cp_calib_copy: dst[:] = src[:] (both contiguous device tensors of the
    same size in bytes, a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous and of the same size")
    stream = _stream(stream)
    s = _lib.cp_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                           ctypes.c_void_p(_stream_handle(stream)))
    if s != CP_OK:
        raise CpError(s, "cp_calib_copy")
    return dst


PASS_KV, PASS_Q = 0, 1


def choose_pass(new_tokens: int, cached_tokens: int, n_heads: int, n_kv_heads: int):
    """cp_choose_pass: (pass, miss_rate, h) -- PASS_Q when the miss rate is
    within 2 * n_kv_heads / n_heads, else PASS_KV; h is the printed empirical
    score (h > 0 favours pass-KV)."""
    p = ctypes.c_int32()
    m, h = ctypes.c_double(), ctypes.c_double()
    s = _lib.cp_choose_pass(new_tokens, cached_tokens, n_heads, n_kv_heads, ctypes.byref(p),
                            ctypes.byref(m), ctypes.byref(h))
    if s != CP_OK:
        raise CpError(s, "cp_choose_pass")
    return p.value, m.value, h.value


def ring_pad_len(cp_size: int, cached_per_rank: Sequence[int], new_tokens: int) -> int:
    """cp_ring_pad_len: max_i P_i + ceil(T / N)."""
    arr = (ctypes.c_int64 * max(1, len(cached_per_rank)))(*cached_per_rank)
    out = ctypes.c_int64()
    s = _lib.cp_ring_pad_len(cp_size, arr if cached_per_rank else None, new_tokens,
                             ctypes.byref(out))
    if s != CP_OK:
        raise CpError(s, "cp_ring_pad_len")
    return out.value

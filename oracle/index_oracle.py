"""Index oracle: which new tokens a CP rank owns, in what local order, with
which positions and causal KV extents; the restore permutation; causal tile
loads.  Pure Python integers, written for clarity, not speed.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources (the pages' titles and sections):

* "Prefill Context Parallelism" (SGLang docs), section "Zigzag strategy":
  each request's new tokens are cut into 2C contiguous blocks; rank r takes
  block r and block 2C-1-r; the cut restarts for every request; early blocks
  take the remainder when the length does not divide; buffers are padded;
  the metadata keeps separate q and kv lengths for the early and the late
  block, cached prefix included.
* Same page, section "Interleave strategy": rank r owns flattened new-token
  indices r, r+C, r+2C, ...; the index runs over the whole batch without
  resetting at request boundaries; positions keep their original values;
  the per-request metadata keeps each query's own causal extent.
* "What is Context Parallelism" (blog), section 2, figure on the split and
  causal-mask matrices: with C=4 and 2C query blocks, a contiguous split
  gives causal tile loads 3/7/11/15 and the zigzag pairing gives 9 each.
* Same blog, section 2.1 and section 5.1: after the all-gather a restore
  index puts the interleaved token order back into causal order.

Readings where the pages leave a step open:

* Remainder rule: block k of request b has floor(T/2C) tokens plus one more
  when k < T mod 2C (the first blocks are the "early blocks").
* Local row order: zigzag is request-major, and within a request the early
  block comes before the late block.  Interleave is ascending flattened index.
* A segment is one owned, non-empty block (zigzag) or the owned tokens of one
  request (interleave).  Its kv range is the request's rows in the gathered
  KV buffer (requests packed as prefix then new tokens) up to and including
  the segment's last query position (bottom-right causal alignment).
* Padding: every rank's slice of the gathered buffer has the length of the
  largest rank's slice; ``restore[g]`` is the slot of new token g in that
  rank-major, padded buffer, so ``gathered[restore]`` is causal order.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple


@dataclass(frozen=True)
class Token:
    req: int      # request index b
    t: int        # offset among request b's new tokens
    pos: int      # absolute position = prefix_b + t
    g: int        # flattened new-token index over the batch


@dataclass(frozen=True)
class Segment:
    req: int
    q_begin: int     # first local row
    q_end: int       # one past the last local row
    pos_begin: int   # position of row q_begin
    pos_stride: int  # position step between consecutive rows
    kv_begin: int    # first row of the request in the gathered KV buffer
    kv_end: int      # one past the last visible KV row of this segment


def _check(cp_size: int, new_lens: Sequence[int], prefix_lens: Sequence[int]):
    if cp_size < 1:
        raise ValueError("cp_size must be >= 1")
    if len(new_lens) != len(prefix_lens):
        raise ValueError("new_lens and prefix_lens differ in length")
    if any(x < 0 for x in new_lens) or any(x < 0 for x in prefix_lens):
        raise ValueError("lengths must be >= 0")


def zigzag_blocks(T: int, C: int) -> List[Tuple[int, int]]:
    """The 2C contiguous blocks [start, end) of T tokens; the first
    T mod 2C blocks hold one token more than the others."""
    n = 2 * C
    base, rem = divmod(T, n)
    blocks = []
    start = 0
    for k in range(n):
        size = base + (1 if k < rem else 0)
        blocks.append((start, start + size))
        start += size
    assert start == T
    return blocks


def _flat_offsets(new_lens):
    offs, acc = [], 0
    for t in new_lens:
        offs.append(acc)
        acc += t
    return offs


def _kv_offsets(new_lens, prefix_lens):
    offs, acc = [], 0
    for t, p in zip(new_lens, prefix_lens):
        offs.append(acc)
        acc += p + t
    return offs


def zigzag_tokens(C: int, r: int, new_lens, prefix_lens) -> List[Token]:
    _check(C, new_lens, prefix_lens)
    out = []
    goff = _flat_offsets(new_lens)
    for b, (T, P) in enumerate(zip(new_lens, prefix_lens)):
        blocks = zigzag_blocks(T, C)
        for k in (r, 2 * C - 1 - r):
            s, e = blocks[k]
            for t in range(s, e):
                out.append(Token(b, t, P + t, goff[b] + t))
    return out


def interleave_tokens(C: int, r: int, new_lens, prefix_lens) -> List[Token]:
    _check(C, new_lens, prefix_lens)
    out = []
    g = 0
    for b, (T, P) in enumerate(zip(new_lens, prefix_lens)):
        for t in range(T):
            if g % C == r:
                out.append(Token(b, t, P + t, g))
            g += 1
    return out


def rank_tokens(strategy: str, C: int, r: int, new_lens, prefix_lens) -> List[Token]:
    if not 0 <= r < C:
        raise ValueError("cp_rank out of range")
    if strategy == "zigzag":
        return zigzag_tokens(C, r, new_lens, prefix_lens)
    if strategy == "interleave":
        return interleave_tokens(C, r, new_lens, prefix_lens)
    raise ValueError(f"unknown strategy {strategy!r}")


def segments(strategy: str, C: int, r: int, new_lens, prefix_lens) -> List[Segment]:
    """Segments of rank r's local rows (see module docstring)."""
    toks = rank_tokens(strategy, C, r, new_lens, prefix_lens)
    kvoff = _kv_offsets(new_lens, prefix_lens)
    segs = []
    row = 0
    if strategy == "zigzag":
        for b, (T, P) in enumerate(zip(new_lens, prefix_lens)):
            blocks = zigzag_blocks(T, C)
            for k in (r, 2 * C - 1 - r):
                s, e = blocks[k]
                if e == s:
                    continue
                segs.append(Segment(b, row, row + (e - s), P + s, 1,
                                    kvoff[b], kvoff[b] + P + e))
                row += e - s
    else:
        for b, (T, P) in enumerate(zip(new_lens, prefix_lens)):
            mine = [tk for tk in toks if tk.req == b]
            if not mine:
                continue
            segs.append(Segment(b, row, row + len(mine), mine[0].pos, C,
                                kvoff[b], kvoff[b] + mine[-1].pos + 1))
            row += len(mine)
    assert row == len(toks)
    # every row's position must follow the segment's arithmetic rule
    for sg in segs:
        for i in range(sg.q_begin, sg.q_end):
            assert toks[i].pos == sg.pos_begin + (i - sg.q_begin) * sg.pos_stride
            assert toks[i].req == sg.req
    return segs


def padded_local(strategy: str, C: int, new_lens, prefix_lens=None) -> int:
    if prefix_lens is None:
        prefix_lens = [0] * len(new_lens)
    return max(len(rank_tokens(strategy, C, r, new_lens, prefix_lens)) for r in range(C))


def restore_index(strategy: str, C: int, new_lens) -> Tuple[List[int], int]:
    """restore[g] = slot of new token g in the rank-major gathered buffer of
    C x padded_local slots."""
    prefix = [0] * len(new_lens)
    pad = padded_local(strategy, C, new_lens, prefix)
    total = sum(new_lens)
    restore = [-1] * total
    for r in range(C):
        for i, tk in enumerate(rank_tokens(strategy, C, r, new_lens, prefix)):
            restore[tk.g] = r * pad + i
    assert all(x >= 0 for x in restore)
    return restore, pad


def gathered_global_idx(strategy: str, C: int, new_lens) -> List[int]:
    """The rank-major gathered buffer's content: flattened index per slot,
    -1 for padding."""
    prefix = [0] * len(new_lens)
    pad = padded_local(strategy, C, new_lens, prefix)
    out = []
    for r in range(C):
        toks = rank_tokens(strategy, C, r, new_lens, prefix)
        out += [tk.g for tk in toks] + [-1] * (pad - len(toks))
    return out


def sequential_tokens(C: int, r: int, T: int) -> List[int]:
    """Contiguous split (the unbalanced baseline): rank r owns T/C
    consecutive tokens, remainder to the first ranks."""
    base, rem = divmod(T, C)
    start = r * base + min(r, rem)
    size = base + (1 if r < rem else 0)
    return list(range(start, start + size))


def causal_tile_loads(owner_of_block: Sequence[int], C: int) -> List[int]:
    """Count, per rank, the tiles of the block-level causal mask it computes.

    The mask matrix has one row per query block and one column per key block;
    tile (i, j) is computed when j <= i (diagonal included, counted as one
    tile).  Row i is computed by ``owner_of_block[i]``."""
    nb = len(owner_of_block)
    loads = [0] * C
    for i in range(nb):
        for j in range(nb):
            if j <= i:
                loads[owner_of_block[i]] += 1
    return loads


def block_owners(layout: str, C: int) -> List[int]:
    """Owner rank of each of the 2C equal query blocks, derived from the
    token-level plans with one token per block."""
    T = 2 * C
    owner = [-1] * T
    for r in range(C):
        if layout == "sequential":
            toks = sequential_tokens(C, r, T)
        else:
            toks = [tk.g for tk in rank_tokens(layout, C, r, [T], [0])]
        for g in toks:
            owner[g] = r
    return owner


def visible_pairs(strategy: str, C: int, r: int, new_lens, prefix_lens) -> int:
    """Number of (query, key) pairs rank r computes per head: a query at
    position p sees the p+1 keys of its own request at positions 0..p."""
    return sum(tk.pos + 1 for tk in rank_tokens(strategy, C, r, new_lens, prefix_lens))

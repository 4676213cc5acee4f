// C ABI: argument checks, launch planning and kernel dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdio>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "cp_attn.h"
#include "internal.h"

using namespace cpattn;

namespace {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

enum class Path { None, Bf16Mfma, F32, DecodeMla };

Path pick_path(const cp_attn_args &a) {
  if (a.dtype == CP_BF16) {
    // MLA-absorbed latent attention: V must be the first 512 columns of K
    if (a.dqk == 576 && a.dv == 512)
      return (a.v == a.k && a.v_row_stride == a.k_row_stride &&
              a.v_head_stride == a.k_head_stride)
                 ? Path::DecodeMla
                 : Path::None;
    if ((a.dqk == 128 && a.dv == 128) || (a.dqk == 192 && a.dv == 128) ||
        (a.dqk == 64 && a.dv == 64))
      return Path::Bf16Mfma;
    return Path::None;
  }
  if (a.dtype == CP_F32) {
    if (a.dqk == a.dv && (a.dqk == 64 || a.dqk == 128)) return Path::F32;
    return Path::None;
  }
  return Path::None;
}

cp_status check_attn(const cp_attn_args *a) {
  if (!a) return CP_ERR_ARG;
  if (a->dtype != CP_BF16 && a->dtype != CP_F32) return CP_ERR_UNSUPPORTED;
  if (a->o_dtype != CP_BF16 && a->o_dtype != CP_F32) return CP_ERR_UNSUPPORTED;
  if (a->num_q_rows < 0 || a->num_kv_rows < 0 || a->num_segs < 0) return CP_ERR_ARG;
  if (a->accumulate != 0 && a->accumulate != 1) return CP_ERR_ARG;
  if (a->hq < 1 || a->hkv < 1 || a->hq % a->hkv != 0) return CP_ERR_ARG;
  if (a->dqk < 1 || a->dv < 1) return CP_ERR_ARG;
  if (!std::isfinite(a->scale) || !(a->scale > 0.f)) return CP_ERR_ARG;
  if (a->num_segs > 0 && !a->segs) return CP_ERR_ARG;
  for (int32_t i = 0; i < a->num_segs; ++i) {
    const cp_segment &s = a->segs[i];
    if (s.q_begin < 0 || s.q_end < s.q_begin || s.q_end > a->num_q_rows) return CP_ERR_ARG;
    if (s.kv_begin < 0 || s.kv_end < s.kv_begin) return CP_ERR_ARG;
    // paged KV: kv ranges count logical rows of the request (checked below)
    if (!a->block_table && s.kv_end > a->num_kv_rows) return CP_ERR_ARG;
    if (s.pos_stride < 0) return CP_ERR_ARG;
    // every row position must fit int32 with room for the kernels' sentinels
    const int64_t n = s.q_end - s.q_begin;
    if (n > 0) {
      const int64_t last = static_cast<int64_t>(s.pos_begin) + (n - 1) * s.pos_stride;
      if (s.pos_begin < -(1 << 29) || last > (INT32_MAX >> 1)) return CP_ERR_ARG;
    }
  }
  const Path path = pick_path(*a);
  if (path == Path::None) return CP_ERR_UNSUPPORTED;
  if (path == Path::Bf16Mfma) {
    // a K or V tile (up to 64 rows) is addressed with 32-bit byte offsets
    const int64_t rs = std::max(a->k_row_stride, a->v_row_stride);
    if (64 * rs * 2 > INT32_MAX) return CP_ERR_UNSUPPORTED;
  }
  if (a->block_table) {
    // paged KV: the decode shape only; blocks hold whole 32-row tiles
    if (path != Path::DecodeMla) return CP_ERR_UNSUPPORTED;
    if (a->block_size < 32 || a->block_size % 32 != 0 || a->block_table_stride < 1)
      return CP_ERR_ARG;
    if (a->num_kv_rows < a->block_size) return CP_ERR_ARG;
    for (int32_t i = 0; i < a->num_segs; ++i) {
      const cp_segment &g = a->segs[i];
      if (g.req < 0 || g.kv_begin % 32 != 0 ||
          g.kv_end > static_cast<int64_t>(a->block_table_stride) * a->block_size)
        return CP_ERR_ARG;
    }
    if (static_cast<int64_t>(a->block_size) * a->k_row_stride * 2 > INT32_MAX) return CP_ERR_UNSUPPORTED;
  }
  if (path == Path::DecodeMla && !a->block_table) {
    // the latent rows of a segment are addressed with 32-bit byte offsets
    for (int32_t i = 0; i < a->num_segs; ++i) {
      const int64_t rows = a->segs[i].kv_end - a->segs[i].kv_begin;
      if (rows * a->k_row_stride * 2 > INT32_MAX) return CP_ERR_UNSUPPORTED;
    }
  }
  return CP_OK;
}

cp_status check_attn_buffers(const cp_attn_args *a) {
  const bool any_rows = a->num_segs > 0;
  if (!any_rows) return CP_OK;
  if (!a->q || !a->k || !a->v || !a->o || !a->lse) return CP_ERR_ARG;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return CP_ERR_ARG;
  const int64_t in_vec = a->dtype == CP_BF16 ? 8 : 4;
  const int64_t out_vec = a->o_dtype == CP_BF16 ? 8 : 4;
  const int64_t s_in[6] = {a->q_row_stride, a->q_head_stride, a->k_row_stride,
                           a->k_head_stride, a->v_row_stride, a->v_head_stride};
  for (int64_t s : s_in)
    if (s < 0 || s % in_vec != 0) return CP_ERR_ARG;
  if (a->o_row_stride < 0 || a->o_head_stride < 0 || a->o_row_stride % out_vec != 0 ||
      a->o_head_stride % out_vec != 0)
    return CP_ERR_ARG;
  if (a->lse_row_stride < a->hq && a->num_q_rows > 1) return CP_ERR_ARG;
  return CP_OK;
}

AttnParams make_params(const cp_attn_args &a) {
  AttnParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.kv_pos = a.kv_pos;
  p.q_rs = a.q_row_stride;
  p.q_hs = a.q_head_stride;
  p.k_rs = a.k_row_stride;
  p.k_hs = a.k_head_stride;
  p.v_rs = a.v_row_stride;
  p.v_hs = a.v_head_stride;
  p.o_rs = a.o_row_stride;
  p.o_hs = a.o_head_stride;
  p.lse_rs = a.lse_row_stride;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.scale = a.scale;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.causal = a.causal ? 1 : 0;
  p.o_bf16 = a.o_dtype == CP_BF16;
  p.accumulate = a.accumulate ? 1 : 0;
  p.pack = 1;
  p.block_table = a.block_table;
  p.bt_stride = a.block_table_stride;
  p.block_size = a.block_size;
  p.pool_blocks = a.block_table && a.block_size > 0 ? a.num_kv_rows / a.block_size : 0;
  p.ws = a.workspace;
  p.ws_bytes = static_cast<int64_t>(a.workspace_bytes);
  return p;
}

// One segment as a launch sees it: the caller's segment, or one key chunk of
// it (split calls), with the row its outputs go to.
struct PlanSeg {
  cp_segment g;
  int32_t o_begin;
};

std::vector<PlanSeg> plain_segs(const cp_attn_args &a) {
  std::vector<PlanSeg> v;
  for (int32_t i = 0; i < a.num_segs; ++i) v.push_back({a.segs[i], a.segs[i].q_begin});
  return v;
}

// Splits the non-empty segments into launches of at most kMaxLaunchSegs,
// heaviest first (largest visible KV extent), numbering their tiles.
std::vector<LaunchSegs> plan_launches(const std::vector<PlanSeg> &segs, int tile_rows,
                                      bool causal) {
  std::vector<int32_t> order;
  for (size_t i = 0; i < segs.size(); ++i)
    if (segs[i].g.q_end > segs[i].g.q_begin && segs[i].g.kv_end > segs[i].g.kv_begin)
      order.push_back(static_cast<int32_t>(i));
  // segments with the most work first (the kernel starts the heaviest query
  // tiles of a segment first; across segments this order decides): more keys
  // first, and among equal key ranges of a causal call the later positions
  // (key positions increase, so a later row sees at least as many keys)
  auto last_pos = [&](int32_t x) {
    const cp_segment &g = segs[x].g;
    return static_cast<int64_t>(g.pos_begin) +
           static_cast<int64_t>(g.q_end - g.q_begin - 1) * g.pos_stride;
  };
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    const int32_t kx = segs[x].g.kv_end - segs[x].g.kv_begin;
    const int32_t ky = segs[y].g.kv_end - segs[y].g.kv_begin;
    if (kx != ky) return kx > ky;
    return causal && last_pos(x) > last_pos(y);
  });
  std::vector<LaunchSegs> out;
  for (size_t i = 0; i < order.size(); i += kMaxLaunchSegs) {
    LaunchSegs L{};
    const size_t n = std::min<size_t>(kMaxLaunchSegs, order.size() - i);
    int32_t tiles = 0;
    for (size_t j = 0; j < n; ++j) {
      const PlanSeg &ps = segs[order[i + j]];
      const cp_segment &s = ps.g;
      SegDesc &d = L.s[j];
      d.q_begin = s.q_begin;
      d.q_len = s.q_end - s.q_begin;
      d.pos_begin = s.pos_begin;
      d.pos_stride = s.pos_stride;
      d.kv_begin = s.kv_begin;
      d.kv_len = s.kv_end - s.kv_begin;
      d.tile_begin = tiles;
      d.req = s.req;
      d.o_begin = ps.o_begin;
      tiles += (d.q_len + tile_rows - 1) / tile_rows;
    }
    L.num_segs = static_cast<int32_t>(n);
    L.num_tiles = tiles;
    out.push_back(L);
  }
  return out;
}

// Below this many workgroups a bf16 call is too small to fill the 256
// compute units well.
constexpr int64_t kSmallGridWorkgroups = 512;
// Split calls: the key chunk size comes from a model of the launch.  W
// workgroups of 256 rows (one per compute unit: their LDS fills it) run in
// ceil(W / kComputeUnits) rounds, each as long as its longest workgroup: its
// key tiles plus a fixed cost of kWorkgroupFixedTiles tiles (Q load, the
// pipeline's fill and drain, the epilogue; measured on MI355X at qk 128:
// 1.0 us per 32-key tile and 12-13 us per workgroup).  Chunks have at least
// kMinSplitKeys keys, a segment at most kMaxSplitParts of them.
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kWorkgroupFixedTiles = 12;
constexpr int64_t kMinSplitKeys = 256;
constexpr int32_t kMaxSplitParts = 16;

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// The bf16 launch plan.  A call whose segments give fewer than
// kSmallGridWorkgroups 128-row workgroups has its long key ranges cut into
// chunks: every chunk of a segment is a launch segment of its own (same
// query rows, positions shifted with the chunk when they are implicit) that
// writes a normalised partial (O_s, LSE_s) to the workspace, and the parts
// of each segment are merged by log-sum-exp into the caller's rows
// ("What is Context Parallelism" blog, section 3.6: the merge is exact for
// any partition of the keys).  Otherwise: 256-row workgroups, or 128-row
// ones below kSmallGridWorkgroups, writing O and LSE directly.
struct Bf16Plan {
  int tile_rows = 0;               // query rows x heads of one workgroup, in rows of one head
  int pack = 1;                    // query heads per workgroup (GQA packing)
  int32_t parts = 0;               // > 0: split; parts per segment in seg_parts
  std::vector<int32_t> seg_parts;  // per caller segment
  std::vector<int32_t> seg_row;    // per caller segment: its first compact partial row
  int64_t part_rows = 0;           // compact rows per part (rows of the split segments)
  std::vector<LaunchSegs> launches;
  size_t flag_bytes = 0, part_o_bytes = 0, part_lse_bytes = 0;
  size_t bytes() const { return flag_bytes + part_o_bytes + part_lse_bytes; }
};

Bf16Plan plan_bf16(const cp_attn_args &a) {
  Bf16Plan P;
  const int small = attn_bf16_tile_rows(a.dqk, a.dv, true);
  const int big = attn_bf16_tile_rows(a.dqk, a.dv, false);
  int64_t wgs_small = 0, wgs_big = 0, max_kv = 0;
  for (int32_t i = 0; i < a.num_segs; ++i) {
    const cp_segment &g = a.segs[i];
    const int64_t nq = g.q_end - g.q_begin, nk = g.kv_end - g.kv_begin;
    if (nq <= 0 || nk <= 0) continue;
    wgs_small += (nq + small - 1) / small * a.hq;
    wgs_big += (nq + big - 1) / big * a.hq;
    max_kv = std::max(max_kv, nk);
  }
  // the merge writes whole (row, head) runs: dense O and LSE rows only
  const bool dense = a.o_head_stride == a.dv &&
                     a.o_row_stride == static_cast<int64_t>(a.hq) * a.dv &&
                     a.lse_row_stride == a.hq;
  // (fewer than kSmallGridWorkgroups 128-row workgroups also bounds the rows:
  // kMaxSplitParts x rows stays far inside int32)
  const bool can_split = !a.accumulate && !a.block_table && dense &&
                         wgs_small < kSmallGridWorkgroups && max_kv <= (1 << 28);
  // GQA packing: when every KV head serves a multiple of 4 query heads, a
  // workgroup takes 4 of them over tile_rows / 4 rows (each wave, or wave
  // pair, one head of the same rows), so the 4 heads share each K/V tile in
  // LDS and every wave sees the same key range ("What is Context
  // Parallelism" blog, section 4.1: the query heads of a group read the same
  // K and V)
  P.pack = (a.hkv > 0 && a.hq % a.hkv == 0 && (a.hq / a.hkv) % 4 == 0) ? 4 : 1;
  std::vector<PlanSeg> segs;
  if (can_split) {
    // the chunk size with the shortest modelled launch, among those that cut
    // some segment into 1 .. kMaxSplitParts equal whole-tile parts
    auto tiles32 = [](int64_t x) { return (x + 31) / 32 * 32; };
    auto parts_of = [](int64_t nk, int64_t c) {
      return std::min<int64_t>(kMaxSplitParts, (nk + c - 1) / c);
    };
    const int64_t rows_wg = big / P.pack, groups = a.hq / P.pack;
    std::vector<int64_t> cands;
    for (int32_t i = 0; i < a.num_segs; ++i) {
      const int64_t nk = a.segs[i].kv_end - a.segs[i].kv_begin;
      if (a.segs[i].q_end <= a.segs[i].q_begin || nk <= 0) continue;
      for (int64_t np = 1; np <= kMaxSplitParts; ++np) {
        const int64_t c = tiles32((nk + np - 1) / np);
        if (np == 1 || c >= kMinSplitKeys) cands.push_back(c);
      }
    }
    std::sort(cands.begin(), cands.end());
    cands.erase(std::unique(cands.begin(), cands.end()), cands.end());
    int64_t chunk = 0, best_est = 0, best_wgs = 0;
    for (const int64_t c : cands) {
      int64_t wgs = 0, tiles = 0;
      for (int32_t i = 0; i < a.num_segs; ++i) {
        const cp_segment &g = a.segs[i];
        const int64_t nq = g.q_end - g.q_begin, nk = g.kv_end - g.kv_begin;
        if (nq <= 0 || nk <= 0) continue;
        const int64_t np = parts_of(nk, c);
        wgs += np * ((nq + rows_wg - 1) / rows_wg) * groups;
        tiles = std::max(tiles, tiles32((nk + np - 1) / np) / 32);
      }
      const int64_t est = (wgs + kComputeUnits - 1) / kComputeUnits * (tiles + kWorkgroupFixedTiles);
      if (chunk == 0 || est < best_est || (est == best_est && wgs < best_wgs)) {
        chunk = c;
        best_est = est;
        best_wgs = wgs;
      }
    }
    P.seg_parts.assign(a.num_segs, 0);
    P.seg_row.assign(a.num_segs, 0);
    // partial rows are compact: the rows of the split segments, numbered in
    // segment order, one block of them per part
    for (int32_t i = 0; i < a.num_segs; ++i) {
      const cp_segment &g = a.segs[i];
      if (g.q_end > g.q_begin && g.kv_end > g.kv_begin) {
        P.seg_row[i] = static_cast<int32_t>(P.part_rows);
        P.part_rows += g.q_end - g.q_begin;
      }
    }
    for (int32_t i = 0; i < a.num_segs; ++i) {
      const cp_segment &g = a.segs[i];
      const int64_t nq = g.q_end - g.q_begin, nk = g.kv_end - g.kv_begin;
      if (nq <= 0 || nk <= 0) continue;
      const int64_t np = parts_of(nk, chunk);
      const int64_t c = tiles32((nk + np - 1) / np);  // whole tiles per chunk
      int32_t made = 0;
      for (int64_t off = 0; off < nk; off += c, ++made) {
        PlanSeg ps{g, 0};
        ps.g.kv_begin = static_cast<int32_t>(g.kv_begin + off);
        ps.g.kv_end = static_cast<int32_t>(std::min<int64_t>(g.kv_end, g.kv_begin + off + c));
        // implicit key positions count from the chunk start: shift the rows'
        // positions with it (kv_pos gives absolute positions)
        if (!a.kv_pos) ps.g.pos_begin = static_cast<int32_t>(g.pos_begin - off);
        ps.o_begin = static_cast<int32_t>(made * P.part_rows + P.seg_row[i]);
        segs.push_back(ps);
      }
      P.seg_parts[i] = made;
      P.parts = std::max(P.parts, made);
    }
    if (P.parts <= 1) {  // nothing long enough to split
      P.parts = 0;
      P.part_rows = 0;
      P.seg_parts.clear();
      P.seg_row.clear();
      segs.clear();
    }
  }
  if (P.parts > 0) {
    P.tile_rows = big;
    const size_t elt = a.o_dtype == CP_BF16 ? 2 : 4;
    P.part_o_bytes = round256(static_cast<size_t>(P.parts) * P.part_rows * a.hq * a.dv * elt);
    P.part_lse_bytes = round256(static_cast<size_t>(P.parts) * P.part_rows * a.hq * 4);
  } else {
    P.tile_rows = wgs_big < kSmallGridWorkgroups ? small : big;
    segs = plain_segs(a);
  }
  P.launches = plan_launches(segs, P.tile_rows / P.pack, a.causal != 0);
  int64_t wgs = 0;
  for (const LaunchSegs &L : P.launches) wgs += static_cast<int64_t>(L.num_tiles) * a.hq / P.pack;
  // one int32 flag per workgroup of every launch (16-byte rounded; the
  // partials that follow start on a 256-byte boundary)
  P.flag_bytes = (static_cast<size_t>(wgs) * 4 + 15) / 16 * 16;
  if (P.parts > 0) P.flag_bytes = round256(P.flag_bytes);
  return P;
}

size_t plan_decode(const cp_attn_args &a, std::vector<DecodeLaunch> *out) {
  const int G = a.hq / a.hkv;
  const int htiles = (G + kDecodeHeadsPerBlock - 1) / kDecodeHeadsPerBlock;
  size_t ws = 0;
  std::vector<int32_t> idx;
  for (int32_t i = 0; i < a.num_segs; ++i)
    if (a.segs[i].q_end > a.segs[i].q_begin && a.segs[i].kv_end > a.segs[i].kv_begin)
      idx.push_back(i);
  for (size_t i = 0; i < idx.size(); i += kMaxLaunchSegs) {
    DecodeLaunch D{};
    const size_t n = std::min<size_t>(kMaxLaunchSegs, idx.size() - i);
    int32_t items = 0, min_kv = INT32_MAX;
    for (size_t j = 0; j < n; ++j) {
      const cp_segment &g = a.segs[idx[i + j]];
      SegDesc &d = D.s[j];
      d.q_begin = g.q_begin;
      d.q_len = g.q_end - g.q_begin;
      d.pos_begin = g.pos_begin;
      d.pos_stride = g.pos_stride;
      d.kv_begin = g.kv_begin;
      d.kv_len = g.kv_end - g.kv_begin;
      d.req = g.req;
      d.tile_begin = items;
      items += d.q_len * a.hkv * htiles;
      min_kv = std::min(min_kv, d.kv_len);
    }
    // one workgroup per compute unit, slices of at least 256 keys
    const int32_t target = 256;
    int32_t nsplit = std::max<int32_t>(1, (target + items - 1) / items);
    nsplit = std::min<int32_t>(nsplit, std::max<int32_t>(1, min_kv / 256));
    if (a.block_table) {
      // a slice's block ids must fit the kernel's LDS table
      int32_t max_kv = 0;
      for (size_t j = 0; j < n; ++j) max_kv = std::max(max_kv, D.s[j].kv_len);
      const int64_t per = static_cast<int64_t>(kDecodeMaxSliceBlocks - 2) * a.block_size;
      nsplit = std::max<int32_t>(nsplit, static_cast<int32_t>((max_kv + per - 1) / per));
    }
    D.num_segs = static_cast<int32_t>(n);
    D.items = items;
    D.nsplit = nsplit;
    D.htiles = htiles;
    D.hkv = a.hkv;
    ws = std::max(ws, static_cast<size_t>(items) * nsplit *
                          (kDecodeHeadsPerBlock * (512 + 1) * sizeof(float) + sizeof(int32_t)));
    if (out) out->push_back(D);
  }
  return ws;
}

// Rows that no kernel writes because their segment sees no KV row at all
// (kv_end == kv_begin) still get O = 0, LSE = -inf: handled by a tiny fill.
__global__ void fill_empty_rows(float *lse, int64_t lse_rs, void *o, int64_t o_rs,
                                int64_t o_hs, int o_bf16, int hq, int dv, int q_begin,
                                int q_len) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)hq * dv;
  if (e >= per_row * q_len) return;
  const int64_t r = q_begin + e / per_row;
  const int h = (int)((e % per_row) / dv), d = (int)(e % dv);
  if (o_bf16)
    ((__bf16 *)o)[r * o_rs + h * o_hs + d] = (__bf16)0.f;
  else
    ((float *)o)[r * o_rs + h * o_hs + d] = 0.f;
  if (d == 0) lse[r * lse_rs + h] = -INFINITY;
}


// Segments that see no KV row at all get O = 0, LSE = -inf.
cp_status fill_empty_segments(const cp_attn_args *a, hipStream_t s) {
  if (a->accumulate) return CP_OK;  // an empty partial leaves the accumulator as it is
  for (int32_t i = 0; i < a->num_segs; ++i) {
    const cp_segment &g = a->segs[i];
    const int32_t n = g.q_end - g.q_begin;
    if (n > 0 && g.kv_end == g.kv_begin) {
      const int64_t elems = static_cast<int64_t>(n) * a->hq * a->dv;
      hipLaunchKernelGGL(fill_empty_rows, dim3((unsigned)((elems + 255) / 256)), dim3(256), 0,
                         s, a->lse, a->lse_row_stride, a->o, a->o_row_stride,
                         a->o_head_stride, a->o_dtype == CP_BF16 ? 1 : 0, a->hq, a->dv,
                         g.q_begin, n);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return cpattn::device_error(e);
    }
  }
  return CP_OK;
}

}  // namespace

extern "C" const char *cp_status_str(int32_t s) {
  switch (s) {
    case CP_OK: return "CP_OK";
    case CP_ERR_ARG: return "CP_ERR_ARG: invalid argument";
    case CP_ERR_UNSUPPORTED: return "CP_ERR_UNSUPPORTED: no kernel for this dtype/shape";
    case CP_ERR_SMALL_BUFFER: return "CP_ERR_SMALL_BUFFER: output capacity too small";
    case CP_ERR_DEVICE: return "CP_ERR_DEVICE: HIP launch error";
    default: return "unknown cp_status";
  }
}

extern "C" const char *cp_version(void) { return "0.1.0"; }

namespace {
thread_local char g_last_error[256] = "";
}  // namespace

namespace cpattn {
cp_status device_error(hipError_t e) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return CP_ERR_DEVICE;
}
}  // namespace cpattn

extern "C" const char *cp_last_error(void) { return g_last_error; }

extern "C" cp_status cp_attn_workspace_size(const cp_attn_args *a, size_t *bytes) {
  cp_status st = check_attn(a);
  if (st != CP_OK) return st;
  if (!bytes) return CP_ERR_ARG;
  *bytes = 0;
  const Path path = pick_path(*a);
  if (path == Path::DecodeMla) *bytes = plan_decode(*a, nullptr);
  if (path == Path::Bf16Mfma) *bytes = plan_bf16(*a).bytes();
  return CP_OK;
}

namespace {

// The attention call with its scratch in (ws, ws_bytes): the caller's
// workspace (cp_attn_fwd) or the library's static scratch
// (cp_attn_fwd_noalloc).  Arguments are already checked.
cp_status attn_fwd_impl(const cp_attn_args *a, void *ws_ptr, size_t ws_bytes, hipStream_t s) {
  AttnParams p = make_params(*a);
  p.ws = ws_ptr;
  p.ws_bytes = static_cast<int64_t>(ws_bytes);
  const Path path = pick_path(*a);
  (void)hipGetLastError();  // clear an error left by an earlier, unrelated call
  if (path == Path::DecodeMla) {
    std::vector<DecodeLaunch> launches;
    const size_t need = plan_decode(*a, &launches);
    if (need > 0 && (!ws_ptr || ws_bytes < need)) return CP_ERR_SMALL_BUFFER;
    if (need > 0 && !aligned16(ws_ptr)) return CP_ERR_ARG;
    for (DecodeLaunch &D : launches) {
      D.ws_o = static_cast<float *>(ws_ptr);
      D.ws_lse = D.ws_o + static_cast<size_t>(D.items) * D.nsplit * kDecodeHeadsPerBlock * 512;
      D.ws_flags = reinterpret_cast<int32_t *>(
          D.ws_lse + static_cast<size_t>(D.items) * D.nsplit * kDecodeHeadsPerBlock);
      const hipError_t e = launch_attn_decode_mla(p, D, s);
      if (e != hipSuccess) return device_error(e);
    }
    return fill_empty_segments(a, s);
  }
  if (path == Path::F32) {
    for (const LaunchSegs &L : plan_launches(plain_segs(*a), attn_f32_tile_rows(a->dqk), a->causal != 0)) {
      const hipError_t e = launch_attn_f32(p, L, a->dqk, s);
      if (e != hipSuccess) return device_error(e);
    }
    return fill_empty_segments(a, s);
  }
  // bf16: one int32 flag per workgroup, then (split calls) the partials
  const Bf16Plan P = plan_bf16(*a);
  const size_t need = P.bytes();
  if (need > 0 && (!ws_ptr || ws_bytes < need)) return CP_ERR_SMALL_BUFFER;
  if (need > 0 && !aligned16(ws_ptr)) return CP_ERR_ARG;
  char *ws = static_cast<char *>(ws_ptr);
  AttnParams q = p;
  const int o_bf16 = a->o_dtype == CP_BF16 ? 1 : 0;
  const int64_t part_rows = P.part_rows * a->hq;  // (row, head) pairs per part
  if (P.parts > 0) {
    // partial j of segment i's rows: compact rows j * part_rows + seg_row[i] + [0, q_len)
    q.o = ws + P.flag_bytes;
    q.o_rs = static_cast<int64_t>(a->hq) * a->dv;
    q.o_hs = a->dv;
    q.lse = reinterpret_cast<float *>(ws + P.flag_bytes + P.part_o_bytes);
    q.lse_rs = a->hq;
  }
  int32_t *flags = reinterpret_cast<int32_t *>(ws);
  q.pack = P.pack;
  for (const LaunchSegs &L : P.launches) {
    q.ws = flags;
    const hipError_t e = launch_attn_bf16(q, L, a->dqk, a->dv, P.tile_rows, s);
    if (e != hipSuccess) return device_error(e);
    flags += static_cast<int64_t>(L.num_tiles) * a->hq / P.pack;
  }
  // the split segments' merges, up to kMaxMergeSegs per launch
  if (P.parts > 0) {
    const int64_t ppw = lse_merge_pairs_per_workgroup(a->dv);
    MergeSegs T{};
    auto flush = [&]() -> hipError_t {
      if (T.n == 0) return hipSuccess;
      const hipError_t e = launch_lse_merge_segs(T, a->dv, q.o, o_bf16, part_rows, q.lse, a->o,
                                                 o_bf16, a->lse, s);
      T = MergeSegs{};
      return e;
    };
    for (int32_t i = 0; i < a->num_segs; ++i) {
      const cp_segment &g = a->segs[i];
      const int32_t np = P.seg_parts[i];
      if (np == 0) continue;
      const int64_t pairs = static_cast<int64_t>(g.q_end - g.q_begin) * a->hq;
      T.parts[T.n] = np;
      T.pairs[T.n] = pairs;
      T.src[T.n] = static_cast<int64_t>(P.seg_row[i]) * a->hq;  // first (row, head) pair
      T.dst[T.n] = static_cast<int64_t>(g.q_begin) * a->hq;
      T.wg_begin[T.n + 1] = T.wg_begin[T.n] + static_cast<int32_t>((pairs + ppw - 1) / ppw);
      if (++T.n == kMaxMergeSegs) {
        const hipError_t e = flush();
        if (e != hipSuccess) return device_error(e);
      }
    }
    const hipError_t e = flush();
    if (e != hipSuccess) return device_error(e);
  }
  return fill_empty_segments(a, s);
}

// Scratch of cp_attn_fwd_noalloc: one copy per GPU, in the code object's
// static device memory (the runtime places it when the library's code is
// loaded on that GPU; it stays until the process ends).  In host code the
// name `scratch` is only a handle for hipGetSymbolAddress, never a device
// address: kernels get the per-device address below.
static __device__ __align__(256) unsigned char scratch[CP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch, looked up once per device with that
// device current.
cp_status scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(e);
  if (dev < 0 || dev >= kMaxDevices) return CP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_error(e);
    if (!ptr) return CP_ERR_DEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CP_OK;
}

}  // namespace

extern "C" cp_status cp_attn_fwd(const cp_attn_args *a, void *stream) {
  cp_status st = check_attn(a);
  if (st != CP_OK) return st;
  st = check_attn_buffers(a);
  if (st != CP_OK) return st;
  return attn_fwd_impl(a, a->workspace, a->workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" cp_status cp_attn_fwd_noalloc(const cp_attn_args *a, void *stream) {
  cp_status st = check_attn(a);
  if (st != CP_OK) return st;
  st = check_attn_buffers(a);
  if (st != CP_OK) return st;
  size_t need = 0;
  const Path path = pick_path(*a);
  if (path == Path::DecodeMla) need = plan_decode(*a, nullptr);
  if (path == Path::Bf16Mfma) need = plan_bf16(*a).bytes();
  if (need > CP_NOALLOC_SCRATCH_BYTES) {
    snprintf(g_last_error, sizeof g_last_error,
             "cp_attn_fwd_noalloc: the call needs %zu bytes of scratch, the library holds %zu",
             need, static_cast<size_t>(CP_NOALLOC_SCRATCH_BYTES));
    return CP_ERR_SMALL_BUFFER;
  }
  void *ws = nullptr;
  if (need > 0) {
    st = scratch_for_current_device(&ws);
    if (st != CP_OK) return st;
  }
  return attn_fwd_impl(a, ws, need > 0 ? CP_NOALLOC_SCRATCH_BYTES : 0,
                       static_cast<hipStream_t>(stream));
}

extern "C" cp_status cp_lse_merge(int32_t num_parts, int32_t rows, int32_t heads,
                                  int32_t dv, const void *o_parts, int32_t part_dtype,
                                  int64_t o_part_stride, const float *lse_parts,
                                  int64_t lse_part_stride, void *o_out, int32_t out_dtype,
                                  float *lse_out, void *stream) {
  if ((part_dtype != CP_BF16 && part_dtype != CP_F32) ||
      (out_dtype != CP_BF16 && out_dtype != CP_F32))
    return CP_ERR_UNSUPPORTED;
  if (num_parts < 1 || rows < 0 || heads < 0 || dv < 8 || dv % 8 != 0) return CP_ERR_ARG;
  // dv/8 lanes per (row, head) must tile a 256-lane workgroup
  const int32_t lanes = dv / 8;
  if (lanes > 256 || (lanes & (lanes - 1)) != 0) return CP_ERR_ARG;
  const int64_t pairs = static_cast<int64_t>(rows) * heads;
  if (pairs == 0) return CP_OK;
  if (!o_parts || !lse_parts || !o_out) return CP_ERR_ARG;
  if (!aligned16(o_parts) || !aligned16(o_out)) return CP_ERR_ARG;
  if (o_part_stride < pairs * dv && num_parts > 1) return CP_ERR_ARG;
  if (lse_part_stride < pairs && num_parts > 1) return CP_ERR_ARG;
  if (o_part_stride % 8 != 0 || o_part_stride < 0 || lse_part_stride < 0) return CP_ERR_ARG;
  (void)hipGetLastError();
  hipError_t e = launch_lse_merge(num_parts, pairs, dv, o_parts, part_dtype == CP_BF16,
                                  o_part_stride, lse_parts, lse_part_stride, o_out,
                                  out_dtype == CP_BF16, lse_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CP_OK : device_error(e);
}

extern "C" cp_status cp_calib_mfma(int32_t workgroups, int32_t iters, float *out, void *stream) {
  if (workgroups < 1 || iters < 1 || !out) return CP_ERR_ARG;
  if (iters > (1 << 17)) return CP_ERR_ARG;  // 8 * 16 * iters stays exact in fp32
  (void)hipGetLastError();
  const hipError_t e = launch_calib_mfma(workgroups, iters, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CP_OK : device_error(e);
}

extern "C" cp_status cp_calib_copy(const void *src, void *dst, int64_t bytes, void *stream) {
  if (bytes < 0 || bytes % 16 != 0) return CP_ERR_ARG;
  if (bytes == 0) return CP_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return CP_ERR_ARG;
  if (bytes / 1024 >= INT32_MAX) return CP_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = launch_calib_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CP_OK : device_error(e);
}

extern "C" cp_status cp_restore_apply(const int32_t *index, int64_t n, const void *src,
                                      int64_t src_rows, int64_t src_row_stride, void *dst,
                                      int64_t dst_row_stride, int64_t row_bytes, void *stream) {
  if (n < 0 || src_rows < 0 || row_bytes < 0) return CP_ERR_ARG;
  if (n == 0 || row_bytes == 0) return CP_OK;
  if (!index || !dst || (src_rows > 0 && !src)) return CP_ERR_ARG;
  if (row_bytes % 16 != 0 || src_row_stride % 16 != 0 || dst_row_stride % 16 != 0)
    return CP_ERR_ARG;
  if (src_row_stride < row_bytes || dst_row_stride < row_bytes) return CP_ERR_ARG;
  if (!aligned16(dst) || (src && !aligned16(src))) return CP_ERR_ARG;
  if (row_bytes / 16 > INT32_MAX) return CP_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = launch_restore_apply(index, n, src, src_rows, src_row_stride, dst,
                                            dst_row_stride, row_bytes,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CP_OK : device_error(e);
}

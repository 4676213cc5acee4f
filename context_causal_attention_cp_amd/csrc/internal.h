// Internal launch descriptors shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "cp_attn.h"

namespace cpattn {

// MI355X: 256 compute units in 8 XCDs; consecutive workgroup ids are dealt
// round-robin over the XCDs, each of which has its own L2.
constexpr int kNumXcd = 8;

// Segments per launch travel in the kernel arguments.
constexpr int kMaxLaunchSegs = 64;

// One segment as a kernel sees it.  Tiles of a launch are numbered heaviest
// first: segments in descending kv_len, and inside a segment from its last
// q tile (longest causal extent) to its first.
struct SegDesc {
  int32_t q_begin;     // first local row
  int32_t q_len;       // rows
  int32_t pos_begin;   // position of the first row
  int32_t pos_stride;  // position step per row
  int32_t kv_begin;    // first KV row
  int32_t kv_len;      // KV rows visible at most
  int32_t tile_begin;  // first launch tile number of this segment
  int32_t req;         // request index (paged KV: the block-table row)
  int32_t o_begin;     // output row (O, LSE) of the first row (q_begin unless split)
  int32_t reserved;
};

struct LaunchSegs {
  int32_t num_segs;
  int32_t num_tiles;   // tiles over all segments of this launch
  SegDesc s[kMaxLaunchSegs];
};

struct AttnParams {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  const int32_t *kv_pos;  // null: position = kv row - kv_begin
  int64_t q_rs, q_hs;
  int64_t k_rs, k_hs;
  int64_t v_rs, v_hs;
  int64_t o_rs, o_hs;
  int64_t lse_rs;
  int32_t hq, hkv;
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  int32_t causal;
  int32_t o_bf16;     // 1: o is bf16, 0: fp32
  int32_t accumulate; // 1: merge into the (O, LSE) already in o / lse
  int32_t pack;       // bf16 path: query heads of one KV head per workgroup (1, or 4:
                      // one per wave (pair), the same rows; K/V tiles shared)
  const int32_t *block_table;  // paged KV, or null
  int64_t bt_stride;           // entries per request row
  int32_t block_size;          // rows per block
  int32_t pool_blocks;         // blocks in the k / v pool
  void *ws;           // workspace (device)
  int64_t ws_bytes;
};

// Decode path (MLA-absorbed shape): one workgroup per (query row, KV head,
// block of kDecodeHeadsPerBlock query heads, key slice).  Segments travel in
// the kernel arguments; tile_begin counts work items (q_len * hkv * htiles
// per segment).  Slice partials go to the workspace:
//   ws_o     fp32 [items][nsplit][kDecodeHeadsPerBlock][512]
//   ws_lse   fp32 [items][nsplit][kDecodeHeadsPerBlock]
//   ws_flags int32 [items][nsplit]  (main pass: 1 = recompute in the exact pass)
constexpr int kDecodeHeadsPerBlock = 128;
// paged KV: block ids of one key slice staged in LDS
constexpr int kDecodeMaxSliceBlocks = 1024;

struct DecodeLaunch {
  int32_t num_segs;
  int32_t items;
  int32_t nsplit;
  int32_t htiles;   // ceil(G / kDecodeHeadsPerBlock)
  int32_t hkv;
  int32_t reserved;
  float *ws_o;
  float *ws_lse;
  int32_t *ws_flags;
  SegDesc s[kMaxLaunchSegs];
};

// Records the HIP error for cp_last_error and returns CP_ERR_DEVICE.
cp_status device_error(hipError_t e);

// Kernel entry points (one translation unit each).  They enqueue on
// `stream` and return the launch status.
hipError_t launch_attn_bf16(const AttnParams &p, const LaunchSegs &L, int dqk, int dv,
                            int tile_rows, hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams &p, const LaunchSegs &L, int d,
                           hipStream_t stream);
hipError_t launch_attn_decode_mla(const AttnParams &p, const DecodeLaunch &D,
                                  hipStream_t stream);
// query rows per bf16 workgroup: 256, or 128 for calls too small to give
// every compute unit two workgroups with 256-row tiles
int attn_bf16_tile_rows(int dqk, int dv, bool small);
int attn_f32_tile_rows(int d);

hipError_t launch_calib_mfma(int32_t workgroups, int32_t iters, float *out, hipStream_t stream);
hipError_t launch_calib_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);
hipError_t launch_restore_apply(const int32_t *index, int64_t n, const void *src, int64_t src_rows,
                                int64_t src_stride, void *dst, int64_t dst_stride,
                                int64_t row_bytes, hipStream_t stream);

// Several independent LSE merges in one launch (the key-split segments of an
// attention call).  Segment i: `parts[i]` partials of `pairs[i]` (row, head)
// pairs; partial j of its pair x at pair index j * part_stride + src[i] + x
// of the partial buffers, its output at pair index dst[i] + x; it owns
// workgroups wg_begin[i] .. wg_begin[i + 1] - 1, one per
// lse_merge_pairs_per_workgroup(dv) pairs.
constexpr int kMaxMergeSegs = 64;
struct MergeSegs {
  int32_t n;
  int32_t wg_begin[kMaxMergeSegs + 1];
  int32_t parts[kMaxMergeSegs];
  int64_t pairs[kMaxMergeSegs];
  int64_t src[kMaxMergeSegs];
  int64_t dst[kMaxMergeSegs];
};
int lse_merge_pairs_per_workgroup(int32_t dv);
hipError_t launch_lse_merge_segs(const MergeSegs &T, int32_t dv, const void *o_parts,
                                 int part_bf16, int64_t part_stride, const float *lse_parts,
                                 void *o_out, int out_bf16, float *lse_out, hipStream_t stream);
hipError_t launch_lse_merge(int32_t parts, int64_t pairs, int32_t dv,
                            const void *o_parts, int part_bf16,
                            int64_t o_part_stride, const float *lse_parts,
                            int64_t lse_part_stride, void *o_out, int out_bf16,
                            float *lse_out, hipStream_t stream);

}  // namespace cpattn

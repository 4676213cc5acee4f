// Decode-CP shard attention for the MLA-absorbed shape on gfx950.
//
// "What is Context Parallelism" (blog): section 2.2 -- decode is a
// memory-bound scan of a large KV cache; the cache is sharded along the
// sequence (token i on shard i mod W) and the small Q is brought to every
// shard (section 3.3); each shard returns its normalised partial output and
// log-sum-exp for an LSE merge (section 3.6).  Section 4.2 -- with the
// absorbed MLA form every query head attends directly to the shared latent
// row: K = [c_KV (512) | k_pe (64)], and V is the first 512 columns of the
// same row.
//
// One workgroup (8 waves, two per SIMD) computes, for one query row and 128
// query heads of one KV head, the partial attention over one contiguous
// slice of the shard's keys, in tiles of 32 latent rows (36 KiB) copied
// HBM -> LDS by buffer loads straight into LDS (no register staging):
//   * main pass (attn_decode_rs_kernel), with split roles: waves 0-3 hold Q
//     of 32 heads each, compute S^T = K Q^T and write the softmax numerators
//     P to LDS; after the tile's barrier every wave multiplies all 128
//     heads' P by its own columns of V^T, read from the same row-major tile
//     with the transposing ds_read_b64_tr_b16 (each latent row crosses HBM
//     once and sits in LDS once).  Every head's softmax reference is fixed
//     at its first tile; a slice whose row sums outgrow 2^64 (or whose
//     accumulators are not finite) is flagged;
//   * exact pass (attn_decode_mla_kernel): recomputes only the flagged
//     slices, each wave with 16 heads' whole 512 x 16 O^T and a reference
//     that moves (with a rescale) when a tile outgrows it by 2^8;
//   * the tiles are XOR-swizzled in 16-byte chunks so that the row reads and
//     the transposing reads are free of bank conflicts under gfx950's lane
//     grouping of 16- and 8-byte LDS reads;
// and writes the slice's normalised partial (O_s, LSE_s) to the workspace.
//
// Paged KV (the cache of a rank that holds whole blocks of tokens, section
// 2.2's block interleave): a 32-row tile never crosses a block (blocks are
// multiples of 32 rows and segments start on a tile), so each tile gets its
// own buffer resource at its block's pool row and the per-lane offsets stay
// those of a contiguous tile (the main pass reads the tile's block id from
// the table; the exact pass stages the slice's ids in LDS once).
// A third kernel merges the slices of each (row, head) by LSE.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 8;                    // waves
constexpr int NT = 64 * NW;              // threads
constexpr int HW = 16;                   // heads per wave
constexpr int HT = kDecodeHeadsPerBlock; // heads per workgroup
static_assert(HT == HW * NW, "heads per workgroup");
constexpr int BN = 32;                   // keys per tile
constexpr int DQK = 576, DV = 512;
constexpr int KCH = DQK / 8;             // 16-byte chunks per latent row
constexpr int TILE_CH = BN * KCH;        // 2304 chunks = 36 KiB
constexpr int TILE_WI = TILE_CH / 64;    // 36 wave-instructions of LDS DMA per tile
constexpr int NBUF = 3;
constexpr int QS = DQK / 32;             // MFMA k-steps for S (18)
constexpr int OB = DV / 16;              // 16-row dv blocks of O^T (32)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescale = 8.0f;         // log2 headroom before the reference max moves
static_assert(TILE_WI == 36, "DMA split below assumes 36 instructions per tile");

// XOR swizzle of the 16-byte chunk index within a latent row; it stays in
// its aligned group of 8 chunks (72 is a multiple of 8).  With key bits
// k0..k2: f = k0 | (k0^k1)<<1 | (k0^k2)<<2.
// gfx950 serves a ds_read_b128 16 lanes at a time over a 256-byte bank row,
// in the lane groups {0-3, 12-15, 20-23, 24-27} and {4-11, 16-19, 28-31}
// (and the same +32); a row is 1152 bytes, so a key's parity picks the half
// of the bank row.  In the row reads a group holds the 16 keys of one block,
// keys 0-3 and 12-15 at chunk c and keys 4-11 at chunk c+1 (or the
// reverse): the chunk step flips bit 0 exactly for k2^k3 = 1, so bit 0 of f
// must not hold k2 or k3 (an earlier k0^k3 made the row reads 2-way
// conflicted).  ds_read_b64(_tr) serves 32 lanes at a time; the
// transposing reads cover 8 keys x 2 chunks per half-wave, which bits 1-2
// of f spread over the bank row.
__device__ inline int swz(int key) {
  const int k0 = key & 1, k1 = (key >> 1) & 1, k2 = (key >> 2) & 1;
  return k0 | ((k0 ^ k1) << 1) | ((k0 ^ k2) << 2);
}

// two floats -> packed bf16 (round to nearest even), one v_cvt_pk_bf16_f32
__device__ inline uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// max / sum over the four 16-lane groups that hold the same head
__device__ inline float max_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ inline float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

// ds_read_b64_tr_b16 through inline asm.  The intrinsic makes the waitcnt pass
// assume it may alias the LDS-DMA writes still in flight and drain them
// (vmcnt(0)) before every use; the tile it reads was already completed by
// an explicit vmcnt wait and a barrier.  The compiler does not count these
// reads, so their results are consumed only after an explicit lgkmcnt wait
// that takes the result registers as operands (the data dependency keeps
// the consumers after it).
__device__ inline u32x2 lds_read_tr16(const void *p) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1"
               : "=v"(r)
               : "v"((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p));
  return r;
}
// The four reads in r are complete once at most 4 LDS operations issued
// after them are pending: LDS operations complete in issue order, so while
// one of r is pending all later ones are too.  (Operations the compiler adds
// in between only make the wait stricter.)
__device__ inline void lds_wait4_later(u32x2 (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
}
__device__ inline void lds_wait0(u32x2 (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
}

// vmcnt wait with the other counters left alone (gfx9 encoding)
template <int N>
__device__ inline void wait_vm() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ inline void decode_item(const DecodeLaunch &D, int item, int &si, int &row, int &kvh,
                                   int &ht) {
  si = 0;
  for (int i = 1; i < D.num_segs; ++i)
    if (item >= D.s[i].tile_begin) si = i;
  int rem = item - D.s[si].tile_begin;
  ht = rem % D.htiles;
  rem /= D.htiles;
  kvh = rem % D.hkv;
  row = rem / D.hkv;
}

// The exact pass: recomputes the slices the main pass (attn_decode_rs_kernel)
// flagged, with a per-head reference max that moves (and rescales the
// accumulator) whenever a tile outgrows it by more than 2^8.  Each wave keeps
// 16 heads' Q and their whole 512 x 16 O^T, so no state crosses waves.
// Unflagged workgroups read their flag and leave (a few microseconds per
// call; folding this pass into the main kernel made the compiler spill).
template <bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void attn_decode_mla_kernel(const AttnParams p, const DecodeLaunch D) {
  if (D.ws_flags[blockIdx.x] == 0) return;  // the main pass wrote this slice
  // key tiles, then (paged) the slice's block ids, in ONE LDS object: with a
  // second LDS variable the waitcnt pass can no longer tell the tile reads
  // from the in-flight LDS-DMA writes and drains them (vmcnt(0)) every tile
  constexpr int TBL = PAGED ? kDecodeMaxSliceBlocks / 4 : 0;
  __shared__ __attribute__((aligned(1024))) u32x4 lds[NBUF * TILE_CH + TBL];
  u32x4(*sk)[TILE_CH] = reinterpret_cast<u32x4(*)[TILE_CH]>(lds);
  int32_t *s_blk = reinterpret_cast<int32_t *>(lds + NBUF * TILE_CH);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int item = blockIdx.x / D.nsplit, split = blockIdx.x % D.nsplit;
  if (item >= D.items) return;
  int si, row, kvh, ht;
  decode_item(D, item, si, row, kvh, ht);
  const SegDesc sd = D.s[si];
  const int G = p.hq / p.hkv;
  const int hl = ht * HT + w * HW + n;           // head within the KV group
  const bool hvalid = hl < G;
  const int h = kvh * G + hl;
  const int64_t qrow = (int64_t)sd.q_begin + row;
  const int qpos = sd.pos_begin + row * sd.pos_stride;

  // this workgroup's key slice
  const int chunk = ((sd.kv_len + D.nsplit - 1) / D.nsplit + BN - 1) / BN * BN;
  const int k_lo = min(sd.kv_len, split * chunk);
  const int k_hi = min(sd.kv_len, k_lo + chunk);
  // paged: kv_pos is indexed by the request's logical rows
  const int64_t pos_base =
      PAGED ? (int64_t)sd.req * p.bt_stride * p.block_size + sd.kv_begin : (int64_t)sd.kv_begin;
  const int32_t *kvp = p.kv_pos ? p.kv_pos + pos_base : nullptr;
  auto key_pos = [&](int j) -> int { return kvp ? kvp[j] : j; };
  // keys past the query's position end the slice early (positions increase)
  int k_vis = k_hi;
  if (p.causal && k_hi > k_lo && key_pos(k_hi - 1) > qpos) {
    int lo = k_lo, hi = k_hi;  // first key with position > qpos
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (key_pos(mid) <= qpos) lo = mid + 1; else hi = mid;
    }
    k_vis = lo;
  }
  const int ntiles = (k_vis - k_lo + BN - 1) / BN;

  // Q fragments: B operand of S^T = K Q^T (n = head, k = d: 8 per lane group)
  bf16x8 qf[QS];
  {
    const __bf16 *qp = (const __bf16 *)p.q + qrow * p.q_rs + (int64_t)h * p.q_hs + 8 * g;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (hvalid) x = *(const u32x4 *)(qp + 32 * s);
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // LDS DMA: waves 0-3 issue 5 and waves 4-7 issue 4 of the 36 instructions
  const __bf16 *kbase = (const __bf16 *)p.k + (int64_t)sd.kv_begin * p.k_rs + (int64_t)kvh * p.k_hs;
  const int wi0 = w < 4 ? 5 * w : 20 + 4 * (w - 4);
  const int wn = w < 4 ? 5 : 4;
  // LDS DMA goes through a buffer resource that ends at the slice end: rows
  // past k_hi read as zeros (hardware range check), so the last tile needs no
  // clamping.  Per-lane byte offsets are relative to the tile's first row.
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)kbase, (short)0, (int)((int64_t)k_hi * p.k_rs * 2), 0x00020000);
  // paged: the slice's block ids (clamped into the pool) -> LDS
  const int x_lo = sd.kv_begin + k_lo;  // first logical row of the slice
  const int blk0 = x_lo / p.block_size;
  if (PAGED) {
    if (k_vis > k_lo) {
      const int nblk = (sd.kv_begin + k_vis - 1) / p.block_size - blk0 + 1;
      const int32_t *bt = p.block_table + (int64_t)sd.req * p.bt_stride + blk0;
      for (int i = tid; i < nblk; i += NT) s_blk[i] = min(max(bt[i], 0), p.pool_blocks - 1);
    }
    __syncthreads();
  }
  auto tile_rsrc = [&](int t, uint32_t &row0) -> __amdgpu_buffer_rsrc_t {
    if (!PAGED) {
      row0 = (uint32_t)((k_lo + t * BN) * p.k_rs) * 2u;
      return krsrc;
    }
    // the tile's 32 rows sit in one block; rows past the slice read zero
    const int x0 = x_lo + t * BN;
    const int b = __builtin_amdgcn_readfirstlane(s_blk[x0 / p.block_size - blk0]);
    const int64_t prow = (int64_t)b * p.block_size + x0 % p.block_size;
    const int rows = min(BN, k_hi - (k_lo + t * BN));
    row0 = 0u;
    return __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const __bf16 *)p.k + prow * p.k_rs + (int64_t)kvh * p.k_hs), (short)0,
        (int)(rows * p.k_rs * 2), 0x00020000);
  };
  // per-lane DMA byte offsets inside a tile, computed once (5 registers;
  // recomputing them every tile cost 3 % of the shard time)
  uint32_t dma_off[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int slot = (wi0 + i) * 64 + lane;
    const int key = slot / KCH, cs = slot % KCH;
    dma_off[i] = (uint32_t)(key * p.k_rs + (cs ^ swz(key)) * 8) * 2u;
  }
  auto issue = [&](int t) {
    uint32_t row0;
    const __amdgpu_buffer_rsrc_t trsrc = tile_rsrc(t, row0);
    u32x4 *dst = sk[t % NBUF];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      if (i < wn) {
        const uint32_t off = dma_off[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            trsrc, (__attribute__((address_space(3))) void *)(dst + (wi0 + i) * 64), 16,
            row0 + off, 0, 0, 0);
      }
    }
  };

  f32x4 oacc[OB];
#pragma unroll
  for (int b = 0; b < OB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[b][i] = 0.f;
  float m_ref = -INFINITY;  // reference max of this lane's head (log2 units)
  float l_run = 0.f;        // this lane's partial row sum
  const float sl2 = p.scale_log2;

  // Per-lane LDS byte offsets.  The swizzle only touches the low 3 bits of
  // the chunk index, so every read below is one of a few per-lane bases plus
  // a compile-time offset (128 bytes per group of 8 chunks).
  //  row reads (QK): key 16*mb + n, chunk 4*st + g = 8*(st>>1) + (4*(st&1) + g).
  //  The swizzle only depends on key bits 0..3, so key + 16 is the same read
  //  shifted by 16 rows (kRow16 bytes).
  constexpr int kRow16 = 16 * KCH * 16;
  //  transposing reads (PV): lane li of group g addresses key 4g + li/4 (+16),
  //  dv 16*b + 4*(li%4): chunk 2*b + (li%4)/2 = 8*(b>>2) + (2*(b&3) + (li%4)/2),
  //  byte 8*(li&1) inside the chunk.
  //  The bases are rebuilt every tile from an opaque copy of the lane id (a
  //  few integer ops) rather than kept live across the loop.
  auto lds_bases = [&](int (&qk_base)[2], int (&tr_base)[4]) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int nn = ln & 15, gg = ln >> 4;
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) qk_base[odd] = 16 * (nn * KCH + ((4 * odd + gg) ^ swz(nn)));
    const int key = 4 * gg + (nn >> 2);
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4)
      tr_base[b4] = 16 * (key * KCH + ((2 * b4 + ((nn & 3) >> 1)) ^ swz(key))) + 8 * (nn & 1);
  };

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      if (w < 4) wait_vm<5>(); else wait_vm<4>();
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (t + 2 < ntiles) issue(t + 2);
    const char *tile = (const char *)sk[t % NBUF];
    const int j0 = k_lo + t * BN;
    int qk_base[2], tr_base[4];
    lds_bases(qk_base, tr_base);

    // ---- S^T = K Q^T : two 16-key blocks x 16 heads
    f32x4 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[mb][i] = 0.f;
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        const bf16x8 a =
            *(const bf16x8 *)(tile + qk_base[st & 1] + kRow16 * mb + 128 * (st >> 1));
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[st], s[mb], 0, 0, 0);
      }
    }
    // Three row reads in flight ahead of the MFMA that consumes them.  Left
    // to itself the scheduler keeps one or two, and in the paged variant
    // (a few more live scalars) only one: every MFMA then waits out a full
    // LDS latency, which made the paged shard 25 % slower than the
    // contiguous one.
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // 3 LDS reads
#pragma unroll
    for (int i = 0; i < 2 * QS - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);  // last 3 MFMAs
    // ---- mask (keys at or past k_vis are after the query or past the
    // slice; positions increase), lane-local max
    const bool full = j0 + BN <= k_vis;
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float u = s[mb][i] * sl2;
        if (!full) u = (j0 + 16 * mb + 4 * g + i < k_vis) ? u : -INFINITY;
        s[mb][i] = u;
        mx = fmaxf(mx, u);
      }
    // move the reference (wave-wide, rare) only if some lane outgrew it by > 2^8
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescale) != 0) {
      const float m_new = fmaxf(m_ref, max_groups(mx));
      const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < OB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[b][i] *= alpha;
      m_ref = m_new;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    // P as the B operand: element e <-> key (e<4 ? 4g+e : 16+4g+e-4)
    u32x4 pk;
    float ls = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float p0 = __builtin_amdgcn_exp2f(s[mb][0] - m_use), p1 = __builtin_amdgcn_exp2f(s[mb][1] - m_use);
      const float p2 = __builtin_amdgcn_exp2f(s[mb][2] - m_use), p3 = __builtin_amdgcn_exp2f(s[mb][3] - m_use);
      ls += (p0 + p1) + (p2 + p3);
      pk[2 * mb] = pack_bf16(p0, p1);
      pk[2 * mb + 1] = pack_bf16(p2, p3);
    }
    l_run += ls;
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
    // ---- O^T += V^T P^T : V^T from the same tile by transposing reads, in
    // batches of 2 dv blocks, double-buffered: batch i + 1's reads are issued
    // before the wait for batch i, so the reads of one batch run under the
    // MFMAs of the previous one (4.7 % faster than batches of 4 with a full
    // drain; deeper pipelines measured slower)
    constexpr int PB = 2, NBT = OB / PB;
    u32x2 vb[2][2 * PB];
    auto pv_issue = [&](int bi, u32x2 (&r)[2 * PB]) {
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const int b = bi * PB + j;
        r[2 * j] = lds_read_tr16(tile + tr_base[b & 3] + 128 * (b >> 2));
        r[2 * j + 1] = lds_read_tr16(tile + tr_base[b & 3] + kRow16 + 128 * (b >> 2));
      }
    };
    pv_issue(0, vb[0]);
#pragma unroll
    for (int bi = 0; bi < NBT; ++bi) {
      u32x2 (&cur)[2 * PB] = vb[bi & 1];
      if (bi + 1 < NBT) {
        pv_issue(bi + 1, vb[(bi + 1) & 1]);
        lds_wait4_later(cur);
      } else {
        lds_wait0(cur);
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const u32x4 av = {cur[2 * j][0], cur[2 * j][1], cur[2 * j + 1][0], cur[2 * j + 1][1]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, av);
        oacc[bi * PB + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[bi * PB + j], 0, 0, 0);
      }
    }
  }

  // ---- normalised partial of this slice -> workspace
  const float l_tot = sum_groups(l_run);
  if (!hvalid) return;
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const int64_t part = (int64_t)item * D.nsplit + split;
  const int hb = w * HW + n;
  float *wo = D.ws_o + (part * HT + hb) * DV + 4 * g;
  if (g == 0) D.ws_lse[part * HT + hb] = any ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
#pragma unroll
  for (int b = 0; b < OB; ++b)
    *(float4 *)(wo + 16 * b) =
        make_float4(oacc[b][0] * inv, oacc[b][1] * inv, oacc[b][2] * inv, oacc[b][3] * inv);
}

// Main pass (attn_decode_rs_kernel) LDS: four tile stages and two P
// buffers.  P units are 16 bytes: unit (g * 128 + head) holds the eight
// numerators of `head` that lane group g of an MFMA operand carries (keys
// 4g..4g+3 and 16+4g..16+4g+3), so the S owner writes its lane's eight at
// once, and a 16-lane run of a reader covers 16 consecutive units (one
// 256-byte bank row), free of bank conflicts under gfx950's lane groups.
constexpr int NBUF_X = 4;                   // main pass: LDS stages
constexpr int PB_UNITS = 4 * HT;            // one P buffer, 16-byte units (8 KiB)
constexpr int HBK = HT / 16;                // 16-head blocks (8)
constexpr float kMaxSum = 18446744073709551616.0f;  // 2^64: largest accepted row sum
static_assert((NBUF_X * TILE_CH + 2 * PB_UNITS) * 16 <= 160 * 1024, "LDS");

// x, hidden from the optimiser (keeps per-lane values that are cheap to
// rebuild from being hoisted and kept live across the loop).  A __device__
// function: inline asm with a VGPR constraint inside a kernel's lambda is
// also checked for the host, where the constraint does not exist, and the
// kernel's host-side launch stub then silently disappears.
__device__ inline int opaque_lane(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// byte offset of lane ln's 16-byte chunk in DMA instruction wi of a tile
// (rows k_rs elements apart, chunks swizzled as in the LDS tile)
__device__ inline uint32_t dma_lane_offset(int wi, int ln, int k_rs) {
  const int slot = wi * 64 + ln;
  const int key = slot / KCH, cs = slot % KCH;
  return (uint32_t)(key * k_rs + (cs ^ swz(key)) * 8) * 2u;
}

__device__ inline uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
// vmcnt(N) and lgkmcnt(0) in one wait (gfx9 encoding)
template <int N>
__device__ inline void wait_vm_lgkm0() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// ---------------------------------------------------------------------------
// Main pass with split roles (attn_decode_rs_kernel).  Waves 0-3 ("score
// waves") each hold Q of 32 heads, so every K fragment they read from LDS
// feeds two products and the K tile is read 4 times per tile (with 16 heads
// per wave, 8 times: 288 of ~428 KiB of LDS traffic per tile, which bound an
// earlier P-exchange pass); waves 4-7 ("output waves") only multiply and copy.
// The softmax numerators P go through LDS: after the tile's barrier every
// wave multiplies all 128 heads' P by its own columns of V^T.  Score wave s
// and output wave s + 4 share a SIMD and together own the 128 columns
// [128 s, 128 s + 128) of O^T: the score wave 32 of them (beside its 144
// registers of Q), the output wave 96.  The output waves copy the tiles
// (rows 8 s'..8 s' + 7 of each tile for output wave s').  Per tile and CU:
// 144 KiB of K reads, 8 KiB of P written and 64 KiB read, 32 KiB of V^T and
// the 36 KiB copy, about 284 KiB.
//   * one barrier per tile: iteration t runs S of tile t (score waves) and
//     PV of tile t - 1 (all waves); the score waves multiply after writing
//     P(t), the output waves after issuing the copy of tile t + 2 (both
//     orders measured faster than the reverse); four stages and two P
//     buffers (160 KiB); all waves at the same priority;
//   * every head's softmax reference is the max over the first 16 keys of
//     its first tile (the first key of the slice is always visible) and
//     never moves; a slice whose row sums outgrow 2^64 or whose accumulators
//     are not finite is flagged (one int32 per workgroup in the workspace)
//     and recomputed by the exact pass (attn_decode_mla_kernel);
//   * every LDS access in the loops is inline asm with its wait tied to the
//     registers it fills (compiler-visible LDS reads there can make the
//     wait-count pass drain the copies in flight).
constexpr int RS_SDB = 2;                 // 16-column dv blocks of O^T per score wave
constexpr int RS_ODB = 8 - RS_SDB;        // per output wave (a SIMD owns 8 blocks)
constexpr int RS_KLA = 3;                 // K fragment reads in flight in S
constexpr int RS_DMA = TILE_WI / 4;       // copy instructions per output wave and tile
static_assert(TILE_WI % 4 == 0 && RS_DMA * 64 == 8 * KCH, "an output wave copies 8 rows");
static_assert(4 * 8 * 16 == DV, "four SIMDs x 8 blocks of 16 columns");

template <int OFF>
__device__ inline u32x4 ds_read_b128_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ inline u32x2 ds_read_tr16_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ inline void ds_write_b128_at(uint32_t addr, const u32x4 &v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF) : "memory");
}
// x is complete once at most LATER LDS operations issued after it are pending
// (LDS operations complete in issue order)
template <int LATER, typename T>
__device__ inline void lgkm_tie(T &x) {
  static_assert(LATER >= 0 && LATER < 16, "lgkmcnt");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(LATER));
}
template <int LATER>
__device__ inline void lgkm_tie2(u32x2 (&v)[2]) {
  static_assert(LATER >= 0 && LATER < 16, "lgkmcnt");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v[0]), "+v"(v[1]) : "i"(LATER));
}
__device__ inline void lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// K fragment of S step U: key block U / QS, k-step U % QS (two per-lane bases
// for even and odd k-steps, as lds_bases builds them)
template <int U>
__device__ inline bf16x8 rs_kread(uint32_t kb0, uint32_t kb1) {
  constexpr int MB = U / QS, ST = U % QS;
  constexpr int OFF = 16 * KCH * 16 * MB + 128 * (ST >> 1);
  return __builtin_bit_cast(bf16x8, ds_read_b128_at<OFF>((ST & 1) ? kb1 : kb0));
}
template <int U>
__device__ inline void rs_kfirst(uint32_t kb0, uint32_t kb1, bf16x8 (&kf)[RS_KLA]) {
  if constexpr (U < RS_KLA) {
    kf[U] = rs_kread<U>(kb0, kb1);
    rs_kfirst<U + 1>(kb0, kb1, kf);
  }
}
// S^T = K Q^T of one tile for the score wave's two head blocks, step U
// onwards (key block 0's 18 steps, then key block 1's); mid() runs after key
// block 0's last products
template <int U, typename F>
__device__ inline void rs_qk(uint32_t kb0, uint32_t kb1, bf16x8 (&kf)[RS_KLA],
                             const bf16x8 (&qf)[2][QS], f32x4 (&sc)[2][2], F &&mid) {
  if constexpr (U < 2 * QS) {
    constexpr int MB = U / QS, ST = U % QS;
    constexpr int LATER = (2 * QS - 1 - U) < (RS_KLA - 1) ? (2 * QS - 1 - U) : (RS_KLA - 1);
    lgkm_tie<LATER>(kf[U % RS_KLA]);
    const bf16x8 a = kf[U % RS_KLA];
    if constexpr (U + RS_KLA < 2 * QS) kf[U % RS_KLA] = rs_kread<U + RS_KLA>(kb0, kb1);
    sc[MB][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][ST], sc[MB][0], 0, 0, 0);
    sc[MB][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][ST], sc[MB][1], 0, 0, 0);
    if constexpr (U == QS - 1) mid();
    rs_qk<U + 1>(kb0, kb1, kf, qf, sc, mid);
  }
}

// V^T fragment of this SIMD's dv block B (0..7) for keys 4g.. and 16 + 4g..
// (ta: the stage's address plus the SIMD's 256 bytes; trb: lds_bases)
template <int B>
__device__ inline void rs_vread(uint32_t ta, const int (&trb)[4], u32x2 (&v)[2]) {
  constexpr int OFF = 128 * (B >> 2);
  v[0] = ds_read_tr16_at<OFF>(ta + trb[B & 3]);
  v[1] = ds_read_tr16_at<OFF + 16 * KCH * 16>(ta + trb[B & 3]);
}
__device__ inline bf16x8 rs_vfrag(const u32x2 (&v)[2]) {
  const u32x4 av = {v[0][0], v[0][1], v[1][0], v[1][1]};
  return __builtin_bit_cast(bf16x8, av);
}

// Score wave's PV: its two dv blocks (both read first), P streamed one head
// block at a time, three reads ahead (registers: Q and S are its bulk)
template <int HB>
__device__ inline void rs_pv_score_step(uint32_t pa, u32x4 (&pr)[3], const bf16x8 (&va)[2],
                                        f32x4 (&oacc)[HBK][RS_SDB]) {
  if constexpr (HB < HBK) {
    constexpr int LATER = (HBK - 1 - HB) < 2 ? (HBK - 1 - HB) : 2;
    lgkm_tie<LATER>(pr[HB % 3]);
    const bf16x8 b = __builtin_bit_cast(bf16x8, pr[HB % 3]);
    if constexpr (HB + 3 < HBK) pr[HB % 3] = ds_read_b128_at<256 * (HB + 3)>(pa);
    oacc[HB][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[0], b, oacc[HB][0], 0, 0, 0);
    oacc[HB][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[1], b, oacc[HB][1], 0, 0, 0);
    rs_pv_score_step<HB + 1>(pa, pr, va, oacc);
  }
}
__device__ inline void rs_pv_score(uint32_t ta, uint32_t pa, const int (&trb)[4],
                                   f32x4 (&oacc)[HBK][RS_SDB]) {
  u32x2 v0[2], v1[2];
  rs_vread<0>(ta, trb, v0);
  rs_vread<1>(ta, trb, v1);
  u32x4 pr[3];
  pr[0] = ds_read_b128_at<0>(pa);
  pr[1] = ds_read_b128_at<256>(pa);
  pr[2] = ds_read_b128_at<512>(pa);
  lgkm_tie2<3>(v0);
  lgkm_tie2<3>(v1);
  const bf16x8 va[2] = {rs_vfrag(v0), rs_vfrag(v1)};
  rs_pv_score_step<0>(pa, pr, va, oacc);
}

// Output wave's PV: all eight P reads first, then its six dv blocks (2..7)
// stream one block ahead of their eight products each
template <int J>
__device__ inline void rs_pv_out_step(uint32_t ta, const int (&trb)[4], const u32x4 (&pr)[HBK],
                                      u32x2 (&vr)[2][2], f32x4 (&oacc)[HBK][RS_ODB]) {
  if constexpr (J < RS_ODB) {
    u32x2 (&cur)[2] = vr[J & 1];
    if constexpr (J + 1 < RS_ODB) {
      lgkm_tie2<2>(cur);
    } else {
      lgkm_tie2<0>(cur);
    }
    const bf16x8 a = rs_vfrag(cur);
#pragma unroll
    for (int hb = 0; hb < HBK; ++hb)
      oacc[hb][J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, pr[hb]),
                                                            oacc[hb][J], 0, 0, 0);
    if constexpr (J + 2 < RS_ODB) rs_vread<RS_SDB + J + 2>(ta, trb, cur);
    rs_pv_out_step<J + 1>(ta, trb, pr, vr, oacc);
  }
}
__device__ inline void rs_pv_out(uint32_t ta, uint32_t pa, const int (&trb)[4],
                                 f32x4 (&oacc)[HBK][RS_ODB]) {
  u32x4 pr[HBK];
#pragma unroll
  for (int hb = 0; hb < HBK; ++hb) pr[hb] = ds_read_b128_at<0>(pa + 256 * hb);
  u32x2 vr[2][2];
  rs_vread<RS_SDB>(ta, trb, vr[0]);
  rs_vread<RS_SDB + 1>(ta, trb, vr[1]);
  // the P reads and block 0's two are complete (block 1's two may pend)
  asm volatile("s_waitcnt lgkmcnt(2)"
               : "+v"(pr[0]), "+v"(pr[1]), "+v"(pr[2]), "+v"(pr[3]), "+v"(pr[4]), "+v"(pr[5]),
                 "+v"(pr[6]), "+v"(pr[7]), "+v"(vr[0][0]), "+v"(vr[0][1]));
  rs_pv_out_step<0>(ta, trb, pr, vr, oacc);
}

template <bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
void attn_decode_rs_kernel(const AttnParams p, const DecodeLaunch D) {
  __shared__ __attribute__((aligned(1024))) u32x4 lds[NBUF_X * TILE_CH + 2 * PB_UNITS];
  char *const pbuf = (char *)(lds + NBUF_X * TILE_CH);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const bool score = w < 4;
  const int s = w & 3;  // the SIMD: heads 32 s.. (score), columns 128 s.. (both)
  const int lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int item = blockIdx.x / D.nsplit, split = blockIdx.x % D.nsplit;
  if (item >= D.items) return;
  int si, row, kvh, ht;
  decode_item(D, item, si, row, kvh, ht);
  const SegDesc sd = D.s[si];
  const int G = p.hq / p.hkv;
  const int64_t qrow = (int64_t)sd.q_begin + row;
  const int qpos = sd.pos_begin + row * sd.pos_stride;

  // this workgroup's key slice (as in the exact pass)
  const int chunk = ((sd.kv_len + D.nsplit - 1) / D.nsplit + BN - 1) / BN * BN;
  const int k_lo = min(sd.kv_len, split * chunk);
  const int k_hi = min(sd.kv_len, k_lo + chunk);
  const int64_t pos_base =
      PAGED ? (int64_t)sd.req * p.bt_stride * p.block_size + sd.kv_begin : (int64_t)sd.kv_begin;
  const int32_t *kvp = p.kv_pos ? p.kv_pos + pos_base : nullptr;
  auto key_pos = [&](int j) -> int { return kvp ? kvp[j] : j; };
  int k_vis = k_hi;
  if (p.causal && k_hi > k_lo && key_pos(k_hi - 1) > qpos) {
    int lo = k_lo, hi = k_hi;  // first key with position > qpos
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (key_pos(mid) <= qpos) lo = mid + 1; else hi = mid;
    }
    k_vis = lo;
  }
  const int ntiles = (k_vis - k_lo + BN - 1) / BN;

  const uint32_t lds0 = lds_addr(lds);
  auto stage_addr = [&](int t) -> uint32_t {
    return lds0 + (uint32_t)((t % NBUF_X) * TILE_CH * 16);
  };
  // P unit of this lane as a reader (head block 0; +256 bytes per block)
  auto p_read_addr = [&](int u) -> uint32_t {
    const int ln = opaque_lane(lane);
    return lds_addr(pbuf) + (uint32_t)((u & 1) * PB_UNITS * 16) +
           (uint32_t)((((ln >> 4) * HT) + (ln & 15)) * 16);
  };
  auto tr_bases = [&](int (&trb)[4]) {
    const int ln = opaque_lane(lane);
    const int nn = ln & 15, gg = ln >> 4;
    const int key = 4 * gg + (nn >> 2);
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4)
      trb[b4] = 16 * (key * KCH + ((2 * b4 + ((nn & 3) >> 1)) ^ swz(key))) + 8 * (nn & 1);
  };

  float l_tot[2] = {0.f, 0.f};  // score waves: row sums of the lane's two heads
  float m_ref[2] = {0.f, 0.f};  // and their references (log2 units)
  bool bad = false;
  const int64_t part = (int64_t)item * D.nsplit + split;
  int flagged = 0;

  if (score) {
    // ---- score wave: S, the numerators of heads 32 s + 16 hb + n, PV of
    // columns [128 s, 128 s + 32)
    bf16x8 qf[2][QS];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int hl = ht * HT + 32 * s + 16 * hb + n;
      const bool hvalid = hl < G;
      const __bf16 *qp = (const __bf16 *)p.q + qrow * p.q_rs + (int64_t)(kvh * G + hl) * p.q_hs + 8 * g;
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (hvalid && ntiles > 0) x = *(const u32x4 *)(qp + 32 * st);
        qf[hb][st] = __builtin_bit_cast(bf16x8, x);
      }
    }
    f32x4 oacc[HBK][RS_SDB];
#pragma unroll
    for (int hb = 0; hb < HBK; ++hb)
#pragma unroll
      for (int j = 0; j < RS_SDB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[hb][j][i] = 0.f;
    float l_run[2] = {0.f, 0.f};
    const float sl2 = p.scale_log2;
    auto pv = [&](int u) {
      int trb[4];
      tr_bases(trb);
      rs_pv_score(stage_addr(u) + 256u * (uint32_t)s, p_read_addr(u), trb, oacc);
    };
    // K row bases of this lane for even and odd k-steps (kept across the loop)
    const uint32_t kl0 = (uint32_t)(16 * (n * KCH + (g ^ swz(n))));
    const uint32_t kl1 = (uint32_t)(16 * (n * KCH + ((4 + g) ^ swz(n))));
    for (int t = 0; t < ntiles; ++t) {
      lgkm0();  // this wave's P(t - 1) is written
      __builtin_amdgcn_s_barrier();
      const int j0 = k_lo + t * BN;
      const bool full = j0 + BN <= k_vis;
      // K row bases of this lane for even and odd k-steps
      const uint32_t kb0 = stage_addr(t) + kl0, kb1 = stage_addr(t) + kl1;
      f32x4 sc[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[mb][hb][i] = 0.f;
      u32x4 pk[2];
      // numerators of key block mb against the fixed references: P-unit
      // elements 4 mb .. 4 mb + 3 (keys 16 mb + 4g + i)
      auto numer = [&](int mb) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          if (mb == 0 && t == 0) {  // the slice's first key is visible
            float u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              u[i] = sc[mb][hb][i] * sl2;
              if (!full) u[i] = (j0 + 16 * mb + 4 * g + i < k_vis) ? u[i] : -INFINITY;
            }
            m_ref[hb] = max_groups(fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3])));
          }
          // scaled score minus the reference in one rounding
          const float nm = -m_ref[hb];
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = fmaf(sc[mb][hb][i], sl2, nm);
          if (!full) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              x[i] = (j0 + 16 * mb + 4 * g + i < k_vis) ? x[i] : -INFINITY;
          }
          const float p0 = __builtin_amdgcn_exp2f(x[0]);
          const float p1 = __builtin_amdgcn_exp2f(x[1]);
          const float p2 = __builtin_amdgcn_exp2f(x[2]);
          const float p3 = __builtin_amdgcn_exp2f(x[3]);
          l_run[hb] += (p0 + p1) + (p2 + p3);
          pk[hb][2 * mb] = pack_bf16(p0, p1);
          pk[hb][2 * mb + 1] = pack_bf16(p2, p3);
        }
      };
      bf16x8 kf[RS_KLA];
      rs_kfirst<0>(kb0, kb1, kf);
      rs_qk<0>(kb0, kb1, kf, qf, sc, [&]() { numer(0); });
      numer(1);
      {
        const int ln = opaque_lane(lane);
        const uint32_t pw = lds_addr(pbuf) + (uint32_t)((t & 1) * PB_UNITS * 16) +
                            (uint32_t)((((ln >> 4) * HT) + 32 * s + (ln & 15)) * 16);
        ds_write_b128_at<0>(pw, pk[0]);
        ds_write_b128_at<256>(pw, pk[1]);
      }
      if (t > 0) pv(t - 1);
    }
    if (ntiles > 0) {
      lgkm0();
      __builtin_amdgcn_s_barrier();
      pv(ntiles - 1);
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      l_tot[hb] = sum_groups(l_run[hb]);
      bad = bad || !(l_tot[hb] <= kMaxSum);
    }
#pragma unroll
    for (int hb = 0; hb < HBK; ++hb)
#pragma unroll
      for (int j = 0; j < RS_SDB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad = bad || !__builtin_isfinite(oacc[hb][j][i]);
    // ---- epilogue below, after the flags are exchanged
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    float *xch = (float *)(pbuf + (ntiles & 1) * PB_UNITS * 16);
    if (g == 0) {
      xch[32 * s + n] = l_tot[0];
      xch[32 * s + 16 + n] = l_tot[1];
    }
    if (lane == 0) ((int *)xch)[HT + w] = wave_bad ? 1 : 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) flagged |= ((const int *)xch)[HT + i];
    if (!flagged) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int hl = ht * HT + 32 * s + 16 * hb + n;
      if (g == 0 && hl < G)
        D.ws_lse[part * HT + 32 * s + 16 * hb + n] =
            l_tot[hb] > 0.f ? (m_ref[hb] + log2f(l_tot[hb])) * kLn2 : -INFINITY;
    }
#pragma unroll
    for (int hb = 0; hb < HBK; ++hb) {
      const float lt = xch[16 * hb + n];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float *wo = D.ws_o + (part * HT + 16 * hb + n) * DV + 128 * s + 4 * g;
#pragma unroll
      for (int j = 0; j < RS_SDB; ++j)
        *(float4 *)(wo + 16 * j) = make_float4(oacc[hb][j][0] * inv, oacc[hb][j][1] * inv,
                                               oacc[hb][j][2] * inv, oacc[hb][j][3] * inv);
    }
    }
  } else {
    // ---- output wave: copies rows 8 s .. 8 s + 7 of each tile, PV of
    // columns [128 s + 32, 128 s + 128)
    const __bf16 *kbase =
        (const __bf16 *)p.k + (int64_t)sd.kv_begin * p.k_rs + (int64_t)kvh * p.k_hs;
    const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)kbase, (short)0, (int)((int64_t)k_hi * p.k_rs * 2), 0x00020000);
    const int x_lo = sd.kv_begin + k_lo;
    // (read through the constant address space: the table is not written
    // during the kernel, so the uniform read is a scalar load, whose wait
    // leaves the copies in flight alone; a vector load here made the
    // compiler wait for every copy in flight, vmcnt(0), each tile)
    const __attribute__((address_space(4))) int32_t *btab =
        (const __attribute__((address_space(4))) int32_t *)(uintptr_t)p.block_table;
    auto tile_block = [&](int t) -> int {
      if (!PAGED) return 0;
      const int x0 = x_lo + t * BN;
      const int b = btab[(int64_t)sd.req * p.bt_stride + x0 / p.block_size];
      return __builtin_amdgcn_readfirstlane(min(max(b, 0), p.pool_blocks - 1));
    };
    auto tile_rsrc = [&](int t, int b, uint32_t &row0) -> __amdgpu_buffer_rsrc_t {
      if (!PAGED) {
        row0 = (uint32_t)((k_lo + t * BN) * p.k_rs) * 2u;
        return krsrc;
      }
      const int x0 = x_lo + t * BN;
      const int64_t prow = (int64_t)b * p.block_size + x0 % p.block_size;
      const int rows = min(BN, k_hi - (k_lo + t * BN));
      row0 = 0u;
      return __builtin_amdgcn_make_buffer_rsrc(
          (void *)((const __bf16 *)p.k + prow * p.k_rs + (int64_t)kvh * p.k_hs), (short)0,
          (int)(rows * p.k_rs * 2), 0x00020000);
    };
    // per-lane copy offsets: four kept, the other five rebuilt at each issue
    uint32_t dma_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_off[i] = dma_lane_offset(RS_DMA * s + i, lane, (int)p.k_rs);
    auto issue = [&](int t, int b) {
      uint32_t row0;
      const __amdgpu_buffer_rsrc_t trsrc = tile_rsrc(t, b, row0);
      u32x4 *dst = lds + (t % NBUF_X) * TILE_CH + RS_DMA * s * 64;
#pragma unroll
      for (int i = 0; i < RS_DMA; ++i) {
        const uint32_t off =
            i < 4 ? dma_off[i] : dma_lane_offset(RS_DMA * s + i, opaque_lane(lane), (int)p.k_rs);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            trsrc, (__attribute__((address_space(3))) void *)(dst + i * 64), 16, row0 + off, 0, 0,
            0);
      }
    };
    f32x4 oacc[HBK][RS_ODB];
#pragma unroll
    for (int hb = 0; hb < HBK; ++hb)
#pragma unroll
      for (int j = 0; j < RS_ODB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[hb][j][i] = 0.f;
    auto pv = [&](int u) {
      int trb[4];
      tr_bases(trb);
      rs_pv_out(stage_addr(u) + 256u * (uint32_t)s, p_read_addr(u), trb, oacc);
    };
    if (ntiles > 0) issue(0, tile_block(0));
    if (ntiles > 1) issue(1, tile_block(1));
    for (int t = 0; t < ntiles; ++t) {
      const int bnext = t + 2 < ntiles ? tile_block(t + 2) : 0;
      // this wave's rows of tile t have landed (tile t + 1's may pend)
      if (t + 1 < ntiles) wait_vm_lgkm0<RS_DMA>(); else wait_vm_lgkm0<0>();
      if (PAGED) asm volatile("" : : "s"(bnext));
      __builtin_amdgcn_s_barrier();
      // tile t + 2 goes to the stage of tile t - 2, free since the barrier
      if (t + 2 < ntiles) issue(t + 2, bnext);
      if (t > 0) pv(t - 1);
    }
    if (ntiles > 0) {
      wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      pv(ntiles - 1);
    }
#pragma unroll
    for (int hb = 0; hb < HBK; ++hb)
#pragma unroll
      for (int j = 0; j < RS_ODB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad = bad || !__builtin_isfinite(oacc[hb][j][i]);
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    float *xch = (float *)(pbuf + (ntiles & 1) * PB_UNITS * 16);
    if (lane == 0) ((int *)xch)[HT + w] = wave_bad ? 1 : 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) flagged |= ((const int *)xch)[HT + i];
    if (tid == 256) D.ws_flags[blockIdx.x] = flagged;
    if (!flagged) {
#pragma unroll
    for (int hb = 0; hb < HBK; ++hb) {
      const float lt = xch[16 * hb + n];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float *wo = D.ws_o + (part * HT + 16 * hb + n) * DV + 128 * s + 16 * RS_SDB + 4 * g;
#pragma unroll
      for (int j = 0; j < RS_ODB; ++j)
        *(float4 *)(wo + 16 * j) = make_float4(oacc[hb][j][0] * inv, oacc[hb][j][1] * inv,
                                               oacc[hb][j][2] * inv, oacc[hb][j][3] * inv);
    }
    }
  }
}

// Merge of the slices of one (row, head): one wave per (item, head), 8 dv
// elements per lane, LSE merge over the slices.
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(const AttnParams p,
                                                                  const DecodeLaunch D) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int item = wv / HT, hloc = wv % HT;
  if (item >= D.items) return;
  int si, row, kvh, ht;
  decode_item(D, item, si, row, kvh, ht);
  const SegDesc sd = D.s[si];
  const int G = p.hq / p.hkv;
  const int hl = ht * HT + hloc;
  if (hl >= G) return;
  const int h = kvh * G + hl;
  const int64_t qrow = (int64_t)sd.q_begin + row;
  const int64_t part0 = (int64_t)item * D.nsplit;
  const int ns = D.nsplit;
  // the first CMB_PRE slices' log-sum-exps and partial rows are loaded at
  // once, before any of them is used (every slice's partial is written, by
  // the main or the exact pass), so the wave waits for memory once
  constexpr int CMB_PRE = 4;
  float lsv[CMB_PRE];
  float4 xa[CMB_PRE], xb[CMB_PRE];
#pragma unroll
  for (int s = 0; s < CMB_PRE; ++s) {
    lsv[s] = -INFINITY;
    xa[s] = xb[s] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s < ns) {
      lsv[s] = D.ws_lse[(part0 + s) * HT + hloc];
      const float *src = D.ws_o + ((part0 + s) * HT + hloc) * DV + lane * 8;
      xa[s] = *(const float4 *)src;
      xb[s] = *(const float4 *)(src + 4);
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < CMB_PRE; ++s) m = fmaxf(m, lsv[s]);
  for (int s = CMB_PRE; s < ns; ++s) m = fmaxf(m, D.ws_lse[(part0 + s) * HT + hloc]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  auto add = [&](float ls, const float4 &a, const float4 &b) {
    const float wgt = expf(ls - m);
    wsum += wgt;
    acc[0] += wgt * a.x; acc[1] += wgt * a.y; acc[2] += wgt * a.z; acc[3] += wgt * a.w;
    acc[4] += wgt * b.x; acc[5] += wgt * b.y; acc[6] += wgt * b.z; acc[7] += wgt * b.w;
  };
  if (m != -INFINITY) {
#pragma unroll
    for (int s = 0; s < CMB_PRE; ++s)
      if (lsv[s] != -INFINITY) add(lsv[s], xa[s], xb[s]);
    for (int s = CMB_PRE; s < ns; ++s) {
      const float ls = D.ws_lse[(part0 + s) * HT + hloc];
      if (ls == -INFINITY) continue;
      const float *src = D.ws_o + ((part0 + s) * HT + hloc) * DV + lane * 8;
      add(ls, *(const float4 *)src, *(const float4 *)(src + 4));
    }
  }
  float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float lse_out = wsum > 0.f ? m + logf(wsum) : -INFINITY;
  if (p.accumulate) {
    // merge into the running (O, LSE) of this (row, head): an empty new
    // partial leaves it; an empty accumulator (LSE = -inf) is replaced
    if (!(wsum > 0.f)) return;
    const float la = p.lse[qrow * p.lse_rs + h];
    if (la != -INFINITY) {
      const float mm = fmaxf(la, lse_out);
      const float wa = expf(la - mm), wn = expf(lse_out - mm);
      const float winv = 1.f / (wa + wn);
      float oa[8];
      if (p.o_bf16) {
        const u32x4 v = *(const u32x4 *)((const __bf16 *)p.o + qrow * p.o_rs + (int64_t)h * p.o_hs + lane * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          oa[2 * i] = __uint_as_float(v[i] << 16);
          oa[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
      } else {
        const float *op = (const float *)p.o + qrow * p.o_rs + (int64_t)h * p.o_hs + lane * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) oa[i] = op[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = (wa * oa[i] + wn * acc[i] * inv) * winv;
      inv = 1.f;
      lse_out = mm + logf(wa + wn);
    }
  }
  if (p.o_bf16) {
    __bf16 *op = (__bf16 *)p.o + qrow * p.o_rs + (int64_t)h * p.o_hs + lane * 8;
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    *(u32x4 *)op = v;
  } else {
    float *op = (float *)p.o + qrow * p.o_rs + (int64_t)h * p.o_hs + lane * 8;
    *(float4 *)op = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *(float4 *)(op + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (lane == 0) p.lse[qrow * p.lse_rs + h] = lse_out;
}

}  // namespace

hipError_t launch_attn_decode_mla(const AttnParams &p, const DecodeLaunch &D, hipStream_t stream) {
  if (D.items <= 0) return hipSuccess;
  const dim3 grid((unsigned)(D.items * D.nsplit));
  // main pass (flags the slices it cannot keep exact), then the exact pass
  // over the flagged slices only
  if (p.block_table) {
    hipLaunchKernelGGL(attn_decode_rs_kernel<true>, grid, dim3(NT), 0, stream, p, D);
    hipLaunchKernelGGL(attn_decode_mla_kernel<true>, grid, dim3(NT), 0, stream, p, D);
  } else {
    hipLaunchKernelGGL(attn_decode_rs_kernel<false>, grid, dim3(NT), 0, stream, p, D);
    hipLaunchKernelGGL(attn_decode_mla_kernel<false>, grid, dim3(NT), 0, stream, p, D);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = (int64_t)D.items * HT;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                     stream, p, D);
  return hipGetLastError();
}

}  // namespace cpattn

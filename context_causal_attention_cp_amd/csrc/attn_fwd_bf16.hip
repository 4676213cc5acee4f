// Causal varlen flash-attention forward, bf16 in / fp32 accumulate, on the
// CDNA4 (gfx950) matrix cores.
//
// What it computes ("What is Context Parallelism" blog, sections 2.1 and 3.1:
// a rank's queries attend over the full or a partial KV; the partial output
// is normalised and comes with its log-sum-exp): for every row of every
// segment and every query head, O = softmax(scale * q K^T) V over the keys
// whose position is <= the row's position, and LSE = ln sum exp(scale q k).
// Query head h reads KV head h / (hq/hkv) (GQA, blog section 4.1).
//
// One workgroup = 4 waves = 256 query rows of one segment and one head; each
// wave owns 64 rows (two 32-row MFMA column blocks), one wave per SIMD (128
// rows and one block per wave for calls too small to fill the chip otherwise;
// with GQA packing, 4 query heads of one KV head over 64 or 32 rows, one head
// per wave):
//   * K and V tiles of 32 keys are copied HBM -> LDS by range-checked buffer
//     loads straight into LDS (no register staging), in keys-fastest layouts
//     that need no swizzle; up to eight stages, five or six tiles in flight;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys = M, query rows = N): each
//     lane holds scores of one query row, so the softmax is lane-local; the
//     Q fragments stay in registers; every K fragment read from LDS feeds two
//     MFMAs (both row blocks);
//   * O^T += V^T P^T: P leaves the score registers as the B operand; V^T is
//     read from the row-major V tile with the transposing LDS read
//     ds_read_b64_tr_b16, in the accumulator's key order;
//   * the loop is software-pipelined: the products of tile t + 1 run on the
//     matrix cores while the exponentials of tile t run on the VALU;
//   * exp2 with scale*log2(e) folded into one FMA; each row's reference max
//     is fixed from its first tile (main pass), so later tiles take no row
//     max at all; a workgroup where some row's sum of probabilities ends
//     above 2^64 (or not finite) is flagged and recomputed by an exact pass
//     that moves the reference (with an accumulator rescale) instead;
//   * per wave, the number of visible tiles and of fully visible tiles is
//     counted once up front from the tiles' first/last key positions (one
//     wave-wide vector load per 64 tiles); only boundary tiles are masked;
//   * O is transposed through LDS and written as whole rows (or merged into
//     a running (O, LSE) in accumulate mode).
// Work mapping: all workgroups of one KV head go to one XCD (id mod 8) so the
// ones streaming the same K/V share that XCD's L2; inside a head the
// heaviest tiles (longest causal extent) start first.
//
// For qk 192 (the MLA shape) and qk 128 the main pass of 256-row workgroups runs
// as attn_fwd_bf16_split_kernel instead: 8 waves, two per SIMD, the score waves
// holding Q and the output waves holding O of the same 64 rows, with the
// probabilities handed over through LDS (five stages at qk 192, six at qk
// 128).
// A single wave per SIMD issues its products, exponentials, DMA descriptors
// and waits in order and leaves the matrix core idle whenever it stalls; with
// two waves per SIMD the other wave's products fill those gaps.  Same
// arithmetic in the same order: the results are bitwise those of the
// one-wave kernel.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <utility>

#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 4;          // waves
constexpr int NT = 64 * NW;    // threads
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescale = 8.0f;   // exact mode: log2 headroom before the reference moves
constexpr float kGrowMax = 64.0f;  // main mode: log2 headroom before the workgroup is flagged
constexpr float kMaxSum = 18446744073709551616.0f;  // 2^kGrowMax: largest accepted row sum
constexpr int kNoPos = -(1 << 30);

// workgroup id -> (query tile, first query head).  A KV head's G query heads
// come in G / pack groups of pack heads (pack = 4 with GQA packing: the
// workgroup's waves take its 4 heads over the same rows).
__device__ inline void map_work(int id, int num_tiles, int hq, int hkv, int pack, int &tile_order,
                                int &h) {
  const int G = hq / hkv;
  const int GP = G / pack;
  const int per_kvh = num_tiles * GP;
  int kvh, rem;
  if (hkv % kNumXcd == 0) {
    const int x = id % kNumXcd, slot = id / kNumXcd;
    kvh = x + kNumXcd * (slot / per_kvh);
    rem = slot % per_kvh;
  } else {
    kvh = id / per_kvh;
    rem = id % per_kvh;
  }
  tile_order = rem / GP;
  h = kvh * G + (rem % GP) * pack;
}

__device__ inline int find_seg(const LaunchSegs &L, int tile_order) {
  int si = 0;
  for (int i = 1; i < L.num_segs; ++i)
    if (tile_order >= L.s[i].tile_begin) si = i;
  return si;
}

// two floats -> two bf16 (round to nearest even) in one instruction
__device__ inline uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ inline float max_xor32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float sum_xor32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// ds_read_b64_tr_b16 through inline asm.  The intrinsic makes the waitcnt pass
// assume it may alias the LDS-DMA writes still in flight and drain them
// (vmcnt(0)) before every use; the tile it reads was already completed by
// an explicit vmcnt wait and a barrier.  The compiler does not count these
// reads: their results are consumed only after an explicit lgkmcnt wait
// that takes the result registers as operands.
__device__ inline u32x2 lds_read_tr16(const void *p) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1"
               : "=v"(r)
               : "v"((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p));
  return r;
}
// The reads in vl/vh are complete once at most LATER LDS operations issued
// after them are pending: LDS operations complete in issue order, so while
// one of them is pending all later ones are too.  (Reads the compiler issues
// in between only make the wait stricter.)
template <int LATER>
__device__ inline void lds_wait_later(u32x2 (&vl)[4], u32x2 (&vh)[4]) {
  static_assert(LATER == 0 || LATER == 8, "count");
  if constexpr (LATER == 8)
    asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(vl[0]), "+v"(vl[1]), "+v"(vl[2]), "+v"(vl[3]),
                 "+v"(vh[0]), "+v"(vh[1]), "+v"(vh[2]), "+v"(vh[3]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vl[0]), "+v"(vl[1]), "+v"(vl[2]), "+v"(vl[3]),
                 "+v"(vh[0]), "+v"(vh[1]), "+v"(vh[2]), "+v"(vh[3]));
}
template <int LATER>
__device__ inline void lds_wait_later(u32x2 (&vl)[2], u32x2 (&vh)[2]) {
  static_assert(LATER == 0 || LATER == 4, "count");
  if constexpr (LATER == 4)
    asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(vl[0]), "+v"(vl[1]), "+v"(vh[0]), "+v"(vh[1]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vl[0]), "+v"(vl[1]), "+v"(vh[0]), "+v"(vh[1]));
}

template <int N>
__device__ inline void wait_vm() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait until at most `later` tiles of PER instructions each are outstanding
// (later <= MAXL, uniform)
template <int PER, int MAXL>
__device__ inline void wait_later(int later) {
  if constexpr (MAXL >= 5) if (later >= 5) { wait_vm<5 * PER>(); return; }
  if constexpr (MAXL >= 4) if (later == 4) { wait_vm<4 * PER>(); return; }
  if constexpr (MAXL >= 3) if (later == 3) { wait_vm<3 * PER>(); return; }
  if constexpr (MAXL >= 2) if (later == 2) { wait_vm<2 * PER>(); return; }
  if constexpr (MAXL >= 1) if (later == 1) { wait_vm<PER>(); return; }
  wait_vm<0>();
}

// Accumulate mode: merge a row's new normalised partial (8 elements a, c at
// dv offset d0, log-sum-exp ln) into the running (O, LSE) of output row orow
// in p.o / p.lse, in place: m = max(la, ln), w = exp(l - m),
// O = (wa Oa + wn On) / (wa + wn), L = m + ln(wa + wn).  la = -inf means an
// empty accumulator (Oa not read).  Returns false if ln = -inf (nothing to
// merge: the row is left as it is).  The lane with write_lse stores L.
__device__ inline bool merge_into(const AttnParams &p, int64_t orow, int h, int d0, float ln,
                                  bool write_lse, float4 &a, float4 &c) {
  if (ln == -INFINITY) return false;
  float *lp = p.lse + orow * p.lse_rs + h;
  const float la = *lp;
  float lnew = ln;
  if (la != -INFINITY) {
    const float m = fmaxf(la, ln);
    const float wa = expf(la - m), wn = expf(ln - m);
    const float inv = 1.f / (wa + wn);
    float oa[8];
    if (p.o_bf16) {
      const u32x4 v = *(const u32x4 *)((const __bf16 *)p.o + orow * p.o_rs + (int64_t)h * p.o_hs + d0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        oa[2 * i] = __uint_as_float(v[i] << 16);
        oa[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
      }
    } else {
      const float *op = (const float *)p.o + orow * p.o_rs + (int64_t)h * p.o_hs + d0;
      const float4 x = *(const float4 *)op, y = *(const float4 *)(op + 4);
      oa[0] = x.x; oa[1] = x.y; oa[2] = x.z; oa[3] = x.w;
      oa[4] = y.x; oa[5] = y.y; oa[6] = y.z; oa[7] = y.w;
    }
    a = make_float4((wa * oa[0] + wn * a.x) * inv, (wa * oa[1] + wn * a.y) * inv,
                    (wa * oa[2] + wn * a.z) * inv, (wa * oa[3] + wn * a.w) * inv);
    c = make_float4((wa * oa[4] + wn * c.x) * inv, (wa * oa[5] + wn * c.y) * inv,
                    (wa * oa[6] + wn * c.z) * inv, (wa * oa[7] + wn * c.w) * inv);
    lnew = m + logf(wa + wn);
  }
  if (write_lse) *lp = lnew;
  return true;
}

// This lane's index, recomputed where it is used (2 VALU): an asm barrier on
// the input keeps the compiler from hoisting it out of the loop and holding
// it (or spilling it) across the loop.
__device__ inline uint32_t lane_id_here() {
  uint32_t z = 0;
  asm volatile("" : "+v"(z));
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, z));
}

// LDS accesses inside the key loops, all through inline asm.  The
// compiler's wait-count pass cannot tell an LDS access from the LDS-DMA
// writes still in flight into other stages; for a compiler-visible LDS read
// or write in the loop it may drain every outstanding DMA (vmcnt(0)) first,
// which empties the prefetch pipeline (measured: 30 % slower whenever it
// appears).  These accesses are invisible to that pass; their completion is
// waited for explicitly (lgkmcnt) with the result registers tied to the wait.
template <int OFF>
__device__ inline u32x2 lds_read_tr16_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// the V^T fragments of 16-key step C of a stage (addr: the stage's LDS address
// plus this lane's offset), one pair of reads per 32-row dv block B
template <int VCH, int OB, int C, int... B>
__device__ inline void split_tr_reads(uint32_t addr, u32x2 (&vl)[OB], u32x2 (&vh)[OB],
                                      std::integer_sequence<int, B...>) {
  ((vl[B] = lds_read_tr16_at<64 * (4 * VCH * C + 4 * B)>(addr),
    vh[B] = lds_read_tr16_at<64 * (4 * VCH * C + 4 * B) + 128 * VCH>(addr)),
   ...);
}
// O^T += V^T P^T for 16-key step C (both row blocks) from registers; each
// dv block's V^T registers take the same block of the next tile (the stage at
// addr) right after their two products, so the reads run among the products
// and no second register set is needed
template <int VCH, int OB, int C, int... B>
__device__ inline void reload_mma(uint32_t addr, u32x2 (&vl)[OB], u32x2 (&vh)[OB],
                                  const bf16x8 (&pf)[2], f32x16 (&oacc)[OB][2],
                                  std::integer_sequence<int, B...>) {
  ((oacc[B][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, (u32x4){vl[B][0], vl[B][1], vh[B][0], vh[B][1]}), pf[0],
        oacc[B][0], 0, 0, 0),
    oacc[B][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8, (u32x4){vl[B][0], vl[B][1], vh[B][0], vh[B][1]}), pf[1],
        oacc[B][1], 0, 0, 0),
    vl[B] = lds_read_tr16_at<64 * (4 * VCH * C + 4 * B)>(addr),
    vh[B] = lds_read_tr16_at<64 * (4 * VCH * C + 4 * B) + 128 * VCH>(addr)),
   ...);
}
template <int OFF>
__device__ inline u32x4 lds_read_b128_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ inline void lds_write_b128_at(uint32_t addr, u32x4 v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}
// complete once at most LATER LDS operations issued after it are pending
template <int LATER, typename T>
__device__ inline void lds_wait_tie(T &x) {
  static_assert(LATER >= 0 && LATER < 16, "lgkmcnt");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(LATER));
}
__device__ inline uint32_t lds_u32(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// S^T = K Q^T of one tile, k-step ST onwards: the fragment of step ST was read
// KLA steps earlier; the read of step ST + KLA goes out once it is consumed
template <int ST, int KS, int KLA, int RB>
__device__ inline void split_qk(uint32_t ka, bf16x8 (&kf)[KLA], const bf16x8 (&qf)[RB][KS],
                                f32x16 (&sc)[RB]) {
  if constexpr (ST < KS) {
    constexpr int LATER = (KS - 1 - ST) < (KLA - 1) ? (KS - 1 - ST) : (KLA - 1);
    lds_wait_tie<LATER>(kf[ST % KLA]);
    const bf16x8 a = kf[ST % KLA];
    if constexpr (ST + KLA < KS)
      kf[ST % KLA] = __builtin_bit_cast(bf16x8, lds_read_b128_at<512 * (ST + KLA)>(ka));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      sc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][ST], sc[rb], 0, 0, 0);
    split_qk<ST + 1, KS, KLA, RB>(ka, kf, qf, sc);
  }
}
template <int ST, int KLA>
__device__ inline void split_k_first(uint32_t ka, bf16x8 (&kf)[KLA]) {
  if constexpr (ST < KLA) {
    kf[ST] = __builtin_bit_cast(bf16x8, lds_read_b128_at<512 * ST>(ka));
    split_k_first<ST + 1, KLA>(ka, kf);
  }
}

// LDS layouts of one stage (16-byte units; keys fastest, so no swizzle):
//   K  unit ((key/16)*KCH + chunk)*16 + key%16   -- a K fragment read (32 keys
//      of one chunk) is 2 x 256 contiguous bytes;
//   V  unit ((key/4)*VCH + chunk)*4 + key%4      -- a transposing read (4 keys
//      x 16 columns per 16 lanes) is 128 contiguous bytes;
//   then BN key positions (4 bytes each).
// One DMA instruction fills 64 consecutive units, so every lane's global
// offset is a per-lane constant plus a per-instruction uniform term.
template <int DQK, int DV>
struct Cfg {
  static constexpr int BN = 32;                    // keys per tile
  static constexpr int KCH = DQK / 8;              // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;               // ... per V row
  static constexpr int KUNITS = BN * KCH;
  static constexpr int VUNITS = BN * VCH;
  static constexpr int KPOS = KUNITS + VUNITS;     // key positions
  static constexpr int STAGE = KPOS + BN / 4;      // units per stage
  static constexpr int NBUF_FIT = 160 * 1024 / (STAGE * 16);
  static constexpr int NBUF = NBUF_FIT < 8 ? NBUF_FIT : 8;  // LDS stages
  // tiles in flight beyond the two being read (K of tile t+1, V of tile t)
  static constexpr int PREF = NBUF - 2;
  static constexpr int KDMA = KUNITS / 64 / NW;    // DMA instructions per wave per stage
  static constexpr int VDMA = VUNITS / 64 / NW;
  static constexpr int KS = DQK / 16;              // QK k-steps
  static constexpr int OB = DV / 32;               // 32-row dv blocks
  static_assert(KUNITS % (64 * NW) == 0 && VUNITS % (64 * NW) == 0, "DMA split");
  static_assert(KCH % 4 == 0 && (VCH == 8 || VCH == 16), "layout");
  static_assert(NBUF >= 3 && PREF * (KDMA + VDMA + 1) < 64, "stages");
};

// RB = 32-row MFMA column blocks per wave: 2 (256-row workgroups) or 1
// (128-row workgroups, for launches too small to fill the chip otherwise).
// EXACT = false: main pass; each row's softmax reference is the max of its
//   first visible tile and never moves, so the accumulator is never rescaled
//   (no VALU touches it inside the loop) and later tiles need no row max.
//   Probabilities stay finite and exact in relative terms while none exceeds
//   2^kGrowMax.  Checked once at the end: every probability is at most its
//   row's sum, so a workgroup where some row sum is above 2^kGrowMax (or not
//   finite) writes a flag (p.ws, one int32 per workgroup of the launch).  A
//   row of many moderately large probabilities can be flagged needlessly;
//   the exact pass still gives the right result.  (Taking the row max of
//   every tile instead cost 4 % of the kernel time.)
// EXACT = true: recomputes only the flagged workgroups (the others return at
//   once), moving the reference with an in-place rescale whenever a row
//   outgrows it by more than 2^kRescale.
template <int DQK, int DV, int RB, bool EXACT>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void attn_fwd_bf16_kernel(const AttnParams p, const LaunchSegs L) {
  using C = Cfg<DQK, DV>;
  constexpr int RW = 32 * RB;    // query rows per wave
  constexpr int BM = RW * NW;    // query rows per workgroup
  constexpr int KCH = C::KCH, VCH = C::VCH, KS = C::KS, OB = C::OB;
  constexpr int BN = C::BN, NBUF = C::NBUF, PREF = C::PREF;
  __shared__ __attribute__((aligned(1024))) u32x4 sm[C::NBUF][C::STAGE];
  __shared__ int s_flag;
  __shared__ float s_lse[NW * 32];  // epilogue: the new log-sum-exp of each staged row
  int32_t *const flags = (int32_t *)p.ws;
  if (EXACT && flags[blockIdx.x] == 0) return;

  const int tid = threadIdx.x;
  // the wave index is uniform per wave: say so, so that everything derived
  // from it (tile counts, DMA slots) stays in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 31, hf = lane >> 5;

  int tile_order, h;
  map_work(blockIdx.x, L.num_tiles, p.hq, p.hkv, p.pack, tile_order, h);
  if (tile_order >= L.num_tiles) return;
  if (!EXACT) {
    if (tid == 0) s_flag = 0;
    __syncthreads();
  }
  // GQA packing: every wave takes the same RW rows of its own query head
  const bool packed = p.pack > 1;
  const int BMr = packed ? RW : BM;    // query rows of the workgroup
  const int wrow = packed ? 0 : w * RW;  // this wave's first row in them
  if (packed) h += w;
  const SegDesc sd = L.s[find_seg(L, tile_order)];
  const int ntile_q = (sd.q_len + BMr - 1) / BMr;
  const int tq = ntile_q - 1 - (tile_order - sd.tile_begin);
  const int row0 = tq * BMr;
  const int rows_here = min(BMr, sd.q_len - row0);
  const int kvh = h / (p.hq / p.hkv);

  // ---- this lane's query rows (one per row block)
  int qpos[RB];
  bool valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = wrow + rb * 32 + n;
    valid[rb] = rr < rows_here;
    qpos[rb] = valid[rb] ? sd.pos_begin + (row0 + rr) * sd.pos_stride : kNoPos;
  }
  const int nvalid_w = max(0, min(RW, rows_here - wrow));
  const int qmin_w = nvalid_w ? sd.pos_begin + (row0 + wrow) * sd.pos_stride : kNoPos;
  const int qmax_w =
      nvalid_w ? sd.pos_begin + (row0 + wrow + nvalid_w - 1) * sd.pos_stride : kNoPos;
  const int qmax_wg = sd.pos_begin + (row0 + rows_here - 1) * sd.pos_stride;

  // ---- tile counts: visible for the workgroup / this wave, fully visible
  const int n_kv = sd.kv_len;
  const int ntiles_all = (n_kv + BN - 1) / BN;
  const int32_t *kvp = p.kv_pos ? p.kv_pos + sd.kv_begin : nullptr;
  int n_wg, n_vis, n_full;
  if (!p.causal) {
    n_wg = n_vis = ntiles_all;
    n_full = n_kv / BN;
  } else if (!kvp) {
    n_wg = (min(n_kv, max(qmax_wg + 1, 0)) + BN - 1) / BN;
    n_vis = (min(n_kv, max(qmax_w + 1, 0)) + BN - 1) / BN;
    n_full = min(n_kv, max(qmin_w + 1, 0)) / BN;
  } else {
    // positions increase: count tiles whose first key is visible to the
    // last row, and tiles whose last key is visible to the first row
    n_wg = n_vis = n_full = 0;
    for (int t0 = 0; t0 < ntiles_all; t0 += 64) {
      const int t = t0 + lane;
      int first = INT_MAX, last = INT_MAX;
      if (t < ntiles_all) {
        first = kvp[t * BN];
        if ((t + 1) * BN <= n_kv) last = kvp[t * BN + BN - 1];
      }
      n_wg += __builtin_popcountll(__builtin_amdgcn_ballot_w64(first <= qmax_wg));
      n_vis += __builtin_popcountll(__builtin_amdgcn_ballot_w64(first <= qmax_w));
      n_full += __builtin_popcountll(__builtin_amdgcn_ballot_w64(last <= qmin_w));
    }
  }
  if (nvalid_w == 0) n_vis = n_full = 0;

  // ---- Q fragments: B operand of S^T = K Q^T (n = row, k = d)
  bf16x8 qf[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t qrow = (int64_t)sd.q_begin + row0 + wrow + rb * 32 + n;
    const __bf16 *qp = (const __bf16 *)p.q + qrow * p.q_rs + (int64_t)h * p.q_hs + 8 * hf;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (valid[rb] && n_vis > 0) x = *(const u32x4 *)(qp + 16 * s);  // no key: Q unused
      qf[rb][s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- LDS DMA of one stage (K units, V units, key positions of a tile).
  // K instruction I: keys 16*(4I/KCH) + lane%16, chunk (4I)%KCH + lane/16.
  // V instruction I: keys 4*(16I/VCH + (lane/4)/VCH) + lane%4, chunk (lane/4)%VCH.
  const __bf16 *kbase = (const __bf16 *)p.k + (int64_t)sd.kv_begin * p.k_rs + (int64_t)kvh * p.k_hs;
  const __bf16 *vbase = (const __bf16 *)p.v + (int64_t)sd.kv_begin * p.v_rs + (int64_t)kvh * p.v_hs;
  const uint32_t k_rb = (uint32_t)p.k_rs * 2u, v_rb = (uint32_t)p.v_rs * 2u;  // row bytes
  const uint32_t k_lane = (uint32_t)(lane & 15) * k_rb + (uint32_t)(lane >> 4) * 16u;
  const uint32_t v_lane =
      (uint32_t)(4 * ((lane >> 2) / VCH) + (lane & 3)) * v_rb + (uint32_t)((lane >> 2) % VCH) * 16u;
  auto issue = [&](int t) {
    const int j0 = t * BN;
    const int nrows = min(BN, n_kv - j0);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(kbase + (int64_t)j0 * p.k_rs), (short)0, (int)(nrows * k_rb), 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(vbase + (int64_t)j0 * p.v_rs), (short)0, (int)(nrows * v_rb), 0x00020000);
    u32x4 *dst = sm[t % NBUF];
#pragma unroll
    for (int i = 0; i < C::KDMA; ++i) {
      const int I = w * C::KDMA + i;
      const uint32_t off = k_lane + (uint32_t)(16 * (4 * I / KCH)) * k_rb + (uint32_t)((4 * I) % KCH) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          kr, (__attribute__((address_space(3))) void *)(dst + I * 64), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::VDMA; ++i) {
      const int I = w * C::VDMA + i;
      const uint32_t off = v_lane + (uint32_t)(4 * (16 * I / VCH)) * v_rb;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vr, (__attribute__((address_space(3))) void *)(dst + C::KUNITS + I * 64), 16, off, 0,
          0, 0);
    }
    if (kvp && w == 0 && lane < BN) {
      const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(kvp + j0), (short)0, nrows * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          pr, (__attribute__((address_space(3))) void *)(dst + C::KPOS), 4, (uint32_t)lane * 4u,
          0, 0, 0);
    }
  };
  constexpr int DMA_W = C::KDMA + C::VDMA;
  // tile u's DMA is complete once at most the later in-flight tiles'
  // instructions are outstanding (loads complete in order); then every wave
  // has it after the barrier
  auto wait_tile = [&](int u) {
    const int later = min(n_wg - 1 - u, PREF - 1);
    if (kvp && w == 0) wait_later<DMA_W + 1, PREF - 1>(later);
    else wait_later<DMA_W, PREF - 1>(later);
    __builtin_amdgcn_s_barrier();
    if (u + PREF < n_wg) issue(u + PREF);
  };

  // per-lane LDS byte offsets inside a stage
  //  K fragment (A of S^T): key n, chunk 2*s + hf   -> kq + 512*s
  //  V^T fragment (A of O^T, transposing read): 16-lane block bb, lane li
  //  addresses key 16*ks + 4*hf + 8*hi + li/4, dv 32*mb + 16*(bb&1) + 4*(li&3)
  //                                                  -> vt + 64*(4*VCH*ks + 2*VCH*hi + 4*mb)
  const int li = lane & 15, bb = lane >> 4;
  const int kq = ((n >> 4) * KCH + hf) * 256 + (n & 15) * 16;
  const int vt = C::KUNITS * 16 +
                 ((hf * VCH + 2 * (bb & 1) + ((li & 3) >> 1)) * 4 + (li >> 2)) * 16 + 8 * (li & 1);

  f32x16 oacc[OB][RB];
#pragma unroll
  for (int b = 0; b < OB; ++b)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[b][rb][i] = 0.f;
  float m_ref[RB], l_run[RB];  // reference max (log2 units), this half's row sums
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_ref[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }
  const float sl2 = p.scale_log2;

  // S^T = K Q^T of one tile (32 keys x RB row blocks); K fragments rotate
  // through KLA registers, each read issued KLA k-steps before its use (hides
  // the LDS latency behind the products)
  auto qk = [&](f32x16 (&sc)[RB], const char *tl) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[rb][i] = 0.f;
    constexpr int KLA = KS < 4 ? KS : 4;
    const uint32_t ka = lds_u32(tl) + (uint32_t)kq;
    bf16x8 kf[KLA];
    split_k_first<0, KLA>(ka, kf);
    split_qk<0, KS, KLA, RB>(ka, kf, qf, sc);
  };
  // boundary tiles: keys past the segment or after the row's position
  auto mask = [&](f32x16 (&sc)[RB], const char *tl, int j0) {
    int kpos[16];
    if (kvp) {
      // this lane's keys: 4 runs of 4 consecutive positions (8g + 4hf + 0..3)
      const uint32_t pa = lds_u32(tl) + (uint32_t)(C::KPOS * 16 + 16 * hf);
      u32x4 r0 = lds_read_b128_at<0>(pa), r1 = lds_read_b128_at<32>(pa);
      u32x4 r2 = lds_read_b128_at<64>(pa), r3 = lds_read_b128_at<96>(pa);
      lds_wait_tie<3>(r0);
      lds_wait_tie<2>(r1);
      lds_wait_tie<1>(r2);
      lds_wait_tie<0>(r3);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kpos[e] = (int)r0[e];
        kpos[4 + e] = (int)r1[e];
        kpos[8 + e] = (int)r2[e];
        kpos[12 + e] = (int)r3[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) kpos[i] = j0 + 8 * (i >> 2) + 4 * hf + (i & 3);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kj = 8 * (i >> 2) + 4 * hf + (i & 3);
      const bool in = j0 + kj < n_kv;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bool vis = in && (!p.causal || kpos[i] <= qpos[rb]);
        sc[rb][i] = vis ? sc[rb][i] : -INFINITY;
      }
    }
  };
  // lane-local row max in log2 units
  auto rowmax = [&](const f32x16 (&sc)[RB], float (&m2)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, sc[rb][i]);
      m2[rb] = m * sl2;
    }
  };
  // P of 16-key step c: exp2(s*scale*log2e - m_ref) as the B operand
  // (element e <-> key 16c + 8*(e/4) + 4*hf + e%4); row sums in fp32 (the
  // log-sum-exp keeps fp32 accuracy)
  auto probs = [&](const f32x16 (&sc)[RB], int c, bf16x8 (&pf)[RB], float (&ls)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mneg = (m_ref[rb] == -INFINITY) ? 0.f : -m_ref[rb];
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[rb][8 * c + 2 * e], sl2, mneg));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[rb][8 * c + 2 * e + 1], sl2, mneg));
        ls[rb] += p0 + p1;
        pk[e] = pack_bf16(p0, p1);
      }
      pf[rb] = __builtin_bit_cast(bf16x8, pk);
    }
  };
  // V^T fragments of 16-key step c of the tile at tl (issued; consumed by pv_mma)
  auto pv_read = [&](const char *tl, int c, u32x2 (&vl)[OB], u32x2 (&vh)[OB]) {
#pragma unroll
    for (int b = 0; b < OB; ++b) {
      const char *vp = tl + vt + 64 * (4 * VCH * c + 4 * b);
      vl[b] = lds_read_tr16(vp);
      vh[b] = lds_read_tr16(vp + 64 * 2 * VCH);
    }
  };
  auto pv_mma = [&](u32x2 (&vl)[OB], u32x2 (&vh)[OB], const bf16x8 (&pf)[RB]) {
#pragma unroll
    for (int b = 0; b < OB; ++b) {
      const u32x4 av = {vl[b][0], vl[b][1], vh[b][0], vh[b][1]};
      const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        oacc[b][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[rb], oacc[b][rb], 0, 0, 0);
    }
  };
  // O^T += V^T P^T for 16-key step c of the tile at tl, reads and products
  auto pv = [&](const char *tl, int c, const bf16x8 (&pf)[RB]) {
    u32x2 vl[OB], vh[OB];
    pv_read(tl, c, vl, vh);
    lds_wait_later<0>(vl, vh);
    pv_mma(vl, vh, pf);
  };
  auto stage = [&](int t) { return (const char *)sm[t % NBUF]; };
  float mx[RB];
  auto grows = [&]() {
    bool g = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) g = g || (mx[rb] > m_ref[rb] + (EXACT ? kRescale : kGrowMax));
    return __builtin_amdgcn_ballot_w64(g) != 0;
  };
  auto add_ls = [&](const float (&ls)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l_run[rb] += ls[rb];
  };
  // One pipelined step: S of tile t + 1 and the first half of PV of tile t on
  // the matrix cores while the exponentials of tile t run; then the second
  // half of PV while the max of tile t + 1 is taken.  Returns whether a row
  // of tile t + 1 outgrew its reference.
  auto step = [&](f32x16 (&cur)[RB], f32x16 (&nxt)[RB], int t) -> bool {
    const int u = t + 1;
    wait_tile(u);
    const char *tc = stage(t), *tn = stage(u);
    float ls[RB] = {};
    bf16x8 pf0[RB], pf1[RB];
    // scheduling hint: interleave the products with the LDS reads and the
    // exponentials of this block (measured: +2-3 % over the default order)
    __builtin_amdgcn_iglp_opt(0);
    // the V^T reads of the second key step go out before the wait for the
    // first one's (1.5 % faster than draining after each step's reads)
    u32x2 vl0[OB], vh0[OB], vl1[OB], vh1[OB];
    qk(nxt, tn);
    pv_read(tc, 0, vl0, vh0);
    probs(cur, 0, pf0, ls);
    pv_read(tc, 1, vl1, vh1);
    lds_wait_later<2 * OB>(vl0, vh0);  // the second step's reads may be pending
    pv_mma(vl0, vh0, pf0);
    probs(cur, 1, pf1, ls);
    if (u >= n_full) mask(nxt, tn, u * BN);
    if (EXACT) rowmax(nxt, mx);
    lds_wait_later<0>(vl1, vh1);
    pv_mma(vl1, vh1, pf1);
    add_ls(ls);
    return EXACT ? grows() : false;
  };
  // move the reference max (rare): O and l of the rows scale by exp2(old - new)
  auto rescale = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float m_new = fmaxf(m_ref[rb], max_xor32(mx[rb]));
      const float alpha = (m_ref[rb] == -INFINITY) ? 0.f : exp2f(m_ref[rb] - m_new);
      l_run[rb] *= alpha;
#pragma unroll
      for (int b = 0; b < OB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][rb][i] *= alpha;
      m_ref[rb] = m_new;
    }
  };

#pragma unroll
  for (int i = 0; i < PREF; ++i)
    if (i < n_wg) issue(i);

  f32x16 sa[RB], sb[RB];
  int t = 0;  // the tile whose scores are in sa
  if (n_vis > 0) {
    wait_tile(0);
    qk(sa, stage(0));
    if (n_full == 0) mask(sa, stage(0), 0);
    rowmax(sa, mx);
    // first keys: O and l are still zero, only the reference is set
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) m_ref[rb] = max_xor32(mx[rb]);
    // The hot loop runs two steps per trip so the score buffers alternate
    // without copies; a reference move (rare) rescales O and l in place.
    // main pass: a row that outgrew its reference flags the workgroup (this
    // tile's probabilities may be out of range; the exact pass redoes it)
    auto outgrown = [&]() {
      if (EXACT) rescale();
      else if (lane == 0) s_flag = 1;
    };
    while (t + 2 < n_vis) {
      if (step(sa, sb, t)) outgrown();
      if (step(sb, sa, t + 1)) outgrown();
      t += 2;
    }
    if (t + 1 < n_vis) {
      if (step(sa, sb, t)) outgrown();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sa[rb] = sb[rb];
      t += 1;
    }
    // the last visible tile: exponentials and PV only
    {
      float ls[RB] = {};
      bf16x8 pf0[RB], pf1[RB];
      const char *tc = stage(t);
      probs(sa, 0, pf0, ls);
      pv(tc, 0, pf0);
      probs(sa, 1, pf1, ls);
      pv(tc, 1, pf1);
      add_ls(ls);
    }
    ++t;
  }
  // tiles other waves still compute: keep the barriers and the DMA in step
  for (; t < n_wg; ++t) wait_tile(t);

  // ---- epilogue: normalise; O^T -> LDS -> whole output rows
  float inv[RB], lse[RB];
  bool bad = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = sum_xor32(l_run[rb]);
    const bool any = l_tot > 0.f;
    inv[rb] = any ? 1.f / l_tot : 0.f;
    lse[rb] = any ? (m_ref[rb] + log2f(l_tot)) * kLn2 : -INFINITY;
    // main pass: every probability is at most its row sum, so a sum above
    // 2^kGrowMax (or not finite) means a score outgrew the reference
    bad = bad || !(l_tot <= kMaxSum);
  }
  if (!EXACT) {
    // probabilities within range can still carry huge values of V past the
    // fp32 range (|v| > 2^128 / row sum): such an accumulator is flagged too,
    // and the exact pass, whose probabilities stay below 2^kRescale,
    // recomputes it (the exact output is a convex combination of V rows)
    bool fin = true;
#pragma unroll
    for (int b = 0; b < OB; ++b)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) fin = fin && __builtin_isfinite(oacc[b][rb][i]);
    bad = bad || !fin;
  }
  if (!EXACT && __builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) s_flag = 1;
  __syncthreads();  // every wave is done with the tiles (and its flag is in)
  if (!EXACT) {
    const int flagged = s_flag;
    if (tid == 0) flags[blockIdx.x] = flagged;
    if (flagged) return;  // the exact pass writes (or merges) these rows
  }
  constexpr int OSZ = 4;                       // bytes per staged element (fp32)
  constexpr int OPITCH = DV * OSZ + 16;        // row pitch of the staging area
  static_assert(NW * 32 * OPITCH <= NBUF * C::STAGE * 16, "staging fits the stages");
  char *ost = (char *)sm + w * 32 * OPITCH;    // 32 rows per wave per pass
  for (int rb = 0; rb < RB; ++rb) {
    // this lane: row n of block rb, dv = 32*b + 8*(i/4) + 4*hf + (i%4)
#pragma unroll
    for (int b = 0; b < OB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 x = make_float4(oacc[b][rb][4 * g] * inv[rb], oacc[b][rb][4 * g + 1] * inv[rb],
                               oacc[b][rb][4 * g + 2] * inv[rb], oacc[b][rb][4 * g + 3] * inv[rb]);
        *(float4 *)(ost + n * OPITCH + (32 * b + 8 * g + 4 * hf) * OSZ) = x;
      }
    if (hf == 0) s_lse[w * 32 + n] = lse[rb];
    if (!p.accumulate && hf == 0 && valid[rb]) {
      const int64_t orow = (int64_t)sd.o_begin + row0 + wrow + rb * 32 + n;
      p.lse[orow * p.lse_rs + h] = lse[rb];
    }
    __builtin_amdgcn_s_barrier();  // (wave-local data; keeps the waves in step)
    // whole rows: 8 output elements per lane
    constexpr int LPR = DV / 8;                // lanes per row
    constexpr int RPI = 64 / LPR;              // rows per instruction
    const int sub = lane % LPR, rsub = lane / LPR;
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPI) {
      const int r = r0 + rsub;
      const int rr = wrow + rb * 32 + r;
      if (rr < rows_here) {
        float4 a = *(const float4 *)(ost + r * OPITCH + sub * 8 * OSZ);
        float4 c = *(const float4 *)(ost + r * OPITCH + sub * 8 * OSZ + 16);
        const int64_t orow = (int64_t)sd.o_begin + row0 + rr;
        if (p.accumulate && !merge_into(p, orow, h, sub * 8, s_lse[w * 32 + r], sub == 0, a, c))
          continue;  // no visible key in this call: the accumulator row stays
        if (p.o_bf16) {
          u32x4 v;
          v[0] = pack_bf16(a.x, a.y);
          v[1] = pack_bf16(a.z, a.w);
          v[2] = pack_bf16(c.x, c.y);
          v[3] = pack_bf16(c.z, c.w);
          *(u32x4 *)((__bf16 *)p.o + orow * p.o_rs + (int64_t)h * p.o_hs + sub * 8) = v;
        } else {
          float *op = (float *)p.o + orow * p.o_rs + (int64_t)h * p.o_hs + sub * 8;
          *(float4 *)op = a;
          *(float4 *)(op + 4) = c;
        }
      }
    }
    __builtin_amdgcn_s_barrier();
  }
}

// wait until this wave's own DMA of a tile is complete (at most `later` later
// tiles of PER instructions each still in flight) and its LDS operations are
// done (the probabilities it wrote, the fragments it read)
template <int N>
__device__ inline void wait_vm_lgkm0() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}
template <int PER, int MAXL>
__device__ inline void wait_later_lgkm0(int later) {
  if constexpr (MAXL >= 5) if (later >= 5) { wait_vm_lgkm0<5 * PER>(); return; }
  if constexpr (MAXL >= 4) if (later == 4) { wait_vm_lgkm0<4 * PER>(); return; }
  if constexpr (MAXL >= 3) if (later == 3) { wait_vm_lgkm0<3 * PER>(); return; }
  if constexpr (MAXL >= 2) if (later == 2) { wait_vm_lgkm0<2 * PER>(); return; }
  if constexpr (MAXL >= 1) if (later == 1) { wait_vm_lgkm0<PER>(); return; }
  wait_vm_lgkm0<0>();
}

// Stages of the split-role main pass: the probabilities of a tile take a
// double buffer of 2 x 4 waves x 4 KiB next to the K/V stages.
template <int DQK, int DV>
struct SplitCfg {
  using C = Cfg<DQK, DV>;
  static constexpr int PBYTES = 2 * 4 * 4096;
  static constexpr int NBUF_FIT = (160 * 1024 - PBYTES - 3 * 1024) / (C::STAGE * 16);
  // at qk 192 five stages, two tiles in flight beyond the three being read:
  // measured faster than the six that fit; at qk 128 six (since the output
  // waves copy whole tiles after their products: 1 % faster than five on the
  // 12-request interleave, seven slower)
  static constexpr int NBUF_MAX = DQK == 128 ? 6 : 5;
  static constexpr int NBUF = NBUF_FIT < NBUF_MAX ? NBUF_FIT : NBUF_MAX;
  // a stage is read in iterations i (K) and i + 2 (V)
  static constexpr int PREF = NBUF - 3;
  static_assert(PREF >= 2, "stages");
};

// Main pass of 256-row workgroups with split roles: 8 waves, two per SIMD.
// Waves 0-3 ("score waves") hold Q of 64 rows each and compute the scores and
// the probabilities; waves 4-7 ("output waves") hold the O accumulators of the
// same rows.  Score wave s and output wave 4 + s share a SIMD, so one wave's
// exponentials run on the VALU while the other's products run on the matrix
// core, and no wave keeps both Q and O (which would not fit the 256 registers
// a wave has at two waves per SIMD for qk 192).  Per iteration i (one barrier):
//   score waves:  S(i) = K(i) Q^T, interleaved with the exponentials of
//                 S(i - 1), which go to LDS as P(i - 1) (bf16, already in the
//                 B-operand layout of the PV product: lane l of the output
//                 wave reads what lane l of its score wave wrote);
//   output waves: O^T += V(i - 3)^T P(i - 3)^T from registers, each operand
//                 register reloaded with its part of V(i - 2) or P(i - 2) for
//                 the next iteration right after its last product.
// The arithmetic and its order are those of attn_fwd_bf16_kernel<.., 2, false>
// (same scores, same bf16 probabilities, same row sums, same product order),
// so outputs, log-sum-exps and flags are bitwise the same; the exact pass of
// that kernel recomputes the flagged workgroups.
template <int DQK, int DV>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_split_kernel(const AttnParams p, const LaunchSegs L) {
  using C = Cfg<DQK, DV>;
  using SC = SplitCfg<DQK, DV>;
  constexpr int RB = 2, RW = 64, BM = 256;
  constexpr int KCH = C::KCH, VCH = C::VCH, KS = C::KS, OB = C::OB;
  constexpr int BN = C::BN, NBUF = SC::NBUF, PREF = SC::PREF;
  __shared__ __attribute__((aligned(1024))) u32x4 sm[NBUF][C::STAGE];
  __shared__ __attribute__((aligned(16))) u32x4 pbuf[2][4][2 * RB][64];  // [i&1][wave][rb,c][lane]
  __shared__ float s_l[BM], s_m[BM];  // row sums and references, score -> output waves
  __shared__ float s_lse[4 * 32];
  __shared__ int s_flag;
  int32_t *const flags = (int32_t *)p.ws;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score = w < 4;
  const int s = w & 3;  // the 64-row slice of this wave
  const int lane = tid & 63, n = lane & 31, hf = lane >> 5;

  int tile_order, h;
  map_work(blockIdx.x, L.num_tiles, p.hq, p.hkv, p.pack, tile_order, h);
  if (tile_order >= L.num_tiles) return;
  if (tid == 0) s_flag = 0;
  __syncthreads();
  // GQA packing: every wave pair takes the same 64 rows of its own query head
  const bool packed = p.pack > 1;
  const int BMr = packed ? RW : BM;    // query rows of the workgroup
  const int wrow = packed ? 0 : s * RW;  // this wave pair's first row in them
  if (packed) h += s;
  const SegDesc sd = L.s[find_seg(L, tile_order)];
  const int ntile_q = (sd.q_len + BMr - 1) / BMr;
  const int tq = ntile_q - 1 - (tile_order - sd.tile_begin);
  const int row0 = tq * BMr;
  const int rows_here = min(BMr, sd.q_len - row0);
  const int kvh = h / (p.hq / p.hkv);

  int qpos[RB];
  bool valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = wrow + rb * 32 + n;
    valid[rb] = rr < rows_here;
    qpos[rb] = valid[rb] ? sd.pos_begin + (row0 + rr) * sd.pos_stride : kNoPos;
  }
  const int nvalid_w = max(0, min(RW, rows_here - wrow));
  const int qmin_w = nvalid_w ? sd.pos_begin + (row0 + wrow) * sd.pos_stride : kNoPos;
  const int qmax_w =
      nvalid_w ? sd.pos_begin + (row0 + wrow + nvalid_w - 1) * sd.pos_stride : kNoPos;
  const int qmax_wg = sd.pos_begin + (row0 + rows_here - 1) * sd.pos_stride;

  const int n_kv = sd.kv_len;
  const int ntiles_all = (n_kv + BN - 1) / BN;
  const int32_t *kvp = p.kv_pos ? p.kv_pos + sd.kv_begin : nullptr;
  int n_wg, n_vis, n_full;
  if (!p.causal) {
    n_wg = n_vis = ntiles_all;
    n_full = n_kv / BN;
  } else if (!kvp) {
    n_wg = (min(n_kv, max(qmax_wg + 1, 0)) + BN - 1) / BN;
    n_vis = (min(n_kv, max(qmax_w + 1, 0)) + BN - 1) / BN;
    n_full = min(n_kv, max(qmin_w + 1, 0)) / BN;
  } else {
    n_wg = n_vis = n_full = 0;
    for (int t0 = 0; t0 < ntiles_all; t0 += 64) {
      const int t = t0 + lane;
      int first = INT_MAX, last = INT_MAX;
      if (t < ntiles_all) {
        first = kvp[t * BN];
        if ((t + 1) * BN <= n_kv) last = kvp[t * BN + BN - 1];
      }
      n_wg += __builtin_popcountll(__builtin_amdgcn_ballot_w64(first <= qmax_wg));
      n_vis += __builtin_popcountll(__builtin_amdgcn_ballot_w64(first <= qmax_w));
      n_full += __builtin_popcountll(__builtin_amdgcn_ballot_w64(last <= qmin_w));
    }
  }
  if (nvalid_w == 0) n_vis = n_full = 0;

  // ---- LDS DMA: the score waves copy K (and wave 0 the key positions), the
  // output waves V; same stage layout as attn_fwd_bf16_kernel
  const __bf16 *kbase = (const __bf16 *)p.k + (int64_t)sd.kv_begin * p.k_rs + (int64_t)kvh * p.k_hs;
  const __bf16 *vbase = (const __bf16 *)p.v + (int64_t)sd.kv_begin * p.v_rs + (int64_t)kvh * p.v_hs;
  const uint32_t k_rb = (uint32_t)p.k_rs * 2u, v_rb = (uint32_t)p.v_rs * 2u;
  const uint32_t k_lane = (uint32_t)(lane & 15) * k_rb + (uint32_t)(lane >> 4) * 16u;
  const uint32_t v_lane =
      (uint32_t)(4 * ((lane >> 2) / VCH) + (lane & 3)) * v_rb + (uint32_t)((lane >> 2) % VCH) * 16u;
  // Who copies a tile: at qk 192 the score waves copy K (and the key
  // positions), the output waves V; at qk 128 the output waves copy the whole
  // tile.  The output waves issue theirs after their products; the score
  // waves, theirs right after the barrier or among their products.  (With
  // the output waves' reads running among their products, the score waves'
  // path is the longer one; handing them no copies at qk 192 measured 2 %
  // slower, on the 8192-token shards at qk 128 about 3 % faster.)
  constexpr bool K_S = DQK != 128;  // K and the key positions: score waves
  constexpr bool V_S = false;       // V: output waves
  constexpr bool O_DMA = !K_S || !V_S;
  auto issue = [&](int t) {
    const int j0 = t * BN;
    const int nrows = min(BN, n_kv - j0);
    u32x4 *dst = sm[t % NBUF];
    if (score == K_S) {
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(kbase + (int64_t)j0 * p.k_rs), (short)0, (int)(nrows * k_rb), 0x00020000);
#pragma unroll
      for (int i = 0; i < C::KDMA; ++i) {
        const int I = s * C::KDMA + i;
        const uint32_t off = k_lane + (uint32_t)(16 * (4 * I / KCH)) * k_rb + (uint32_t)((4 * I) % KCH) * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (__attribute__((address_space(3))) void *)(dst + I * 64), 16, off, 0, 0, 0);
      }
      if (kvp && s == 0 && lane < BN) {
        const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kvp + j0), (short)0, nrows * 4, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            pr, (__attribute__((address_space(3))) void *)(dst + C::KPOS), 4, lane_id_here() * 4u,
            0, 0, 0);
      }
    }
    if (score == V_S) {
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(vbase + (int64_t)j0 * p.v_rs), (short)0, (int)(nrows * v_rb), 0x00020000);
#pragma unroll
      for (int i = 0; i < C::VDMA; ++i) {
        const int I = s * C::VDMA + i;
        const uint32_t off = v_lane + (uint32_t)(4 * (16 * I / VCH)) * v_rb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (__attribute__((address_space(3))) void *)(dst + C::KUNITS + I * 64), 16, off, 0,
            0, 0);
      }
    }
  };
  // iteration i begins: this wave's part of tile i has landed and its LDS
  // operations of iteration i - 1 are done; after the barrier every wave has
  // all of tile i and P(i - 2) of every score wave.  The score waves then
  // issue their part of tile i + PREF; the output waves issue theirs after
  // their products, which then start sooner (2-3 % faster)
  // (s_dma = false: a score wave in its steady-state loop issues the copy
  // inside its fused block instead, among the products: 0.5-2 % faster)
  auto top = [&](int i, bool s_dma = true) {
    const int later = min(n_wg - 1 - i, PREF - 1);
    // copy instructions per tile of a score and of an output wave (wave 0 of
    // the K role also copies the key positions)
    constexpr int SPER = (K_S ? C::KDMA : 0) + (V_S ? C::VDMA : 0);
    constexpr int OPER = (K_S ? 0 : C::KDMA) + (V_S ? 0 : C::VDMA);
    if (score) {
      if (K_S && kvp && s == 0) wait_later_lgkm0<SPER + 1, PREF - 1>(later);
      else wait_later_lgkm0<SPER, PREF - 1>(later);
    } else {
      if (!K_S && kvp && s == 0) wait_later_lgkm0<OPER + 1, PREF - 1>(later);
      else wait_later_lgkm0<OPER, PREF - 1>(later);
    }
    __builtin_amdgcn_s_barrier();
    if (score && s_dma && i + PREF < n_wg) issue(i + PREF);
  };
  auto stage = [&](int t) { return (const char *)sm[t % NBUF]; };

#pragma unroll
  for (int i = 0; i < PREF; ++i)
    if (i < n_wg) issue(i);

  const int li = lane & 15, bb = lane >> 4;
  const int kq = ((n >> 4) * KCH + hf) * 256 + (n & 15) * 16;
  const int vt = C::KUNITS * 16 +
                 ((hf * VCH + 2 * (bb & 1) + ((li & 3) >> 1)) * 4 + (li >> 2)) * 16 + 8 * (li & 1);
  const float sl2 = p.scale_log2;
  bool bad = false;

  if (score) {
    // ---------------- score waves
    // Their in-order instruction stream is the critical path of a tile: when
    // both waves of a SIMD have a product ready, the score wave's goes first
    // and the output wave's fill the matrix core while the score wave runs its
    // exponentials (measured: 5 % faster than equal priorities).
    __builtin_amdgcn_s_setprio(3);
    bf16x8 qf[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t qrow = (int64_t)sd.q_begin + row0 + wrow + rb * 32 + n;
      const __bf16 *qp = (const __bf16 *)p.q + qrow * p.q_rs + (int64_t)h * p.q_hs + 8 * hf;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (valid[rb] && n_vis > 0) x = *(const u32x4 *)(qp + 16 * st);
        qf[rb][st] = __builtin_bit_cast(bf16x8, x);
      }
    }
    float m_ref[RB], l_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m_ref[rb] = -INFINITY;
      l_run[rb] = 0.f;
    }
    const uint32_t kq_lds = lds_u32(sm) + (uint32_t)kq;
    auto qk = [&](f32x16 (&sc)[RB], int t) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[rb][i] = 0.f;
      // K fragment reads in flight: six at qk 192 (1.3 % faster than four
      // since the output waves' reads run among their products), four at qk 128
      constexpr int KLA = DQK == 192 ? 6 : (KS < 4 ? KS : 4);
      const uint32_t ka = kq_lds + (uint32_t)((t % NBUF) * C::STAGE * 16);
      bf16x8 kf[KLA];
      split_k_first<0, KLA>(ka, kf);
      split_qk<0, KS, KLA, RB>(ka, kf, qf, sc);
    };
    auto mask = [&](f32x16 (&sc)[RB], int u) {
      const int j0 = u * BN;
      const int hm = (int)(lane_id_here() >> 5);  // (read again: see the epilogue below)
      int kpos[16];
      if (kvp) {
        // this lane's keys: 4 runs of 4 consecutive positions (8g + 4hm + 0..3)
        const uint32_t pa = lds_u32(sm[u % NBUF]) + (uint32_t)(C::KPOS * 16 + 16 * hm);
        u32x4 r0 = lds_read_b128_at<0>(pa), r1 = lds_read_b128_at<32>(pa);
        u32x4 r2 = lds_read_b128_at<64>(pa), r3 = lds_read_b128_at<96>(pa);
        lds_wait_tie<3>(r0);
        lds_wait_tie<2>(r1);
        lds_wait_tie<1>(r2);
        lds_wait_tie<0>(r3);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kpos[e] = (int)r0[e];
          kpos[4 + e] = (int)r1[e];
          kpos[8 + e] = (int)r2[e];
          kpos[12 + e] = (int)r3[e];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) kpos[i] = j0 + 8 * (i >> 2) + 4 * hm + (i & 3);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = 8 * (i >> 2) + 4 * hm + (i & 3);
        const bool in = j0 + kj < n_kv;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const bool vis = in && (!p.causal || kpos[i] <= qpos[rb]);
          sc[rb][i] = vis ? sc[rb][i] : -INFINITY;
        }
      }
    };
    // exponentials of tile u (scores in sc) -> P(u) in the buffer u & 1, row sums
    const uint32_t pw_lds = lds_u32(&pbuf[0][s][0][lane]);
    auto probs_out = [&](const f32x16 (&sc)[RB], int u) {
      const uint32_t pw = pw_lds + (uint32_t)((u & 1) * 4 * 2 * RB * 64 * 16);
      float ls[RB] = {};
      u32x4 pk[2][RB];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float mneg = (m_ref[rb] == -INFINITY) ? 0.f : -m_ref[rb];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[rb][8 * c + 2 * e], sl2, mneg));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[rb][8 * c + 2 * e + 1], sl2, mneg));
            ls[rb] += p0 + p1;
            pk[c][rb][e] = pack_bf16(p0, p1);
          }
        }
      // P(u) as [rb * 2 + c][lane] units of the wave's buffer
      static_assert(RB == 2, "P layout");
      lds_write_b128_at<0 * 1024>(pw, pk[0][0]);
      lds_write_b128_at<1 * 1024>(pw, pk[1][0]);
      lds_write_b128_at<2 * 1024>(pw, pk[0][1]);
      lds_write_b128_at<3 * 1024>(pw, pk[1][1]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) l_run[rb] += ls[rb];
    };
    // before the exponentials of tile u: mask a boundary tile; the first tile
    // fixes each row's reference
    auto pre = [&](f32x16 (&sc)[RB], int u) {
      if (u >= n_full) mask(sc, u);
      if (u == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float m = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) m = fmaxf(m, sc[rb][i]);
          m_ref[rb] = max_xor32(m * sl2);
        }
      }
    };
    // iteration i of the steady state: S(i) -> nxt while P(i - 1) leaves cur;
    // the copy of tile i + PREF goes out among the products
    auto fused = [&](f32x16 (&cur)[RB], f32x16 (&nxt)[RB], int i) {
      __builtin_amdgcn_iglp_opt(0);
      if (i + PREF < n_wg) issue(i + PREF);
      qk(nxt, i);
      probs_out(cur, i - 1);
    };
    f32x16 sa[RB], sb[RB];
    int i = 0;
    top(0);
    if (n_vis > 0) qk(sa, 0);
    i = 1;
    while (i + 1 < n_vis) {
      top(i, false);
      pre(sa, i - 1);
      fused(sa, sb, i);
      top(i + 1, false);
      pre(sb, i);
      fused(sb, sa, i + 1);
      i += 2;
    }
    if (i < n_vis) {
      top(i, false);
      pre(sa, i - 1);
      fused(sa, sb, i);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sa[rb] = sb[rb];
      ++i;
    }
    if (n_vis > 0) {  // i == n_vis: the last visible tile's exponentials
      top(i);
      pre(sa, i - 1);
      probs_out(sa, i - 1);
      ++i;
    }
    for (; i < n_wg + 2; ++i) top(i);
    // row sums and references for the output waves; a row sum above
    // 2^kGrowMax (or not finite) flags the workgroup
    // (the lane index is read again here rather than kept across the loop,
    // where it would take a register the loop needs)
    const int ln = (int)lane_id_here();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l_tot = sum_xor32(l_run[rb]);
      bad = bad || !(l_tot <= kMaxSum);
      if (ln < 32) {
        s_l[s * RW + rb * 32 + ln] = l_tot;
        s_m[s * RW + rb * 32 + ln] = m_ref[rb];
      }
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && ln == 0) s_flag = 1;
    __syncthreads();
    if (tid == 0) flags[blockIdx.x] = s_flag;
    return;  // the output waves write the rows
  }

  // ---------------- output waves
  f32x16 oacc[OB][RB];
#pragma unroll
  for (int b = 0; b < OB; ++b)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[b][rb][i] = 0.f;
  auto pv_mma = [&](u32x2 (&vl)[OB], u32x2 (&vh)[OB], const bf16x8 (&pf)[RB]) {
#pragma unroll
    for (int b = 0; b < OB; ++b) {
      const u32x4 av = {vl[b][0], vl[b][1], vh[b][0], vh[b][1]};
      const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        oacc[b][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[rb], oacc[b][rb], 0, 0, 0);
    }
  };
  // Iteration i multiplies P(i - 3) and V(i - 3), read into registers during
  // iteration i - 1 (both were complete at its barrier), so the products
  // start right after the barrier instead of behind the burst of LDS reads
  // every wave issues there; meanwhile it reads P(i - 2) and V(i - 2) for
  // the next iteration (complete at the next barrier: top() waits for this
  // wave's LDS operations).  pv_reads and pv_products are the pipeline's
  // fill and drain; pv_products_reload below is its steady state.
  const uint32_t pr_lds = lds_u32(&pbuf[0][s][0][lane]);
  static_assert(RB == 2, "P layout");
  u32x4 q00, q01, q10, q11;
  u32x2 vl0[OB], vh0[OB], vl1[OB], vh1[OB];
  auto pv_reads = [&](int u) {
    const uint32_t pr = pr_lds + (uint32_t)((u & 1) * 4 * 2 * RB * 64 * 16);
    q00 = lds_read_b128_at<0 * 1024>(pr);
    q01 = lds_read_b128_at<1 * 1024>(pr);
    q10 = lds_read_b128_at<2 * 1024>(pr);
    q11 = lds_read_b128_at<3 * 1024>(pr);
    const uint32_t va = lds_u32(stage(u)) + (uint32_t)vt;
    split_tr_reads<VCH, OB, 0>(va, vl0, vh0, std::make_integer_sequence<int, OB>{});
    split_tr_reads<VCH, OB, 1>(va, vl1, vh1, std::make_integer_sequence<int, OB>{});
  };
  auto pv_products = [&]() {
    // (complete since the barrier; the waits order the products after it)
    lds_wait_later<0>(vl0, vh0);
    lds_wait_later<0>(vl1, vh1);
    lds_wait_tie<0>(q00);
    lds_wait_tie<0>(q01);
    lds_wait_tie<0>(q10);
    lds_wait_tie<0>(q11);
    const bf16x8 pf0[RB] = {__builtin_bit_cast(bf16x8, q00), __builtin_bit_cast(bf16x8, q10)};
    const bf16x8 pf1[RB] = {__builtin_bit_cast(bf16x8, q01), __builtin_bit_cast(bf16x8, q11)};
    pv_mma(vl0, vh0, pf0);
    pv_mma(vl1, vh1, pf1);
  };
  // the steady state: the products of tile u - 1 with every operand register
  // reloaded from tile u right after its last product (tile u and P(u) are
  // complete at this iteration's barrier)
  auto pv_products_reload = [&](int u, int i) {
    lds_wait_later<0>(vl0, vh0);
    lds_wait_later<0>(vl1, vh1);
    lds_wait_tie<0>(q00);
    lds_wait_tie<0>(q01);
    lds_wait_tie<0>(q10);
    lds_wait_tie<0>(q11);
    const uint32_t pr = pr_lds + (uint32_t)((u & 1) * 4 * 2 * RB * 64 * 16);
    const uint32_t va = lds_u32(stage(u)) + (uint32_t)vt;
    {
      const bf16x8 pf0[RB] = {__builtin_bit_cast(bf16x8, q00), __builtin_bit_cast(bf16x8, q10)};
      reload_mma<VCH, OB, 0>(va, vl0, vh0, pf0, oacc, std::make_integer_sequence<int, OB>{});
    }
    q00 = lds_read_b128_at<0 * 1024>(pr);
    q10 = lds_read_b128_at<2 * 1024>(pr);
    {
      const bf16x8 pf1[RB] = {__builtin_bit_cast(bf16x8, q01), __builtin_bit_cast(bf16x8, q11)};
      reload_mma<VCH, OB, 1>(va, vl1, vh1, pf1, oacc, std::make_integer_sequence<int, OB>{});
    }
    q01 = lds_read_b128_at<1 * 1024>(pr);
    q11 = lds_read_b128_at<3 * 1024>(pr);
    // the copy after the products: 1 % faster than between the two key
    // steps, 2 % faster than before the products (qk 192)
    if (O_DMA && i + PREF < n_wg) issue(i + PREF);
  };
  // Three loops, so that the steady state's body has no branch: with one,
  // the register allocator gave its two paths different homes for the
  // accumulators and spilled them (120-320 registers) at the join.
  int i = 0;
  for (; i < 3 && i < n_wg + 2; ++i) {
    top(i);
    if (O_DMA && i + PREF < n_wg) issue(i + PREF);
    if (i == 2 && n_vis > 0) pv_reads(0);
  }
  for (; i <= n_vis + 1; ++i) {  // the products of tile i - 3, the reads of tile i - 2
    top(i);
    pv_products_reload(i - 2, i);
  }
  for (; i < n_wg + 2; ++i) {
    top(i);
    if (i - 3 < n_vis) pv_products();
    if (O_DMA && i + PREF < n_wg) issue(i + PREF);
  }
  if (n_wg >= 1 && n_wg - 1 < n_vis) {  // the last tile, read in the last iteration
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    pv_products();
  }
  // probabilities within range can still carry huge values of V past the
  // fp32 range: a non-finite accumulator flags the workgroup too
  {
    bool fin = true;
#pragma unroll
    for (int b = 0; b < OB; ++b)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) fin = fin && __builtin_isfinite(oacc[b][rb][i]);
    bad = !fin;
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) s_flag = 1;
  __syncthreads();  // every wave is done with the tiles; flags and row sums are in
  if (s_flag) return;  // the exact pass writes (or merges) these rows
  float inv[RB], lse[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = s_l[s * RW + rb * 32 + n];
    const float mr = s_m[s * RW + rb * 32 + n];
    const bool any = l_tot > 0.f;
    inv[rb] = any ? 1.f / l_tot : 0.f;
    lse[rb] = any ? (mr + log2f(l_tot)) * kLn2 : -INFINITY;
  }
  // O^T -> LDS (wave-private staging) -> whole output rows
  constexpr int OSZ = 4;
  constexpr int OPITCH = DV * OSZ + 16;
  static_assert(4 * 32 * OPITCH <= NBUF * C::STAGE * 16, "staging fits the stages");
  char *ost = (char *)sm + s * 32 * OPITCH;
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int b = 0; b < OB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 x = make_float4(oacc[b][rb][4 * g] * inv[rb], oacc[b][rb][4 * g + 1] * inv[rb],
                               oacc[b][rb][4 * g + 2] * inv[rb], oacc[b][rb][4 * g + 3] * inv[rb]);
        *(float4 *)(ost + n * OPITCH + (32 * b + 8 * g + 4 * hf) * OSZ) = x;
      }
    if (hf == 0) s_lse[s * 32 + n] = lse[rb];
    if (!p.accumulate && hf == 0 && valid[rb]) {
      const int64_t orow = (int64_t)sd.o_begin + row0 + wrow + rb * 32 + n;
      p.lse[orow * p.lse_rs + h] = lse[rb];
    }
    constexpr int LPR = DV / 8;
    constexpr int RPI = 64 / LPR;
    const int sub = lane % LPR, rsub = lane / LPR;
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPI) {
      const int r = r0 + rsub;
      const int rr = wrow + rb * 32 + r;
      if (rr < rows_here) {
        float4 a = *(const float4 *)(ost + r * OPITCH + sub * 8 * OSZ);
        float4 c = *(const float4 *)(ost + r * OPITCH + sub * 8 * OSZ + 16);
        const int64_t orow = (int64_t)sd.o_begin + row0 + rr;
        if (p.accumulate && !merge_into(p, orow, h, sub * 8, s_lse[s * 32 + r], sub == 0, a, c))
          continue;
        if (p.o_bf16) {
          u32x4 v;
          v[0] = pack_bf16(a.x, a.y);
          v[1] = pack_bf16(a.z, a.w);
          v[2] = pack_bf16(c.x, c.y);
          v[3] = pack_bf16(c.z, c.w);
          *(u32x4 *)((__bf16 *)p.o + orow * p.o_rs + (int64_t)h * p.o_hs + sub * 8) = v;
        } else {
          float *op = (float *)p.o + orow * p.o_rs + (int64_t)h * p.o_hs + sub * 8;
          *(float4 *)op = a;
          *(float4 *)(op + 4) = c;
        }
      }
    }
  }
}

// main pass, then the exact pass over the workgroups it flagged
template <int DQK, int DV, int RB>
hipError_t launch_rb(const AttnParams &p, const LaunchSegs &L, hipStream_t stream) {
  const dim3 grid((unsigned)(L.num_tiles * p.hq / p.pack));
  // the split-role main pass for 256-row workgroups at qk 192 and 128
  // (measured 9-10 % faster than the one-wave kernel at both)
  if constexpr (RB == 2 && (DQK == 192 || DQK == 128))
    hipLaunchKernelGGL((attn_fwd_bf16_split_kernel<DQK, DV>), grid, dim3(512), 0, stream, p, L);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, RB, false>), grid, dim3(NT), 0, stream, p, L);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, RB, true>), grid, dim3(NT), 0, stream, p, L);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch(const AttnParams &p, const LaunchSegs &L, int tile_rows, hipStream_t stream) {
  if (tile_rows == 32 * NW) return launch_rb<DQK, DV, 1>(p, L, stream);
  if (tile_rows == 64 * NW) return launch_rb<DQK, DV, 2>(p, L, stream);
  return hipErrorInvalidValue;
}

}  // namespace

int attn_bf16_tile_rows(int, int, bool small) { return small ? 32 * NW : 64 * NW; }

hipError_t launch_attn_bf16(const AttnParams &p, const LaunchSegs &L, int dqk, int dv,
                            int tile_rows, hipStream_t stream) {
  if (dqk == 128 && dv == 128) return launch<128, 128>(p, L, tile_rows, stream);
  if (dqk == 192 && dv == 128) return launch<192, 128>(p, L, tile_rows, stream);
  if (dqk == 64 && dv == 64) return launch<64, 64>(p, L, tile_rows, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn

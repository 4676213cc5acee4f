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
// Structure of one workgroup (4 waves, 256 threads):
//   * a tile of 128 query rows of one segment and one query head; wave w
//     owns rows 32w..32w+31 and keeps their Q fragments in registers;
//   * the keys are visited in tiles of 64: K and V of the tile are staged in
//     LDS (V transposed, see below), the next tile's global loads are in
//     flight while the current one is computed;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with keys as the M dimension
//     and query rows as N, so every lane holds scores of ONE query row
//     (lane % 32) for 32 of the 64 keys; the row max and the exponentials
//     stay lane-local except for one exchange with lane ^ 32;
//   * online softmax in fp32 with exp2 and scale*log2(e) folded in;
//   * O^T += V^T P^T on the same MFMA with dv as M, keys as the contraction
//     and query rows as N: P leaves the score registers as the B operand
//     with no data movement, because the MFMA's B layout (lane % 32 = column)
//     matches the accumulator layout of S^T.  The contraction order of the
//     keys inside each 16-key step is the accumulator's order; V^T is stored
//     in LDS in that same order, so its A operand is one 16-byte LDS read.
//   * tiles are classified per wave from their endpoint positions: fully
//     visible (no mask), fully hidden (skipped), or on the diagonal (mask).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int NT = 256;   // threads
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kNoPos = -(1 << 30);  // position of a padding row: sees nothing

__device__ inline void map_work(int id, int num_tiles, int hq, int hkv,
                                int &tile_order, int &h) {
  // All work of one KV head goes to one XCD queue (id % 8) so that the
  // workgroups streaming the same K/V share that XCD's L2; within a KV head
  // the heaviest tiles come first.
  const int G = hq / hkv;
  const int per_kvh = num_tiles * G;
  int kvh, rem;
  if (hkv % kNumXcd == 0) {
    const int x = id % kNumXcd, slot = id / kNumXcd;
    kvh = x + kNumXcd * (slot / per_kvh);
    rem = slot % per_kvh;
  } else {
    kvh = id / per_kvh;
    rem = id % per_kvh;
  }
  tile_order = rem / G;
  h = kvh * G + rem % G;
}

__device__ inline int find_seg(const LaunchSegs &L, int tile_order) {
  int si = 0;
  for (int i = 1; i < L.num_segs; ++i)
    if (tile_order >= L.s[i].tile_begin) si = i;
  return si;
}

__device__ inline float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ inline uint32_t pack_bf16(float a, float b) {
  const __bf16 lo = (__bf16)a, hi = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <int DQK, int DV>
struct Smem {
  static constexpr int KP = DQK + 8;  // K row pitch (elements), 16B aligned
  static constexpr int VP = BN + 8;   // V^T row pitch (elements)
  __bf16 k[BN * KP];
  __bf16 vt[DV * VP];
  int kpos[BN];
};

template <int DQK, int DV>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT),
                          amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(const AttnParams p, const LaunchSegs L) {
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims");
  constexpr int KP = Smem<DQK, DV>::KP;
  constexpr int VP = Smem<DQK, DV>::VP;
  constexpr int KCH = DQK / 8;              // 16B chunks per K row
  constexpr int KLD = (BN * KCH) / NT;      // K chunks per thread
  static_assert((BN * KCH) % NT == 0, "K staging");
  constexpr int VPAIRS = (BN / 4) * (DV / 8);  // (4 keys x 8 dv) groups
  static_assert(VPAIRS <= NT, "V staging");
  constexpr int QS = DQK / 16;              // MFMA k-steps for S
  constexpr int OB = DV / 32;               // 32-wide dv blocks of O

  __shared__ __attribute__((aligned(16))) Smem<DQK, DV> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n = lane & 31, hf = lane >> 5;

  int tile_order, h;
  map_work(blockIdx.x, L.num_tiles, p.hq, p.hkv, tile_order, h);
  if (tile_order >= L.num_tiles) return;
  const SegDesc sd = L.s[find_seg(L, tile_order)];
  const int ntile = (sd.q_len + BM - 1) / BM;
  const int t = ntile - 1 - (tile_order - sd.tile_begin);
  const int row0 = t * BM;
  const int rows_here = min(BM, sd.q_len - row0);
  const int kvh = h / (p.hq / p.hkv);

  // ---- this lane's query row
  const int rr = w * 32 + n;
  const bool valid = rr < rows_here;
  const int64_t qrow = (int64_t)sd.q_begin + row0 + rr;
  const int qpos = valid ? sd.pos_begin + (row0 + rr) * sd.pos_stride : kNoPos;
  const int nvalid_w = max(0, min(32, rows_here - w * 32));
  const int qmin_w = nvalid_w ? sd.pos_begin + (row0 + w * 32) * sd.pos_stride : kNoPos;
  const int qmax_w =
      nvalid_w ? sd.pos_begin + (row0 + w * 32 + nvalid_w - 1) * sd.pos_stride : kNoPos;
  const int qmax_wg = sd.pos_begin + (row0 + rows_here - 1) * sd.pos_stride;

  bf16x8 qf[QS];
  {
    const __bf16 *qp = (const __bf16 *)p.q + qrow * p.q_rs + (int64_t)h * p.q_hs + 8 * hf;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (valid) x = *(const u32x4 *)(qp + 16 * s);
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int n_kv = sd.kv_len;
  const int32_t *kvp = p.kv_pos ? p.kv_pos + sd.kv_begin : nullptr;
  auto key_pos = [&](int j) -> int { return kvp ? kvp[j] : j; };
  auto tile_live = [&](int j0) -> bool {
    return j0 < n_kv && (!p.causal || key_pos(j0) <= qmax_wg);
  };

  const __bf16 *kbase = (const __bf16 *)p.k + (int64_t)sd.kv_begin * p.k_rs + (int64_t)kvh * p.k_hs;
  const __bf16 *vbase = (const __bf16 *)p.v + (int64_t)sd.kv_begin * p.v_rs + (int64_t)kvh * p.v_hs;

  // ---- staging registers for the next tile
  u32x4 kreg[KLD];
  u32x4 vreg[4];
  int preg = INT_MAX;
  const int vdc = tid / 16, vkc = tid % 16;  // V group: dv 8*vdc.., keys 4*vkc..
  const bool vthread = tid < VPAIRS;

  auto load_tile = [&](int j0) {
#pragma unroll
    for (int c = 0; c < KLD; ++c) {
      const int ch = tid + NT * c;
      const int kr = ch / KCH, kc = ch % KCH;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j0 + kr < n_kv) x = *(const u32x4 *)(kbase + (int64_t)(j0 + kr) * p.k_rs + kc * 8);
      kreg[c] = x;
    }
    if (vthread) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + vkc * 4 + i;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (j < n_kv) x = *(const u32x4 *)(vbase + (int64_t)j * p.v_rs + vdc * 8);
        vreg[i] = x;
      }
    }
    if (tid < BN) preg = (j0 + tid < n_kv) ? key_pos(j0 + tid) : INT_MAX;
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < KLD; ++c) {
      const int ch = tid + NT * c;
      const int kr = ch / KCH, kc = ch % KCH;
      *(u32x4 *)&sm.k[kr * KP + kc * 8] = kreg[c];
    }
    if (vthread) {
      // 4 keys x 8 dv -> for each dv, the 4 keys as one 8-byte LDS write.
      // Keys go to the accumulator order of a 16-key MFMA step: the 4-key
      // chunks 0,1,2,3 of each 16 keys are stored at chunk slots 0,2,1,3.
      const int g16 = vkc >> 2, c4 = vkc & 3;
      const int slot = g16 * 16 + (((c4 & 1) << 1) | (c4 >> 1)) * 4;
#pragma unroll
      for (int d2 = 0; d2 < 4; ++d2) {
        const uint32_t a0 = vreg[0][d2], a1 = vreg[1][d2], a2 = vreg[2][d2], a3 = vreg[3][d2];
        u32x2 lo, hi;  // dv = 2*d2 (low halves) and 2*d2+1 (high halves)
        lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
        lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
        hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
        hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
        const int dv0 = vdc * 8 + 2 * d2;
        *(u32x2 *)&sm.vt[dv0 * VP + slot] = lo;
        *(u32x2 *)&sm.vt[(dv0 + 1) * VP + slot] = hi;
      }
    }
    if (tid < BN) sm.kpos[tid] = preg;
  };

  f32x16 oacc[OB];
#pragma unroll
  for (int b = 0; b < OB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
  float m_run = -INFINITY;  // running max (log2 units), same in both halves
  float l_run = 0.f;        // this half's partial row sum

  const float sl2 = p.scale_log2;
  int j0 = 0;
  bool live = tile_live(0);
  if (live) load_tile(0);
  while (live) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    const int jn = j0 + BN;
    const bool live_next = tile_live(jn);
    if (live_next) load_tile(jn);

    // classify this tile for this wave
    const int jlast = min(j0 + BN, n_kv) - 1;
    const int kmin = sm.kpos[0];
    const int kmax = sm.kpos[jlast - j0];
    const bool hidden = nvalid_w == 0 || (p.causal && kmin > qmax_w);
    const bool full = (j0 + BN <= n_kv) && (!p.causal || kmax <= qmin_w);
    if (!hidden) {
      f32x16 s[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[nb][i] = 0.f;
        const __bf16 *kp = &sm.k[(32 * nb + n) * KP + 8 * hf];
#pragma unroll
        for (int st = 0; st < QS; ++st) {
          const bf16x8 a = *(const bf16x8 *)(kp + 16 * st);
          s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[nb], 0, 0, 0);
        }
      }
      // scores -> log2 units, mask, row max
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float u = s[nb][i] * sl2;
          if (!full) {
            const int kj = 32 * nb + 8 * (i >> 2) + 4 * hf + (i & 3);
            const bool vis = (j0 + kj < n_kv) && (!p.causal || sm.kpos[kj] <= qpos);
            u = vis ? u : -INFINITY;
          }
          s[nb][i] = u;
          mx = fmaxf(mx, u);
        }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      m_run = m_new;
      float ls = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = exp2f(s[nb][8 * c + 2 * e] - m_use);
            const float p1 = exp2f(s[nb][8 * c + 2 * e + 1] - m_use);
            ls += p0 + p1;
            pk[e] = pack_bf16(p0, p1);
          }
          pf[2 * nb + c] = __builtin_bit_cast(bf16x8, pk);
        }
      l_run = l_run * alpha + ls;
#pragma unroll
      for (int b = 0; b < OB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
#pragma unroll
      for (int b = 0; b < OB; ++b) {
        const __bf16 *vp = &sm.vt[(32 * b + n) * VP + 8 * hf];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a = *(const bf16x8 *)(vp + 16 * ks);
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], oacc[b], 0, 0, 0);
        }
      }
    }
    j0 = jn;
    live = live_next;
  }

  // ---- epilogue: combine the two halves' sums, normalise, write
  const float l_tot = l_run + xor32(l_run);
  if (!valid) return;
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  if (hf == 0)
    p.lse[qrow * p.lse_rs + h] = any ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  if (p.o_bf16) {
    __bf16 *op = (__bf16 *)p.o + qrow * p.o_rs + (int64_t)h * p.o_hs + 4 * hf;
#pragma unroll
    for (int b = 0; b < OB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 x;
        x[0] = pack_bf16(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv);
        x[1] = pack_bf16(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
        *(u32x2 *)(op + 32 * b + 8 * g) = x;
      }
  } else {
    float *op = (float *)p.o + qrow * p.o_rs + (int64_t)h * p.o_hs + 4 * hf;
#pragma unroll
    for (int b = 0; b < OB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 x = make_float4(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv,
                               oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
        *(float4 *)(op + 32 * b + 8 * g) = x;
      }
  }
}

template <int DQK, int DV>
hipError_t launch(const AttnParams &p, const LaunchSegs &L, hipStream_t stream) {
  const dim3 grid((unsigned)(L.num_tiles * p.hq));
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV>), grid, dim3(NT), 0, stream, p, L);
  return hipGetLastError();
}

}  // namespace

int attn_bf16_tile_rows(int, int) { return BM; }

hipError_t launch_attn_bf16(const AttnParams &p, const LaunchSegs &L, int dqk,
                            int dv, hipStream_t stream) {
  if (dqk == 128 && dv == 128) return launch<128, 128>(p, L, stream);
  if (dqk == 192 && dv == 128) return launch<192, 128>(p, L, stream);
  if (dqk == 64 && dv == 64) return launch<64, 64>(p, L, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn

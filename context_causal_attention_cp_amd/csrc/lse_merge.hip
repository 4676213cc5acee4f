// Log-sum-exp merge of partial attention results.
//
// "What is Context Parallelism" (blog), section 3.6: the ring rounds (pass-KV)
// and the KV shards (pass-Q, decode CP) each give a normalised partial O_j
// with its log-sum L_j, and the exact result is their merge: the online
// softmax's rescaling applied to whole partial results.  Per (row, head):
//   m = max_j L_j,  w_j = exp(L_j - m),  O = sum_j w_j O_j / sum_j w_j,
//   L = m + ln sum_j w_j.
// A partial with L_j = -inf has w_j = 0 and its O_j is never read.
//
// Bandwidth-bound.  A workgroup takes PPB consecutive (row, head) pairs at a
// time; dv/8 lanes own one pair, 8 output elements per lane:
//   1. the P x PPB log-sums are read once, coalesced, into LDS (one lane per
//      value);
//   2. every lane reads the log-sums of its pair from LDS (broadcast), issues
//      the loads of all live partials back to back (16 B per lane per bf16
//      partial, 32 B per fp32 partial; streamed, not kept in cache) and
//      writes its 8 outputs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;
constexpr int PMAX = 16;   // partials handled per LDS pass
constexpr int PCHUNK = 8;  // partials whose loads are in flight together

// one lane's 8 elements of partial j: raw bits (bf16: 4 words; fp32: 8 words)
template <bool IN_BF16>
struct Raw8 {
  u32x4 a, b;
};
template <bool IN_BF16>
__device__ inline void load8(const void *base, int64_t off, Raw8<IN_BF16> &r) {
  if (IN_BF16) {
    r.a = __builtin_nontemporal_load((const u32x4 *)((const __bf16 *)base + off));
  } else {
    r.a = __builtin_nontemporal_load((const u32x4 *)((const float *)base + off));
    r.b = __builtin_nontemporal_load((const u32x4 *)((const float *)base + off + 4));
  }
}
template <bool IN_BF16>
__device__ inline void fma8(float w, const Raw8<IN_BF16> &r, float (&acc)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (IN_BF16) {
      acc[2 * i] = fmaf(w, __uint_as_float(r.a[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(w, __uint_as_float(r.a[i] & 0xffff0000u), acc[2 * i + 1]);
    } else {
      acc[i] = fmaf(w, __uint_as_float(r.a[i]), acc[i]);
      acc[4 + i] = fmaf(w, __uint_as_float(r.b[i]), acc[4 + i]);
    }
  }
}

__device__ inline uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// One workgroup pass: pairs base .. base + PPB - 1 (those below `pairs`).
// LPP = dv / 8 lanes per pair, PPB = NT / LPP pairs per workgroup pass.
template <int LPP, bool IN_BF16, bool OUT_BF16>
__device__ inline void merge_pass(float (&s_l)[PMAX][NT / LPP], int32_t parts, int64_t pairs,
                                  int64_t base, const void *__restrict__ o_parts,
                                  int64_t o_part_stride, const float *__restrict__ lse_parts,
                                  int64_t lse_part_stride, void *__restrict__ o_out,
                                  float *__restrict__ lse_out) {
  constexpr int PPB = NT / LPP;
  constexpr int DV = 8 * LPP;
  const int tid = threadIdx.x;
  const int sub = tid % LPP, k = tid / LPP;  // lane in pair, pair in the pass
  const int64_t pr = base + k;
  const int64_t off = pr * DV + sub * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f, m = -INFINITY;
  for (int p0 = 0; p0 < parts; p0 += PMAX) {
    const int np = min(PMAX, parts - p0);
    // 1. log-sums of this pass, one lane per value
    __syncthreads();  // the previous pass is done with s_l
    for (int i = tid; i < np * PPB; i += NT) {
      const int j = i / PPB, kk = i % PPB;
      const int64_t q = base + kk;
      s_l[j][kk] = q < pairs ? lse_parts[(int64_t)(p0 + j) * lse_part_stride + q] : -INFINITY;
    }
    __syncthreads();
    float mp = -INFINITY;
    for (int j = 0; j < np; ++j) mp = fmaxf(mp, s_l[j][k]);
    // rescale what earlier passes accumulated (more than PMAX partials)
    const float m_new = fmaxf(m, mp);
    if (m_new != -INFINITY && m != m_new) {
      const float a = (m == -INFINITY) ? 0.f : __expf(m - m_new);
      wsum *= a;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= a;
      m = m_new;
    }
    // 2. live partials of this pass, PCHUNK loads in flight
    if (m != -INFINITY) {
      for (int j0 = 0; j0 < np; j0 += PCHUNK) {
        float w[PCHUNK];
        Raw8<IN_BF16> x[PCHUNK];
#pragma unroll
        for (int c = 0; c < PCHUNK; ++c) {
          const int j = j0 + c;
          const float lj = j < np ? s_l[j][k] : -INFINITY;
          w[c] = (lj == -INFINITY) ? 0.f : __expf(lj - m);
          if (w[c] != 0.f) load8<IN_BF16>(o_parts, (int64_t)(p0 + j) * o_part_stride + off, x[c]);
        }
#pragma unroll
        for (int c = 0; c < PCHUNK; ++c) {
          if (w[c] != 0.f) {
            wsum += w[c];
            fma8<IN_BF16>(w[c], x[c], acc);
          }
        }
      }
    }
  }
  if (pr < pairs) {
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (OUT_BF16) {
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = pack_bf16(acc[2 * i] * inv, acc[2 * i + 1] * inv);
      __builtin_nontemporal_store(v, (u32x4 *)((__bf16 *)o_out + off));
    } else {
      float *op = (float *)o_out + off;
      __builtin_nontemporal_store(
          (u32x4){__float_as_uint(acc[0] * inv), __float_as_uint(acc[1] * inv),
                  __float_as_uint(acc[2] * inv), __float_as_uint(acc[3] * inv)},
          (u32x4 *)op);
      __builtin_nontemporal_store(
          (u32x4){__float_as_uint(acc[4] * inv), __float_as_uint(acc[5] * inv),
                  __float_as_uint(acc[6] * inv), __float_as_uint(acc[7] * inv)},
          (u32x4 *)(op + 4));
    }
    if (lse_out && sub == 0) lse_out[pr] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
  }
}

template <int LPP, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(NT) void lse_merge_kernel(
    int32_t parts, int64_t pairs, const void *__restrict__ o_parts, int64_t o_part_stride,
    const float *__restrict__ lse_parts, int64_t lse_part_stride, void *__restrict__ o_out,
    float *__restrict__ lse_out) {
  constexpr int PPB = NT / LPP;
  __shared__ float s_l[PMAX][PPB];  // log-sums of the pass, [partial][pair]
  for (int64_t base = (int64_t)blockIdx.x * PPB; base < pairs; base += (int64_t)gridDim.x * PPB)
    merge_pass<LPP, IN_BF16, OUT_BF16>(s_l, parts, pairs, base, o_parts, o_part_stride, lse_parts,
                                       lse_part_stride, o_out, lse_out);
}

// Several independent merges in one launch (the key-split segments of an
// attention call): segment i owns workgroups wg_begin[i] .. wg_begin[i+1] - 1
// of the launch, each a pass over PPB of its pairs; its partial j of pair x
// is at (j * part_stride + src[i] + x), its output at (dst[i] + x).
template <int LPP, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(NT) void lse_merge_segs_kernel(
    const MergeSegs T, const void *__restrict__ o_parts, int64_t part_stride,
    const float *__restrict__ lse_parts, void *__restrict__ o_out, float *__restrict__ lse_out) {
  constexpr int PPB = NT / LPP;
  constexpr int DV = 8 * LPP;
  constexpr int ELT_IN = IN_BF16 ? 2 : 4, ELT_OUT = OUT_BF16 ? 2 : 4;
  __shared__ float s_l[PMAX][PPB];
  const int32_t total = T.wg_begin[T.n];
  for (int32_t v = blockIdx.x; v < total; v += gridDim.x) {
    int i = 0;
    while (v >= T.wg_begin[i + 1]) ++i;  // wave-uniform, at most kMaxMergeSegs steps
    const int64_t base = (int64_t)(v - T.wg_begin[i]) * PPB;
    merge_pass<LPP, IN_BF16, OUT_BF16>(
        s_l, T.parts[i], T.pairs[i], base,
        (const char *)o_parts + T.src[i] * DV * ELT_IN, part_stride * DV, lse_parts + T.src[i],
        part_stride, (char *)o_out + T.dst[i] * DV * ELT_OUT, lse_out + T.dst[i]);
  }
}

template <int LPP, bool I, bool O>
hipError_t launch(int32_t parts, int64_t pairs, const void *o_parts, int64_t ops,
                  const float *lse_parts, int64_t lps, void *o_out, float *lse_out,
                  hipStream_t stream) {
  constexpr int PPB = NT / LPP;
  int64_t blocks = (pairs + PPB - 1) / PPB;
  // one pass per workgroup up to a generous cap; beyond it a grid-stride loop
  const int64_t cap = 1 << 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((lse_merge_kernel<LPP, I, O>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                     parts, pairs, o_parts, ops, lse_parts, lps, o_out, lse_out);
  return hipGetLastError();
}

template <int LPP>
hipError_t launch_dtypes(int32_t parts, int64_t pairs, const void *o_parts, int part_bf16,
                         int64_t ops, const float *lse_parts, int64_t lps, void *o_out,
                         int out_bf16, float *lse_out, hipStream_t stream) {
  if (part_bf16 && out_bf16)
    return launch<LPP, true, true>(parts, pairs, o_parts, ops, lse_parts, lps, o_out, lse_out, stream);
  if (part_bf16)
    return launch<LPP, true, false>(parts, pairs, o_parts, ops, lse_parts, lps, o_out, lse_out, stream);
  if (out_bf16)
    return launch<LPP, false, true>(parts, pairs, o_parts, ops, lse_parts, lps, o_out, lse_out, stream);
  return launch<LPP, false, false>(parts, pairs, o_parts, ops, lse_parts, lps, o_out, lse_out, stream);
}

template <int LPP, bool I, bool O>
hipError_t launch_segs(const MergeSegs &T, const void *o_parts, int64_t part_stride,
                       const float *lse_parts, void *o_out, float *lse_out, hipStream_t stream) {
  int64_t blocks = T.wg_begin[T.n];
  const int64_t cap = 1 << 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL((lse_merge_segs_kernel<LPP, I, O>), dim3((unsigned)blocks), dim3(NT), 0,
                     stream, T, o_parts, part_stride, lse_parts, o_out, lse_out);
  return hipGetLastError();
}

}  // namespace

int lse_merge_pairs_per_workgroup(int32_t dv) { return dv >= 8 && dv <= 2048 ? NT / (dv / 8) : 0; }

hipError_t launch_lse_merge_segs(const MergeSegs &T, int32_t dv, const void *o_parts,
                                 int part_bf16, int64_t part_stride, const float *lse_parts,
                                 void *o_out, int out_bf16, float *lse_out, hipStream_t stream) {
#define CP_MERGE_SEGS_DV(L)                                                                  \
  case L:                                                                                    \
    if (part_bf16 && out_bf16)                                                               \
      return launch_segs<L, true, true>(T, o_parts, part_stride, lse_parts, o_out, lse_out,  \
                                        stream);                                             \
    if (part_bf16)                                                                           \
      return launch_segs<L, true, false>(T, o_parts, part_stride, lse_parts, o_out, lse_out, \
                                         stream);                                            \
    if (out_bf16)                                                                            \
      return launch_segs<L, false, true>(T, o_parts, part_stride, lse_parts, o_out, lse_out, \
                                         stream);                                            \
    return launch_segs<L, false, false>(T, o_parts, part_stride, lse_parts, o_out, lse_out,  \
                                        stream);
  switch (dv / 8) {
    CP_MERGE_SEGS_DV(8)
    CP_MERGE_SEGS_DV(16)
    CP_MERGE_SEGS_DV(64)
    default:
      return hipErrorInvalidValue;
  }
#undef CP_MERGE_SEGS_DV
}

hipError_t launch_lse_merge(int32_t parts, int64_t pairs, int32_t dv,
                            const void *o_parts, int part_bf16,
                            int64_t o_part_stride, const float *lse_parts,
                            int64_t lse_part_stride, void *o_out, int out_bf16,
                            float *lse_out, hipStream_t stream) {
#define CP_MERGE_DV(L)                                                                       \
  case L:                                                                                    \
    return launch_dtypes<L>(parts, pairs, o_parts, part_bf16, o_part_stride, lse_parts,      \
                            lse_part_stride, o_out, out_bf16, lse_out, stream);
  switch (dv / 8) {
    CP_MERGE_DV(1)
    CP_MERGE_DV(2)
    CP_MERGE_DV(4)
    CP_MERGE_DV(8)
    CP_MERGE_DV(16)
    CP_MERGE_DV(32)
    CP_MERGE_DV(64)
    CP_MERGE_DV(128)
    CP_MERGE_DV(256)
    default:
      return hipErrorInvalidValue;
  }
#undef CP_MERGE_DV
}

}  // namespace cpattn

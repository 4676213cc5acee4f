// Log-sum-exp merge of partial attention results.
//
// "What is Context Parallelism" (blog), section 3.6: the ring rounds (pass-KV)
// and the KV shards (pass-Q, decode CP) each give a normalised partial O_j
// with its log-sum L_j, and the exact result is their merge, the
// generalisation of the online softmax.  Per (row, head):
//   m = max_j L_j,  w_j = exp(L_j - m),  O = sum_j w_j O_j / sum_j w_j,
//   L = m + ln sum_j w_j.
// A partial with L_j = -inf has w_j = 0 and its O_j is never read.
//
// Bandwidth-bound.  A group of dv/8 lanes owns one (row, head): every lane
// holds 8 output elements, reads the P log-sums (one cache line shared by
// the group), issues the loads of all live partials back to back (16 B per
// lane per bf16 partial, 32 B per fp32 partial), and writes 8 outputs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;
constexpr int PCHUNK = 8;  // partials whose loads are in flight together

template <bool IN_BF16>
__device__ inline void load8(const void *base, int64_t off, float (&x)[8]) {
  if (IN_BF16) {
    const u32x4 v = *(const u32x4 *)((const __bf16 *)base + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[i] << 16);
      x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *(const float4 *)((const float *)base + off);
    const float4 b = *(const float4 *)((const float *)base + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

__device__ inline uint32_t pack_bf16(float a, float b) {
  const __bf16 lo = (__bf16)a, hi = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(NT) void lse_merge_kernel(
    int32_t parts, int64_t pairs, int32_t dv, const void *__restrict__ o_parts,
    int64_t o_part_stride, const float *__restrict__ lse_parts,
    int64_t lse_part_stride, void *__restrict__ o_out, float *__restrict__ lse_out) {
  const int lanes_per_pair = dv / 8;
  const int pairs_per_block = NT / lanes_per_pair;
  const int sub = threadIdx.x % lanes_per_pair;
  const int64_t pair0 = (int64_t)blockIdx.x * pairs_per_block + threadIdx.x / lanes_per_pair;
  const int64_t pstride = (int64_t)gridDim.x * pairs_per_block;

  for (int64_t pr = pair0; pr < pairs; pr += pstride) {
    float m = -INFINITY;
    for (int j = 0; j < parts; ++j) m = fmaxf(m, lse_parts[j * lse_part_stride + pr]);
    const int64_t off = pr * dv + sub * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != -INFINITY) {
      for (int j0 = 0; j0 < parts; j0 += PCHUNK) {
        float w[PCHUNK];
        float x[PCHUNK][8];
#pragma unroll
        for (int c = 0; c < PCHUNK; ++c) {
          const int j = j0 + c;
          const float lj = j < parts ? lse_parts[j * lse_part_stride + pr] : -INFINITY;
          w[c] = (lj == -INFINITY) ? 0.f : expf(lj - m);
          if (w[c] != 0.f) load8<IN_BF16>(o_parts, j * o_part_stride + off, x[c]);
        }
#pragma unroll
        for (int c = 0; c < PCHUNK; ++c) {
          if (w[c] != 0.f) {
            wsum += w[c];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[c], x[c][i], acc[i]);
          }
        }
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (OUT_BF16) {
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = pack_bf16(acc[2 * i] * inv, acc[2 * i + 1] * inv);
      *(u32x4 *)((__bf16 *)o_out + off) = v;
    } else {
      float *op = (float *)o_out + off;
      *(float4 *)op = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      *(float4 *)(op + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    }
    if (lse_out && sub == 0) lse_out[pr] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
  }
}

template <bool I, bool O>
hipError_t launch(int32_t parts, int64_t pairs, int32_t dv, const void *o_parts,
                  int64_t ops, const float *lse_parts, int64_t lps, void *o_out,
                  float *lse_out, hipStream_t stream) {
  const int ppb = NT / (dv / 8);
  int64_t blocks = (pairs + ppb - 1) / ppb;
  // enough workgroups to cover the chip several times; the rest is a
  // grid-stride loop
  const int64_t cap = 256 * 64;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((lse_merge_kernel<I, O>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                     parts, pairs, dv, o_parts, ops, lse_parts, lps, o_out, lse_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(int32_t parts, int64_t pairs, int32_t dv,
                            const void *o_parts, int part_bf16,
                            int64_t o_part_stride, const float *lse_parts,
                            int64_t lse_part_stride, void *o_out, int out_bf16,
                            float *lse_out, hipStream_t stream) {
  if (part_bf16 && out_bf16)
    return launch<true, true>(parts, pairs, dv, o_parts, o_part_stride, lse_parts,
                              lse_part_stride, o_out, lse_out, stream);
  if (part_bf16 && !out_bf16)
    return launch<true, false>(parts, pairs, dv, o_parts, o_part_stride, lse_parts,
                               lse_part_stride, o_out, lse_out, stream);
  if (!part_bf16 && out_bf16)
    return launch<false, true>(parts, pairs, dv, o_parts, o_part_stride, lse_parts,
                               lse_part_stride, o_out, lse_out, stream);
  return launch<false, false>(parts, pairs, dv, o_parts, o_part_stride, lse_parts,
                              lse_part_stride, o_out, lse_out, stream);
}

}  // namespace cpattn

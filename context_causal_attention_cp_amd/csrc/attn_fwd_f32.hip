// Causal varlen attention forward in fp32 (fp32 in, fp32 math).
//
// Same operation as the bf16 kernel ("What is Context Parallelism" blog,
// sections 2.1 and 3.1; GQA section 4.1), for fp32 inputs where the result
// must stay within fp32 rounding of the exact value.  One wavefront handles
// 64 query rows of one head; each lane owns one row (q and the output
// accumulator live in its registers) and walks the visible keys, which are
// staged 32 at a time in LDS and read as broadcasts.  Exponentials use expf.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

constexpr int BM = 64;
constexpr int BN = 32;
constexpr int kNoPos = -(1 << 30);

__device__ inline void map_work_f32(int id, int num_tiles, int hq, int &tile_order, int &h) {
  h = id % hq;
  tile_order = id / hq;
}

template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(const AttnParams p, const LaunchSegs L) {
  __shared__ float sk[BN][D];
  __shared__ float sv[BN][D];
  __shared__ int skp[BN];

  const int lane = threadIdx.x;
  int tile_order, h;
  map_work_f32(blockIdx.x, L.num_tiles, p.hq, tile_order, h);
  if (tile_order >= L.num_tiles) return;
  int si = 0;
  for (int i = 1; i < L.num_segs; ++i)
    if (tile_order >= L.s[i].tile_begin) si = i;
  const SegDesc sd = L.s[si];
  const int ntile = (sd.q_len + BM - 1) / BM;
  const int t = ntile - 1 - (tile_order - sd.tile_begin);
  const int row0 = t * BM;
  const int rows_here = min(BM, sd.q_len - row0);
  const int kvh = h / (p.hq / p.hkv);

  const bool valid = lane < rows_here;
  const int64_t qrow = (int64_t)sd.q_begin + row0 + lane;
  const int64_t orow = (int64_t)sd.o_begin + row0 + lane;  // output row
  const int qpos = valid ? sd.pos_begin + (row0 + lane) * sd.pos_stride : kNoPos;
  const int qmax = sd.pos_begin + (row0 + rows_here - 1) * sd.pos_stride;

  float q[D], o[D];
  const float *qp = (const float *)p.q + qrow * p.q_rs + (int64_t)h * p.q_hs;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? qp[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int n_kv = sd.kv_len;
  const int32_t *kvp = p.kv_pos ? p.kv_pos + sd.kv_begin : nullptr;
  const float *kb = (const float *)p.k + (int64_t)sd.kv_begin * p.k_rs + (int64_t)kvh * p.k_hs;
  const float *vb = (const float *)p.v + (int64_t)sd.kv_begin * p.v_rs + (int64_t)kvh * p.v_hs;

  for (int j0 = 0; j0 < n_kv; j0 += BN) {
    const int first = kvp ? kvp[j0] : j0;
    if (p.causal && first > qmax) break;
    __syncthreads();
    for (int e = lane; e < BN * D; e += 64) {
      const int r = e / D, d = e % D;
      const bool in = j0 + r < n_kv;
      sk[r][d] = in ? kb[(int64_t)(j0 + r) * p.k_rs + d] : 0.f;
      sv[r][d] = in ? vb[(int64_t)(j0 + r) * p.v_rs + d] : 0.f;
    }
    if (lane < BN) skp[lane] = (j0 + lane < n_kv) ? (kvp ? kvp[j0 + lane] : j0 + lane) : INT_MAX;
    __syncthreads();
    for (int j = 0; j < BN; ++j) {
      if (j0 + j >= n_kv) break;
      if (p.causal && skp[j] > qpos) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], sk[j][d], s);
      s *= p.scale;
      if (s > m) {
        const float a = expf(m - s);  // m = -inf on the first key: a = 0
        l *= a;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= a;
        m = s;
      }
      const float e = expf(s - m);
      l += e;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(e, sv[j][d], o[d]);
    }
  }
  if (!valid) return;
  const bool any = l > 0.f;
  float inv = any ? 1.f / l : 0.f;
  float lse = any ? m + logf(l) : -INFINITY;
  if (p.accumulate) {
    // merge into the running (O, LSE) of this row: an empty new partial
    // leaves it; an empty accumulator (LSE = -inf) is replaced
    if (!any) return;
    const float la = p.lse[orow * p.lse_rs + h];
    if (la != -INFINITY) {
      const float mm = fmaxf(la, lse);
      const float wa = expf(la - mm), wn = expf(lse - mm);
      const float winv = 1.f / (wa + wn);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const float oa = p.o_bf16 ? (float)((const __bf16 *)p.o)[orow * p.o_rs + (int64_t)h * p.o_hs + d]
                                  : ((const float *)p.o)[orow * p.o_rs + (int64_t)h * p.o_hs + d];
        o[d] = (wa * oa + wn * o[d] * inv) * winv;
      }
      inv = 1.f;
      lse = mm + logf(wa + wn);
    }
  }
  p.lse[orow * p.lse_rs + h] = lse;
  if (p.o_bf16) {
    __bf16 *op = (__bf16 *)p.o + orow * p.o_rs + (int64_t)h * p.o_hs;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = (__bf16)(o[d] * inv);
  } else {
    float *op = (float *)p.o + orow * p.o_rs + (int64_t)h * p.o_hs;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  }
}

template <int D>
hipError_t launch(const AttnParams &p, const LaunchSegs &L, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3((unsigned)(L.num_tiles * p.hq)),
                     dim3(64), 0, stream, p, L);
  return hipGetLastError();
}

}  // namespace

int attn_f32_tile_rows(int) { return BM; }

hipError_t launch_attn_f32(const AttnParams &p, const LaunchSegs &L, int d,
                           hipStream_t stream) {
  if (d == 64) return launch<64>(p, L, stream);
  if (d == 128) return launch<128>(p, L, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn

// Device gather of rows by an index: the reorder that follows the KV
// all-gather.
//
// "What is Context Parallelism" (blog), section 2.1 (engineering notes) and
// section 5.1: after the all-gather each rank holds the rank-major
// concatenation of every rank's local tokens; gathering it by the restore
// index (restore[g] = slot of flattened new token g) yields causal order.
// dst row i = src row index[i].
//
// HBM-bound copy (loads and stores streamed past the caches; a lane keeps
// eight 16-byte chunks in flight).  A workgroup pass covers 256 / L rows with L lanes per
// row (L = the power of two nearest above the row's 16-byte chunk count,
// capped at 256), so short rows do not leave lanes idle and long rows are
// streamed by the whole workgroup.  Rows whose index is out of range are
// zero-filled (never read out of bounds).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void restore_apply_kernel(const int32_t *__restrict__ index,
                                                           int64_t n, const char *__restrict__ src,
                                                           int64_t src_rows, int64_t src_stride,
                                                           char *__restrict__ dst,
                                                           int64_t dst_stride, int32_t cpr,
                                                           int32_t log2_lanes) {
  const int lanes = 1 << log2_lanes;
  const int rows_per_pass = NT >> log2_lanes;
  const int sub = threadIdx.x & (lanes - 1);
  const int rloc = threadIdx.x >> log2_lanes;
  for (int64_t r0 = (int64_t)blockIdx.x * rows_per_pass; r0 < n;
       r0 += (int64_t)gridDim.x * rows_per_pass) {
    const int64_t r = r0 + rloc;
    if (r >= n) continue;
    const int64_t s = index[r];
    u32x4 *d = (u32x4 *)(dst + r * dst_stride);
    if (s < 0 || s >= src_rows) {
      for (int c = sub; c < cpr; c += lanes) d[c] = (u32x4){0u, 0u, 0u, 0u};
      continue;
    }
    const u32x4 *sp = (const u32x4 *)(src + s * src_stride);
    // eight, then four chunks in flight per lane; streamed (not kept in cache)
    int c = sub;
    for (; c + 7 * lanes < cpr; c += 8 * lanes) {
      u32x4 x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __builtin_nontemporal_load(sp + c + j * lanes);
#pragma unroll
      for (int j = 0; j < 8; ++j) __builtin_nontemporal_store(x[j], d + c + j * lanes);
    }
    for (; c + 3 * lanes < cpr; c += 4 * lanes) {
      u32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = __builtin_nontemporal_load(sp + c + j * lanes);
#pragma unroll
      for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(x[j], d + c + j * lanes);
    }
    for (; c < cpr; c += lanes) __builtin_nontemporal_store(__builtin_nontemporal_load(sp + c), d + c);
  }
}

}  // namespace

hipError_t launch_restore_apply(const int32_t *index, int64_t n, const void *src, int64_t src_rows,
                                int64_t src_stride, void *dst, int64_t dst_stride,
                                int64_t row_bytes, hipStream_t stream) {
  const int32_t cpr = (int32_t)(row_bytes / 16);
  int log2_lanes = 0;
  while ((1 << log2_lanes) < cpr && log2_lanes < 8) ++log2_lanes;
  const int64_t rows_per_pass = NT >> log2_lanes;
  int64_t blocks = (n + rows_per_pass - 1) / rows_per_pass;
  const int64_t cap = 1 << 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(restore_apply_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, index, n,
                     (const char *)src, src_rows, src_stride, (char *)dst, dst_stride, cpr,
                     log2_lanes);
  return hipGetLastError();
}

}  // namespace cpattn

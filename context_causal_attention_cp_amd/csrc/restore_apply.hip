// Device gather of rows by an index: the reorder that follows the KV
// all-gather.
//
// "What is Context Parallelism" (blog), section 2.1 (engineering notes) and
// section 5.1: after the all-gather each rank holds the rank-major
// concatenation of every rank's local tokens; gathering it by the restore
// index (restore[g] = slot of flattened new token g) yields causal order.
// dst row i = src row index[i].
//
// HBM-bound copy, loads and stores streamed past the caches.  The work is
// cut into many one-wave workgroups, each moving one 16-byte chunk per lane:
// a piece of 64 chunks (1 KiB) of a long row, or 64 / L whole short rows of
// L <= 32 chunks each (L a power of two).  Measured on the 131072-row,
// 48 KiB-per-row K gather: 1 KiB per one-wave workgroup moves 6.7 TB/s,
// against 6.4 TB/s for 4 KiB per 256-lane workgroup and 5.4 TB/s for whole
// rows per 256-lane workgroup with eight chunks in flight per lane; finer
// pieces keep more independent requests spread over the memory channels.
// Rows whose index is out of range are zero-filled (never read out of
// bounds).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 64;                 // one wave per workgroup
constexpr int64_t kMaxGrid = 1 << 24;  // beyond: workgroups loop over pieces

// rows of more than 32 chunks: piece = (row, 64-chunk part), parts = ceil(cpr / 64)
__global__ __launch_bounds__(NT) void restore_apply_long_kernel(
    const int32_t *__restrict__ index, int64_t n, const char *__restrict__ src, int64_t src_rows,
    int64_t src_stride, char *__restrict__ dst, int64_t dst_stride, int32_t cpr, int32_t parts) {
  const int64_t pieces = n * parts;
  const bool narrow = pieces <= (int64_t)UINT32_MAX;  // 32-bit division suffices
  for (int64_t pc = blockIdx.x; pc < pieces; pc += gridDim.x) {
    const int64_t r = narrow ? (int64_t)((uint32_t)pc / (uint32_t)parts) : pc / parts;
    const int c = (int)(pc - r * parts) * NT + (int)threadIdx.x;
    if (c >= cpr) continue;
    const int64_t s = index[r];
    u32x4 *d = (u32x4 *)(dst + r * dst_stride);
    if (s < 0 || s >= src_rows) {
      d[c] = (u32x4){0u, 0u, 0u, 0u};
      continue;
    }
    const u32x4 *sp = (const u32x4 *)(src + s * src_stride);
    __builtin_nontemporal_store(__builtin_nontemporal_load(sp + c), d + c);
  }
}

// short rows (cpr <= 32): 64 / L rows per workgroup, L = 2^log2_lanes lanes each
__global__ __launch_bounds__(NT) void restore_apply_short_kernel(
    const int32_t *__restrict__ index, int64_t n, const char *__restrict__ src, int64_t src_rows,
    int64_t src_stride, char *__restrict__ dst, int64_t dst_stride, int32_t cpr,
    int32_t log2_lanes) {
  const int rows_per_wg = NT >> log2_lanes;
  const int c = threadIdx.x & ((1 << log2_lanes) - 1);
  const int rloc = threadIdx.x >> log2_lanes;
  for (int64_t r0 = (int64_t)blockIdx.x * rows_per_wg; r0 < n;
       r0 += (int64_t)gridDim.x * rows_per_wg) {
    const int64_t r = r0 + rloc;
    if (r >= n || c >= cpr) continue;
    const int64_t s = index[r];
    u32x4 *d = (u32x4 *)(dst + r * dst_stride);
    if (s < 0 || s >= src_rows) {
      d[c] = (u32x4){0u, 0u, 0u, 0u};
      continue;
    }
    const u32x4 *sp = (const u32x4 *)(src + s * src_stride);
    __builtin_nontemporal_store(__builtin_nontemporal_load(sp + c), d + c);
  }
}

}  // namespace

hipError_t launch_restore_apply(const int32_t *index, int64_t n, const void *src, int64_t src_rows,
                                int64_t src_stride, void *dst, int64_t dst_stride,
                                int64_t row_bytes, hipStream_t stream) {
  const int32_t cpr = (int32_t)(row_bytes / 16);
  if (cpr > NT / 2) {
    const int32_t parts = (cpr + NT - 1) / NT;
    int64_t grid = n * parts;
    if (grid > kMaxGrid) grid = kMaxGrid;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(restore_apply_long_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, index,
                       n, (const char *)src, src_rows, src_stride, (char *)dst, dst_stride, cpr,
                       parts);
  } else {
    int log2_lanes = 0;
    while ((1 << log2_lanes) < cpr) ++log2_lanes;
    const int64_t rows_per_wg = NT >> log2_lanes;
    int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
    if (grid > kMaxGrid) grid = kMaxGrid;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(restore_apply_short_kernel, dim3((unsigned)grid), dim3(NT), 0, stream,
                       index, n, (const char *)src, src_rows, src_stride, (char *)dst, dst_stride,
                       cpr, log2_lanes);
  }
  return hipGetLastError();
}

}  // namespace cpattn

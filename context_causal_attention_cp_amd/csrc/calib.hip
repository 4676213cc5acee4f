// Sustained-rate probes of the GPU the library runs on: a matrix-core loop
// and a device copy.  They measure what this chip reaches at the clock it
// holds under load, so that the attention, merge and decode kernels can be
// reported against a measured ceiling beside the published peaks (bf16 dense
// 2.5 PFLOP/s, HBM 8 TB/s).
//
//   * calib_mfma_kernel: every wave runs `iters` rounds of 8 independent
//     v_mfma_f32_32x32x16_bf16 products on register operands (A = B = bf16
//     ones, so every accumulator element gains exactly 16 per product) and
//     writes the sum of its lane-0 accumulator elements: 8 * 16 * iters,
//     exact in fp32 up to 2^24;
//   * calib_copy_kernel: dst = src in 16-byte units, one 1 KiB piece per
//     one-wave workgroup, streamed past the caches (the launch shape that
//     moved rows fastest in the restore gather).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void calib_mfma_kernel(int32_t iters, float *out) {
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
  bf16x8 a = __builtin_bit_cast(bf16x8, ones);
  // an opaque copy: the products must not be folded at compile time
  asm volatile("" : "+v"(a));
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(64) void calib_copy_kernel(const u32x4 *__restrict__ src,
                                                        u32x4 *__restrict__ dst, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (u < units) __builtin_nontemporal_store(__builtin_nontemporal_load(src + u), dst + u);
}

}  // namespace

hipError_t launch_calib_mfma(int32_t workgroups, int32_t iters, float *out, hipStream_t stream) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, iters, out);
  return hipGetLastError();
}

hipError_t launch_calib_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream) {
  const int64_t units = bytes / 16;
  const int64_t blocks = (units + 63) / 64;
  hipLaunchKernelGGL(calib_copy_kernel, dim3((unsigned)blocks), dim3(64), 0, stream,
                     (const u32x4 *)src, (u32x4 *)dst, units);
  return hipGetLastError();
}

}  // namespace cpattn

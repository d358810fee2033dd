// Calibration: a plain 16-byte streaming copy, used to measure the achievable
// HBM copy rate and to scale the FETCH_SIZE / WRITE_SIZE hardware counters.
#include "spr_device.h"
#include "spr_internal.h"

namespace spr {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void sp_region_copy_kernel(const u32x4* __restrict__ src,
                                                                      u32x4* __restrict__ dst, int64_t n16) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyUnroll + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int k = 0; k < kCopyUnroll; ++k) {
    const int64_t i = base + k * kCopyThreads;
    if (i < n16) v[k] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int k = 0; k < kCopyUnroll; ++k) {
    const int64_t i = base + k * kCopyThreads;
    if (i < n16) dst[i] = v[k];
  }
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, size_t nbytes, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(nbytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t per_block = kCopyThreads * kCopyUnroll;
  const dim3 grid(static_cast<unsigned>((n16 + per_block - 1) / per_block)), block(kCopyThreads);
  hipLaunchKernelGGL(sp_region_copy_kernel, grid, block, 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace spr

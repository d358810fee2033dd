// Calibration: a plain 16-byte streaming copy, used to measure the achievable
// HBM copy rate and to scale the FETCH_SIZE / WRITE_SIZE hardware counters.
#include "spr_device.h"
#include "spr_internal.h"

namespace spr {
namespace {

constexpr int kCopyThreads = 256;

// One 16-byte vector per thread and many short-lived blocks: measured on
// MI355X, the fastest form of a plain copy (6.4 TB/s against 5.5-6.1 TB/s
// for 2-8 vectors per thread).
__global__ __launch_bounds__(kCopyThreads) void sp_region_copy_kernel(const u32x4* __restrict__ src,
                                                                      u32x4* __restrict__ dst, int64_t n16) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  if (i < n16) dst[i] = __builtin_nontemporal_load(src + i);
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, size_t nbytes, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(nbytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = (n16 + kCopyThreads - 1) / kCopyThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;   // grid x limit
  const dim3 grid(static_cast<unsigned>(blocks)), block(kCopyThreads);
  hipLaunchKernelGGL(sp_region_copy_kernel, grid, block, 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace spr

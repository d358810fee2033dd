// Host-side contract between the C ABI (abi.cpp) and the kernel TUs.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spr {

// Profiling hook (sp_region_time_next_call): events the next region call on
// this thread stamps from its kernels' dispatch packets -- start at its first
// kernel, stop at its last.  Cleared by the ABI layer after each call.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
extern thread_local LaunchEvents g_launch_events;

enum class KernelRole { kOnly, kFirst, kLast };

// Every region kernel is launched through here: hipExtLaunchKernelGGL with
// the hook's events (none when the hook is clear).
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t stream, KernelRole role, Args... args) {
  hipEvent_t start = role != KernelRole::kLast ? g_launch_events.start : nullptr;
  hipEvent_t stop = role != KernelRole::kFirst ? g_launch_events.stop : nullptr;
  hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, args...);
}

// Parameters of one forward launch (validated by the ABI layer).
struct FwdParams {
  const void* slab[8];    // slab k: [T][h] of TP rank k's partial (k < t), anywhere in device memory
  const void* bias;       // [h] or null
  const void* residual;   // [T][h] or null
  const void* gamma;      // [h]
  const void* beta;       // [h] or null
  const int32_t* cu;      // [nseq+1] local offsets or null (uniform shard)
  int32_t nseq;
  void* z;                // [T][h]
  void* y;                // [T][h]
  float* mean;            // [T] or null (RMSNorm)
  float* rstd;            // [T]
  uint8_t* mask;          // [T][h] or null
  int64_t T;
  int32_t h;
  int32_t t;
  int32_t rank;
  int32_t norm;           // 0 LayerNorm, 1 RMSNorm
  float eps;
  float scale;            // float32(1/(1-p))
  uint32_t thr;           // floor(p * 2^32); dropout active iff drop != 0
  int32_t drop;
  uint32_t key0, key1;    // lo32 / hi32 of the seed
};

struct BwdParams {
  const void* dy;
  const void* z;
  const float* mean;      // null for RMSNorm
  const float* rstd;
  const void* gamma;
  const void* dres;       // [T][h] or null
  void* dx;
  float* ws;              // [G][nparts][h]
  float* dgamma;
  float* dbeta;           // null allowed
  int64_t T;
  int32_t h;
  int32_t norm;
  int32_t G;
  // Partial slots per block: dgamma in slot 0, dbeta / dbias in slot_dbeta /
  // slot_dbias (0: not computed); strides in floats (set by launch_bwd).
  int32_t nparts;
  int64_t ws_sstride;
  int64_t ws_bstride;
  int32_t slot_dbeta;
  int32_t slot_dbias;
  // Dropout backward (dpartial != null): dpartial = dx * keep * scale and the
  // dbias partials, with the forward's mask parameters.
  void* dpartial;         // [T][h] or null
  float* dbias;           // [h] or null
  const int32_t* cu;      // [nseq+1] local offsets or null (uniform shard)
  int32_t nseq;
  int32_t t;
  int32_t rank;
  int32_t drop;           // p > 0
  uint32_t thr;
  float scale;
  uint32_t key0, key1;
  // Nonzero: dgamma / dbeta / dbias hold float32 main gradients and receive
  // old + sum instead of sum.
  int32_t accumulate;
};

// Number of row blocks of the backward's first stage (and of workspace
// partials): a pure function of (T, h) so the workspace size is known
// without a device query.  256 = one block per MI355X compute unit.
#ifndef SPR_BWD_BLOCKS
#define SPR_BWD_BLOCKS 256
#endif
constexpr int kBwdMaxBlocks = SPR_BWD_BLOCKS;
#ifndef SPR_BWD_MIN_ROWS
#define SPR_BWD_MIN_ROWS 4   // rows per row block on small shards (page_demo backward 16.6 -> 15.8 us)
#endif
inline int64_t bwd_blocks(int64_t T, int64_t /*h*/) {
  const int64_t g = (T + SPR_BWD_MIN_ROWS - 1) / SPR_BWD_MIN_ROWS;
  return g < kBwdMaxBlocks ? g : kBwdMaxBlocks;
}

// Workspace layout of the backward's partials (floats): slot j of block b at
// b*ws_block_stride(h, nslots) + j*ws_slot_stride(h).  Both strides are 1 KiB
// past a multiple of 2 KiB.  Every block writes its partial at the same
// moment and stage 2 reads slot c of every block together; at power-of-two
// strides those accesses are congruent modulo a large power of two and pile
// onto the same HBM channels.
#ifndef SPR_WS_PAD
#define SPR_WS_PAD 1
#endif
inline int64_t ws_round(int64_t floats) {
  return SPR_WS_PAD ? (floats + 511) / 512 * 512 + 256 : floats;
}
inline int64_t ws_slot_stride(int64_t h) { return ws_round(h); }
inline int64_t ws_block_stride(int64_t h, int nslots) { return ws_round(nslots * ws_slot_stride(h)); }
// Whole workspace: the G blocks' partials.
inline int64_t ws_total_bytes(int64_t G, int64_t h, int nslots) { return G * ws_block_stride(h, nslots) * 4; }

// Launchers: return hipSuccess or the launch error.  `dtype` 0 = f32, 1 = bf16.
hipError_t launch_fwd(const FwdParams& p, int dtype, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int dtype, hipStream_t stream);
void set_bwd_launches(int n);   // 1: one launch on small shards (default); 2: always the partials' two
hipError_t launch_copy(const void* src, void* dst, size_t nbytes, hipStream_t stream);

// Launch shapes (exposed for tests of the host logic).
struct Shape {
  int vpt;      // 16-byte vectors per thread per row
  int threads;  // block size, a multiple of 64
};
Shape fwd_shape(int h, int dtype);
Shape bwd_shape(int h, int dtype);

}  // namespace spr

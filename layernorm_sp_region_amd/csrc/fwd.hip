// Forward of the sequence-parallel region: WPR wavefronts per local token row.
//
// Per row (hpc.payai.win lesson 7: g* of section 3.A, LayerNorm of section 2):
//   acc = P_0 + P_1 + ... + P_{t-1}      float32, ascending k (g* arithmetic)
//   acc = acc + bias                      if bias
//   d   = keep ? acc * scale : 0          if p > 0 (Philox-4x32-10 keep bit)
//   z   = round(residual + d)             stored; statistics use the rounded z
//   LayerNorm: mean, population variance (second pass over the packed z),
//              y = (z - mean) * rstd * gamma + beta
//   RMSNorm:   y = z * rstd * gamma, rstd = 1/sqrt(mean(z^2) + eps)
//
// The z chain is compiled without floating-point contraction (the build
// passes -ffp-contract=off) so it matches the float32 operation order
// exactly; the normalisation uses explicit fmaf.
//
// Memory plan.  Lane l of wave w of the row owns the 16-byte vectors
// v = l + 64*(w + WPR*k), k < VPL (VPL slots per lane), so every load
// instruction of a wave reads 1 KB of contiguous row.  The row is streamed
// one slot at a time: the t slab vectors, the residual and the bias of slot
// k+1 are in flight while slot k is summed, masked, rounded and stored.  The
// rounded z stays packed -- in LDS for rows of 8-16 slots per lane (each lane
// reads back only what it wrote, so no barrier), in registers for shorter
// rows -- for the statistics (a second pass) and the y phase, which fetches
// gamma/beta one slot ahead.  Wave sums use DPP row steps plus readlane;
// rows of several waves (WPR = 2 for h above 8192 bf16; 4 on shards of at
// most 1024 rows) combine their sums through LDS in wave order.  Every
// memory instruction is unconditional (see the kernel), and row base
// pointers are wave-uniform (SGPR + 32-bit lane offsets).  Slabs and residual use nontemporal loads; gamma, beta and bias
// (read by every row) ordinary cached loads.  z and y take ordinary stores,
// except on shards whose z and y together exceed the 256 MB Infinity Cache:
// there y is stored nontemporally (YNT), so its lines stream to memory instead
// of evicting dirty data through the caches (measured on the 128K-token
// shard: step 669 -> 631 us; on the 70B shard, whose 67 MB of z and y fit,
// the forward was 1 us slower with it).  z always keeps ordinary stores: the
// backward reads it back (nontemporal z as well: 70B step 97.7 us).
#include "spr_device.h"
#include "spr_internal.h"

namespace spr {
namespace {

// Runtime loop over vector slots (1) or full unrolling (0) when z is in LDS;
// measured: unrolled is ~1 us faster on a 2048 x 8192 shard.
#ifndef SPR_FWD_LOOP
#define SPR_FWD_LOOP 0
#endif
// WPR = 1: independent rows per block.  One: every wave is a block of its
// own, so the dispatcher hands rows to compute units one at a time as they
// free up and the last generation of blocks ends evenly (measured against 4
// rows per block: ragged13b 80.5 -> 76.4 us, long128k 537.1 -> 531.7 us, the
// 70B shard 66.5 -> 66.0 us in the step).
#ifndef SPR_FWD_ROWS_PER_BLOCK
#define SPR_FWD_ROWS_PER_BLOCK 1
#endif
constexpr int kRowsPerBlockW1 = SPR_FWD_ROWS_PER_BLOCK;

// Sum over the WPR waves of a row, in wave order (uniform result).
template <int WPR>
__device__ __forceinline__ float row_total(float x, float* slot) {
  x = wave_total(x);
  if constexpr (WPR == 1) {
    return x;
  } else {
    if ((threadIdx.x & 63) == 0) slot[threadIdx.x / 64] = x;
    __syncthreads();
    float s = slot[0];
#pragma unroll
    for (int w = 1; w < WPR; ++w) s += slot[w];
    return s;
  }
}

// Loads of one vector slot: the t slab vectors, the residual and the bias.
template <int NS>
struct Slot {
  u32x4 s[NS];
  u32x4 r;
  u32x4 b;
};

// At least 2 waves per SIMD: 8 rows per CU, which keeps a 2048-row shard
// resident in one pass (the register budget caps how far loads are hoisted).
template <class E, int NS, int VPL, int WPR, bool MASK, bool YNT>
__global__ __launch_bounds__(WPR == 1 ? 64 * kRowsPerBlockW1 : 64 * WPR, 2) void sp_region_fwd_kernel(const FwdParams p) {
  constexpr int V = E::kVec;
  constexpr int EB = 16 / V;
  __shared__ float red[2][WPR];
  // Packed z of the row lives in LDS when the row has 8-16 vectors per lane
  // (each lane reads back only what it wrote, so no barrier is needed); that
  // frees 32-64 VGPRs for the prefetch pipeline.  Short rows keep z in
  // registers.
  constexpr bool ZLDS = VPL <= 16 && VPL >= 8;
  constexpr int ZW = WPR == 1 ? kRowsPerBlockW1 : WPR;
  __shared__ u32x4 zlds[ZLDS ? ZW : 1][ZLDS ? VPL : 1][64];

  const int lane = threadIdx.x & 63;
  // threadIdx.x / 64 is wave-uniform; readfirstlane tells the compiler, so the
  // row's base pointers live in SGPRs.
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 64));
  const int wv = WPR == 1 ? 0 : wave;
  const int64_t row = WPR == 1 ? static_cast<int64_t>(blockIdx.x) * kRowsPerBlockW1 + wave
                               : static_cast<int64_t>(blockIdx.x);
  if (row >= p.T) return;   // the whole wave (WPR = 1) or block (WPR > 1) leaves

  const int h = p.h;
  const int nvec = h / V;
  const int64_t row_off = row * static_cast<int64_t>(h) * EB;   // bytes
  // Each slab through its own base pointer (wave-uniform), so slabs may sit
  // in separate buffers -- or, peer-mapped, in other GPUs' memory.
  const char* srow[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) srow[s] = static_cast<const char*>(p.slab[s]) + row_off;

  // Every memory instruction below is unconditional.  The waitcnt pass
  // cannot count loads or stores issued under a branch, and would then wait
  // for part of the prefetched slot before using the current one.  So:
  //  * an absent residual / bias / beta is replaced by gamma, an in-bounds,
  //    L2-resident stand-in whose values are never used (the branches that
  //    apply them are arithmetic only);
  //  * slots past the end of a row whose vector count is not a multiple of
  //    64*WPR are clamped to the row's last vector: they recompute exactly
  //    that vector's z, y and mask, so their stores write identical bytes.
  const bool has_res = p.residual != nullptr;
  const bool has_bias = p.bias != nullptr;
  const bool has_beta = p.beta != nullptr;
  const char* stand_in = static_cast<const char*>(p.gamma);
  const char* rrow = has_res ? static_cast<const char*>(p.residual) + row_off : stand_in;
  const char* biasp = has_bias ? static_cast<const char*>(p.bias) : stand_in;
  const char* betap = has_beta ? static_cast<const char*>(p.beta) : stand_in;

  auto vec_of = [&](int k) {
    const int v = lane + 64 * (wv + WPR * k);
    return v < nvec ? v : nvec - 1;
  };
  auto valid = [&](int k) { return lane + 64 * (wv + WPR * k) < nvec; };
  // Addresses are a wave-uniform base (SGPRs) plus a zero-extended 32-bit
  // lane offset, the form global loads take as saddr + voffset.
  auto lane_off = [&](int k) { return static_cast<uint32_t>(vec_of(k)) * 16u; };

  auto issue = [&](Slot<NS>& sl, int k) {
    const uint32_t o = lane_off(k);
#pragma unroll
    for (int s = 0; s < NS; ++s) sl.s[s] = ld16_stream(srow[s] + o);
    sl.r = ld16_stream(rrow + o);
    sl.b = ld16(biasp + o);
  };

  const uint64_t g = p.drop ? global_token_of(row, p.T, p.t, p.rank, p.cu, p.nseq) : 0;
  const uint32_t g_lo = static_cast<uint32_t>(g), g_hi = static_cast<uint32_t>(g >> 32);

  u32x4 zs[ZLDS ? 1 : VPL];   // rounded z, packed (when not in LDS)
  auto zput = [&](int k, u32x4 v) {
    if constexpr (ZLDS) zlds[wave][k][lane] = v;
    else zs[k] = v;
  };
  auto zget = [&](int k) -> u32x4 {
    if constexpr (ZLDS) return zlds[wave][k][lane];
    else return zs[k];
  };

  // z of slot k = round(residual + dropout(sum_s P_s + bias)); stores z (and
  // the mask), returns this lane's sum of the rounded values (LayerNorm mean).
  auto process = [&](const Slot<NS>& sl, int k) -> float {
    const int v = vec_of(k);
    float acc[V];
    unpack(E{}, sl.s[0], acc);
#pragma unroll
    for (int s = 1; s < NS; ++s) {
      float f[V];
      unpack(E{}, sl.s[s], f);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = acc[e] + f[e];
    }
    if (has_bias) {
      float f[V];
      unpack(E{}, sl.b, f);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = acc[e] + f[e];
    }
    bool keep[V];
#pragma unroll
    for (int e = 0; e < V; ++e) keep[e] = true;
    if (p.drop) {
      dropout_keep<V>(static_cast<uint32_t>(v), g_lo, g_hi, p.key0, p.key1, p.thr, keep);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = keep[e] ? acc[e] * p.scale : 0.0f;
    }
    if (has_res) {
      float f[V];
      unpack(E{}, sl.r, f);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = f[e] + acc[e];
    }
    const u32x4 zk = pack(E{}, acc);
    zput(k, zk);
    st16(static_cast<char*>(p.z) + row_off + lane_off(k), zk);
    if constexpr (MASK) {
      uint8_t* m = p.mask + row * static_cast<int64_t>(h) + static_cast<uint32_t>(v) * V;
      if constexpr (V == 8) {
        uint2 mv;
        mv.x = keep[0] | (keep[1] << 8) | (keep[2] << 16) | (keep[3] << 24);
        mv.y = keep[4] | (keep[5] << 8) | (keep[6] << 16) | (keep[7] << 24);
        *reinterpret_cast<uint2*>(m) = mv;
      } else {
        *reinterpret_cast<uint32_t*>(m) = keep[0] | (keep[1] << 8) | (keep[2] << 16) | (keep[3] << 24);
      }
    }
    float f[V];
    rounded_values(E{}, zk, f);
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < V; ++e) part += f[e];
    return valid(k) ? part : 0.0f;
  };

  // ---- stream the row: slot k+1's loads are in flight while k is summed ----
  constexpr bool LOOP = ZLDS && SPR_FWD_LOOP;
  float zsum = 0.0f;
  Slot<NS> A, B;
  issue(A, 0);
  if constexpr (LOOP) {
    // Runtime loop over slot pairs; the last pair is peeled so that every
    // iteration issues the same loads (VPL is even here).
#pragma unroll 1
    for (int k = 0; k < VPL - 2; k += 2) {
      issue(B, k + 1);
      __builtin_amdgcn_sched_barrier(0);
      zsum += process(A, k);
      issue(A, k + 2);
      __builtin_amdgcn_sched_barrier(0);
      zsum += process(B, k + 1);
    }
    issue(B, VPL - 1);
    __builtin_amdgcn_sched_barrier(0);
    zsum += process(A, VPL - 2);
    __builtin_amdgcn_sched_barrier(0);
    zsum += process(B, VPL - 1);
  } else {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      if (k + 1 < VPL) issue((k & 1) ? A : B, k + 1);   // compile-time after unrolling
      __builtin_amdgcn_sched_barrier(0);
      zsum += process((k & 1) ? B : A, k);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- statistics over the full h (from the rounded z) --------------------
  // gamma/beta of slot 0 are in flight during the statistics.
  auto issue_gb = [&](u32x4 (&gb)[2], int k) {
    const uint32_t o = lane_off(k);
    gb[0] = ld16(static_cast<const char*>(p.gamma) + o);
    gb[1] = ld16(betap + o);
  };
  u32x4 GA[2], GB[2];
  issue_gb(GA, 0);

  const float inv_h = 1.0f / static_cast<float>(h);
  const bool ln = p.norm == 0;
  const float mean = ln ? row_total<WPR>(zsum, red[0]) * inv_h : 0.0f;
  float q = 0.0f;
#pragma unroll 2
  for (int k = 0; k < VPL; ++k) {
    float f[V];
    rounded_values(E{}, zget(k), f);
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float d = f[e] - mean;   // mean = 0 for RMSNorm: the mean square
      part = __builtin_fmaf(d, d, part);
    }
    q += valid(k) ? part : 0.0f;
  }
  const float rstd = 1.0f / __builtin_sqrtf(row_total<WPR>(q, red[1]) * inv_h + p.eps);

  // ---- y = (z - mean)*rstd*gamma + beta, gamma/beta one slot ahead ---------
  auto emit_y = [&](const u32x4 (&gb)[2], int k) {
    float zf[V], gm[V], bt[V], yv[V];
    rounded_values(E{}, zget(k), zf);
    unpack(E{}, gb[0], gm);
    unpack(E{}, gb[1], bt);
    if (!has_beta) {
#pragma unroll
      for (int e = 0; e < V; ++e) bt[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < V; ++e) yv[e] = __builtin_fmaf((zf[e] - mean) * rstd, gm[e], bt[e]);
    if constexpr (YNT) st16_stream(static_cast<char*>(p.y) + row_off + lane_off(k), pack(E{}, yv));
    else st16(static_cast<char*>(p.y) + row_off + lane_off(k), pack(E{}, yv));
  };
  if constexpr (LOOP) {
#pragma unroll 1
    for (int k = 0; k < VPL - 2; k += 2) {
      issue_gb(GB, k + 1);
      emit_y(GA, k);
      issue_gb(GA, k + 2);
      emit_y(GB, k + 1);
    }
    issue_gb(GB, VPL - 1);
    emit_y(GA, VPL - 2);
    emit_y(GB, VPL - 1);
  } else {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      if (k + 1 < VPL) issue_gb((k & 1) ? GA : GB, k + 1);   // compile-time after unrolling
      emit_y((k & 1) ? GB : GA, k);
    }
  }
  if (threadIdx.x % (64 * WPR) == 0) {
    if (p.mean) p.mean[row] = mean;
    p.rstd[row] = rstd;
  }
}

// Shards whose z and y exceed this many bytes store y nontemporally (rows
// of 8 or more vectors per lane; the mask-writing test path never).
constexpr int64_t kStreamYBytes = int64_t{256} << 20;

template <class E, int VPL, int WPR>
hipError_t launch_ns(const FwdParams& p, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(WPR == 1 ? (p.T + kRowsPerBlockW1 - 1) / kRowsPerBlockW1 : p.T));
  const dim3 block(WPR == 1 ? 64 * kRowsPerBlockW1 : 64 * WPR);
  const bool mask = p.mask != nullptr;
  const bool ynt = VPL >= 8 && !mask && 2 * p.T * p.h * (16 / E::kVec) > kStreamYBytes;
  switch (p.t) {
#define SPR_NS(N)                                                                                          \
  case N:                                                                                                  \
    if (mask)                                                                                              \
      launch_kernel(sp_region_fwd_kernel<E, N, VPL, WPR, true, false>, grid, block, stream, KernelRole::kOnly, p); \
    else if constexpr (VPL >= 8) {                                                                         \
      if (ynt)                                                                                             \
        launch_kernel(sp_region_fwd_kernel<E, N, VPL, WPR, false, true>, grid, block, stream, KernelRole::kOnly, p); \
      else                                                                                                 \
        launch_kernel(sp_region_fwd_kernel<E, N, VPL, WPR, false, false>, grid, block, stream, KernelRole::kOnly, p); \
    } else {                                                                                               \
      launch_kernel(sp_region_fwd_kernel<E, N, VPL, WPR, false, false>, grid, block, stream, KernelRole::kOnly, p); \
    }                                                                                                      \
    break;
    SPR_NS(1) SPR_NS(2) SPR_NS(3) SPR_NS(4) SPR_NS(5) SPR_NS(6) SPR_NS(7) SPR_NS(8)
#undef SPR_NS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Shards of at most kSplitRows rows: one wave per row would leave most of
// the 1024 SIMDs idle, and latency, not bandwidth, bounds the call.  Their
// rows of 4 or 8 vectors per lane get 4 waves, the vectors split between
// them (measured at 512 x 4096 bf16: 11.9 -> 10.8 us; rows of 2 vectors per
// lane on 2 waves measured no better at 64 x 512 fp32).
#ifndef SPR_FWD_SPLIT_T
#define SPR_FWD_SPLIT_T 1024
#endif
constexpr int64_t kSplitRows = SPR_FWD_SPLIT_T;
template <class E>
hipError_t launch_e(const FwdParams& p, const Shape& sh, hipStream_t stream) {
  if (sh.threads == 64 && p.T <= kSplitRows) {
    switch (sh.vpt) {
      case 4: return launch_ns<E, 1, 4>(p, stream);
      case 8: return launch_ns<E, 2, 4>(p, stream);
      default: break;
    }
  }
  if (sh.threads == 64) {
    switch (sh.vpt) {
      case 1: return launch_ns<E, 1, 1>(p, stream);
      case 2: return launch_ns<E, 2, 1>(p, stream);
      case 4: return launch_ns<E, 4, 1>(p, stream);
      case 8: return launch_ns<E, 8, 1>(p, stream);
      case 10: return launch_ns<E, 10, 1>(p, stream);
      case 12: return launch_ns<E, 12, 1>(p, stream);
      case 14: return launch_ns<E, 14, 1>(p, stream);
      case 16: return launch_ns<E, 16, 1>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (sh.threads == 128 && sh.vpt == 16) return launch_ns<E, 16, 2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

// Waves per row and vectors per lane: rows of up to 1024 vectors (h <= 8192
// bf16, 4096 f32) get one wave and the smallest VPL in {1, 2, 4, 8, 10, 12,
// 14, 16} covering them; wider rows (up to 2048 vectors) get two waves of 16.
// Shape.threads is 64 * waves per row.  (h = 8192 bf16 -> 1 x 16; h = 5120
// -> 1 x 10; h = 512 f32 -> 1 x 2; h = 16384 bf16 -> 2 x 16.)
Shape fwd_shape(int h, int dtype) {
  const int vec = dtype == 1 ? 8 : 4;
  const int nvec = h / vec;
  for (int vpl : {1, 2, 4, 8, 10, 12, 14, 16})
    if (nvec <= 64 * vpl) return Shape{vpl, 64};
  if (nvec <= 2 * 64 * 16) return Shape{16, 128};
  return Shape{0, 0};
}

hipError_t launch_fwd(const FwdParams& p, int dtype, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const Shape sh = fwd_shape(p.h, dtype);
  return dtype == 1 ? launch_e<Bf16>(p, sh, stream) : launch_e<F32>(p, sh, stream);
}

}  // namespace spr

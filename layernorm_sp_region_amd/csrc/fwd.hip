// Forward of the sequence-parallel region: one workgroup per local token row.
//
// Per row (hpc.payai.win lesson 7: g* of section 3.A, LayerNorm of section 2):
//   acc = P_0 + P_1 + ... + P_{t-1}      float32, ascending k (g* arithmetic)
//   acc = acc + bias                      if bias
//   d   = keep ? acc * scale : 0          if p > 0 (Philox-4x32-10 keep bit)
//   z   = round(residual + d)             stored; statistics use the rounded z
//   LayerNorm: mean, population variance (two passes over registers),
//              y = (z - mean) * rstd * gamma + beta
//   RMSNorm:   y = z * rstd * gamma, rstd = 1/sqrt(mean(z^2) + eps)
//
// The z chain is compiled without floating-point contraction (the build
// passes -ffp-contract=off) so it matches the float32 operation order
// exactly; the normalisation uses explicit fmaf.
//
// Memory plan: every thread owns VPT 16-byte vectors of the row (vector
// v = tid + k*blockDim), so each slab row is read by fully coalesced 16-byte
// loads.  All t*VPT slab loads, the residual and the parameters are issued
// before any arithmetic, giving t*16 KB (h = 8192, bf16) in flight per row.
// Slabs and residual are streamed with a nontemporal hint; gamma/beta/bias
// (shared by every row) use ordinary cached loads.
#include "spr_device.h"
#include "spr_internal.h"

namespace spr {
namespace {

__device__ __forceinline__ uint64_t global_token(const FwdParams& p, int64_t row) {
  if (p.cu == nullptr) return static_cast<uint64_t>(p.rank) * static_cast<uint64_t>(p.T) + row;
  // Largest q in [0, nseq) with cu[q] <= row (empty sequences are skipped).
  int lo = 0, hi = p.nseq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.cu[mid] <= row) lo = mid; else hi = mid;
  }
  const int64_t start = p.cu[lo];
  const int64_t len = static_cast<int64_t>(p.cu[lo + 1]) - start;
  return static_cast<uint64_t>(p.t * start + p.rank * len + (row - start));
}

template <class E, int NS, int VPT, int MAXBS>
__global__ __launch_bounds__(MAXBS) void sp_region_fwd_kernel(const FwdParams p) {
  constexpr int V = E::kVec;
  constexpr int EB = 16 / V;
  __shared__ float red[2][16];

  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int bs = blockDim.x;
  const int h = p.h;
  const int nvec = h / V;
  const int64_t row_off = row * static_cast<int64_t>(h) * EB;   // bytes
  const int64_t slab_bytes = p.slab_stride * EB;

  int vv[VPT];
  bool valid[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * bs;
    valid[k] = v < nvec;
    vv[k] = valid[k] ? v : nvec - 1;   // clamped: loads stay in bounds
  }

  // ---- issue every load of the row -------------------------------------
  u32x4 raw[VPT][NS];
  u32x4 rres[VPT], rbias[VPT], rgam[VPT], rbet[VPT];
  const char* prow = static_cast<const char*>(p.partials) + row_off;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int s = 0; s < NS; ++s) raw[k][s] = ld16_stream(prow + s * slab_bytes + vv[k] * 16);
  }
  if (p.residual) {
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      rres[k] = ld16_stream(static_cast<const char*>(p.residual) + row_off + vv[k] * 16);
  }
  if (p.bias) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) rbias[k] = ld16(static_cast<const char*>(p.bias) + vv[k] * 16);
  }
#pragma unroll
  for (int k = 0; k < VPT; ++k) rgam[k] = ld16(static_cast<const char*>(p.gamma) + vv[k] * 16);
  if (p.beta) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) rbet[k] = ld16(static_cast<const char*>(p.beta) + vv[k] * 16);
  }

  const uint64_t g = p.drop ? global_token(p, row) : 0;
  const uint32_t g_lo = static_cast<uint32_t>(g), g_hi = static_cast<uint32_t>(g >> 32);

  // ---- z = round(residual + dropout(sum + bias)) ------------------------
  float zr[VPT][V];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float acc[V];
    unpack(E{}, raw[k][0], acc);
#pragma unroll
    for (int s = 1; s < NS; ++s) {
      float f[V];
      unpack(E{}, raw[k][s], f);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = acc[e] + f[e];
    }
    if (p.bias) {
      float f[V];
      unpack(E{}, rbias[k], f);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = acc[e] + f[e];
    }
    uint8_t keep[V];
#pragma unroll
    for (int e = 0; e < V; ++e) keep[e] = 1;
    if (p.drop) {
#pragma unroll
      for (int b4 = 0; b4 < V / 4; ++b4) {
        const uint32_t blk = static_cast<uint32_t>(vv[k] * (V / 4) + b4);   // channel / 4
        const Philox4 r = philox4x32_10(blk, g_lo, g_hi, 0u, p.key0, p.key1);
#pragma unroll
        for (int w = 0; w < 4; ++w) keep[b4 * 4 + w] = r.w[w] >= p.thr;
      }
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = keep[e] ? acc[e] * p.scale : 0.0f;
    }
    if (p.residual) {
      float f[V];
      unpack(E{}, rres[k], f);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = f[e] + acc[e];
    }
    const u32x4 zp = pack(E{}, acc);
    rounded_values(E{}, zp, zr[k]);
    if (valid[k]) {
      st16(static_cast<char*>(p.z) + row_off + vv[k] * 16, zp);
      if (p.mask) {
        uint8_t* m = p.mask + row * static_cast<int64_t>(h) + vv[k] * V;
        if constexpr (V == 8) {
          uint2 mv;
          mv.x = keep[0] | (keep[1] << 8) | (keep[2] << 16) | (keep[3] << 24);
          mv.y = keep[4] | (keep[5] << 8) | (keep[6] << 16) | (keep[7] << 24);
          *reinterpret_cast<uint2*>(m) = mv;
        } else {
          *reinterpret_cast<uint32_t*>(m) = keep[0] | (keep[1] << 8) | (keep[2] << 16) | (keep[3] << 24);
        }
      }
    }
  }

  // ---- statistics over the full h ----------------------------------------
  const float inv_h = 1.0f / static_cast<float>(h);
  float mean = 0.0f, rstd;
  if (p.norm == 0) {
    float s[1] = {0.0f};
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (valid[k]) {
#pragma unroll
        for (int e = 0; e < V; ++e) s[0] += zr[k][e];
      }
    block_sum<1>(s, red[0]);
    mean = s[0] * inv_h;
    float q[1] = {0.0f};
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (valid[k]) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float d = zr[k][e] - mean;
          q[0] = __builtin_fmaf(d, d, q[0]);
        }
      }
    block_sum<1>(q, red[1]);
    rstd = 1.0f / __builtin_sqrtf(q[0] * inv_h + p.eps);
  } else {
    float q[1] = {0.0f};
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (valid[k]) {
#pragma unroll
        for (int e = 0; e < V; ++e) q[0] = __builtin_fmaf(zr[k][e], zr[k][e], q[0]);
      }
    block_sum<1>(q, red[1]);
    rstd = 1.0f / __builtin_sqrtf(q[0] * inv_h + p.eps);
  }
  if (tid == 0) {
    if (p.mean) p.mean[row] = mean;
    p.rstd[row] = rstd;
  }

  // ---- y -------------------------------------------------------------------
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (!valid[k]) continue;
    float gm[V], bt[V], yv[V];
    unpack(E{}, rgam[k], gm);
    if (p.beta) unpack(E{}, rbet[k], bt);
    else {
#pragma unroll
      for (int e = 0; e < V; ++e) bt[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < V; ++e) yv[e] = __builtin_fmaf((zr[k][e] - mean) * rstd, gm[e], bt[e]);
    st16(static_cast<char*>(p.y) + row_off + vv[k] * 16, pack(E{}, yv));
  }
}

template <class E, int VPT>
hipError_t launch_ns(const FwdParams& p, int threads, hipStream_t stream) {
  constexpr int MAXBS = 512;
  const dim3 grid(static_cast<unsigned>(p.T)), block(threads);
  switch (p.t) {
    case 1: hipLaunchKernelGGL((sp_region_fwd_kernel<E, 1, VPT, MAXBS>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((sp_region_fwd_kernel<E, 2, VPT, MAXBS>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((sp_region_fwd_kernel<E, 3, VPT, MAXBS>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((sp_region_fwd_kernel<E, 4, VPT, MAXBS>), grid, block, 0, stream, p); break;
    case 5: hipLaunchKernelGGL((sp_region_fwd_kernel<E, 5, VPT, MAXBS>), grid, block, 0, stream, p); break;
    case 6: hipLaunchKernelGGL((sp_region_fwd_kernel<E, 6, VPT, MAXBS>), grid, block, 0, stream, p); break;
    case 7: hipLaunchKernelGGL((sp_region_fwd_kernel<E, 7, VPT, MAXBS>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((sp_region_fwd_kernel<E, 8, VPT, MAXBS>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class E>
hipError_t launch_e(const FwdParams& p, const Shape& sh, hipStream_t stream) {
  switch (sh.vpt) {
    case 1: return launch_ns<E, 1>(p, sh.threads, stream);
    case 2: return launch_ns<E, 2>(p, sh.threads, stream);
    case 4: return launch_ns<E, 4>(p, sh.threads, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Smallest VPT in {1, 2, 4} giving at most 512 threads; threads rounded up to
// whole waves.  (h = 8192 bf16 -> 2 x 512; h = 5120 -> 2 x 320.)
Shape fwd_shape(int h, int dtype) {
  const int vec = dtype == 1 ? 8 : 4;
  const int nvec = h / vec;
  for (int vpt : {1, 2, 4}) {
    const int need = (nvec + vpt - 1) / vpt;
    if (need <= 512) return Shape{vpt, ((need + 63) / 64) * 64};
  }
  return Shape{0, 0};
}

hipError_t launch_fwd(const FwdParams& p, int dtype, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const Shape sh = fwd_shape(p.h, dtype);
  return dtype == 1 ? launch_e<Bf16>(p, sh, stream) : launch_e<F32>(p, sh, stream);
}

}  // namespace spr

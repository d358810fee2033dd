// Backward of the region's normalisation (the adjoint of the forward, as
// hpc.payai.win lesson 7 section 3.B describes autograd): with
// xhat = (z - mean)*rstd (RMSNorm: z*rstd), g = dy*gamma,
// c1 = mean_j g, c2 = mean_j(g*xhat):
//   LayerNorm dx = rstd*(g - c1 - xhat*c2)     RMSNorm dx = rstd*(g - xhat*c2)
//   plus dres_in (the gradient reaching z through the residual stream);
//   dgamma_j = sum_i dy_ij*xhat_ij,  dbeta_j = sum_i dy_ij over the T rows.
//
// Stage 1 (sp_region_bwd_rows_kernel): G blocks, block b owns the contiguous
// rows [b*T/G, (b+1)*T/G).  Each thread owns a fixed set of columns, keeps
// their gamma and their dgamma/dbeta running sums in registers across rows,
// and the block writes one [2][h] float32 partial to the workspace.  RPI rows
// are loaded together and their 2*RPI row sums share one block reduction.
//
// Stage 2 (sp_region_bwd_cols_kernel): dgamma/dbeta = the G partials summed in
// ascending block order, split over 16 groups whose sums are combined in
// group order -- a fixed tree, so results are bitwise reproducible.
#include "spr_device.h"
#include "spr_internal.h"

namespace spr {
namespace {

template <class E, int VPT, int RPI, int MAXBS>
__global__ __launch_bounds__(MAXBS) void sp_region_bwd_rows_kernel(const BwdParams p) {
  constexpr int V = E::kVec;
  constexpr int EB = 16 / V;
  constexpr int NR = 2 * RPI;
  __shared__ float red[2][NR * 16];

  const int tid = threadIdx.x;
  const int bs = blockDim.x;
  const int h = p.h;
  const int nvec = h / V;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * p.T / p.G;
  const int64_t r1 = static_cast<int64_t>(blockIdx.x + 1) * p.T / p.G;
  const bool ln = p.norm == 0;
  const float inv_h = 1.0f / static_cast<float>(h);

  int vv[VPT];
  bool valid[VPT];
  float gam[VPT][V], dg[VPT][V], db[VPT][V];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * bs;
    valid[k] = v < nvec;
    vv[k] = valid[k] ? v : nvec - 1;
    unpack(E{}, ld16(static_cast<const char*>(p.gamma) + vv[k] * 16), gam[k]);
#pragma unroll
    for (int e = 0; e < V; ++e) dg[k][e] = db[k][e] = 0.0f;
  }

  int parity = 0;
  for (int64_t r = r0; r < r1; r += RPI) {
    u32x4 rdy[RPI][VPT], rz[RPI][VPT], rdr[RPI][VPT];
    float mu[RPI], rs[RPI];
#pragma unroll
    for (int q = 0; q < RPI; ++q) {
      const int64_t row = (r + q < r1) ? r + q : r1 - 1;   // clamped: loads stay in bounds
      const int64_t off = row * static_cast<int64_t>(h) * EB;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        rdy[q][k] = ld16_stream(static_cast<const char*>(p.dy) + off + vv[k] * 16);
        rz[q][k] = ld16_stream(static_cast<const char*>(p.z) + off + vv[k] * 16);
        if (p.dres) rdr[q][k] = ld16_stream(static_cast<const char*>(p.dres) + off + vv[k] * 16);
      }
      mu[q] = ln ? p.mean[row] : 0.0f;
      rs[q] = p.rstd[row];
    }

    float xh[RPI][VPT][V], gg[RPI][VPT][V], dyv[RPI][VPT][V];
    float sums[NR];
#pragma unroll
    for (int q = 0; q < RPI; ++q) {
      sums[2 * q] = 0.0f;
      sums[2 * q + 1] = 0.0f;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        float zv[V];
        unpack(E{}, rz[q][k], zv);
        unpack(E{}, rdy[q][k], dyv[q][k]);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          xh[q][k][e] = (zv[e] - mu[q]) * rs[q];
          gg[q][k][e] = dyv[q][k][e] * gam[k][e];
        }
        if (valid[k]) {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            sums[2 * q] += gg[q][k][e];
            sums[2 * q + 1] = __builtin_fmaf(gg[q][k][e], xh[q][k][e], sums[2 * q + 1]);
          }
        }
      }
    }
    block_sum<NR>(sums, red[parity]);
    parity ^= 1;

#pragma unroll
    for (int q = 0; q < RPI; ++q) {
      if (r + q >= r1) break;
      const int64_t off = (r + q) * static_cast<int64_t>(h) * EB;
      const float c1 = ln ? sums[2 * q] * inv_h : 0.0f;
      const float c2 = sums[2 * q + 1] * inv_h;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        if (!valid[k]) continue;
        float dx[V];
#pragma unroll
        for (int e = 0; e < V; ++e) dx[e] = rs[q] * __builtin_fmaf(-xh[q][k][e], c2, gg[q][k][e] - c1);
        if (p.dres) {
          float f[V];
          unpack(E{}, rdr[q][k], f);
#pragma unroll
          for (int e = 0; e < V; ++e) dx[e] += f[e];
        }
        st16(static_cast<char*>(p.dx) + off + vv[k] * 16, pack(E{}, dx));
#pragma unroll
        for (int e = 0; e < V; ++e) {
          dg[k][e] = __builtin_fmaf(dyv[q][k][e], xh[q][k][e], dg[k][e]);
          db[k][e] += dyv[q][k][e];
        }
      }
    }
  }

  float* wsg = p.ws + static_cast<int64_t>(blockIdx.x) * 2 * h;
  float* wsb = wsg + h;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (!valid[k]) continue;
#pragma unroll
    for (int e0 = 0; e0 < V; e0 += 4) {
      st16(wsg + vv[k] * V + e0, u32x4{__float_as_uint(dg[k][e0]), __float_as_uint(dg[k][e0 + 1]),
                                       __float_as_uint(dg[k][e0 + 2]), __float_as_uint(dg[k][e0 + 3])});
      st16(wsb + vv[k] * V + e0, u32x4{__float_as_uint(db[k][e0]), __float_as_uint(db[k][e0 + 1]),
                                       __float_as_uint(db[k][e0 + 2]), __float_as_uint(db[k][e0 + 3])});
    }
  }
}

// 256 threads = 16 column quads x 16 groups of partials.
constexpr int kColQuads = 16;
constexpr int kGroups = 16;

__global__ __launch_bounds__(256) void sp_region_bwd_cols_kernel(const float* __restrict__ ws, int G, int h,
                                                                 float* __restrict__ dgamma,
                                                                 float* __restrict__ dbeta) {
  __shared__ float4 part[2][kGroups][kColQuads];
  const int cq = threadIdx.x % kColQuads;
  const int grp = threadIdx.x / kColQuads;
  const int nq = h / 4;
  const int c4 = blockIdx.x * kColQuads + cq;
  float4 sg = make_float4(0.f, 0.f, 0.f, 0.f), sb = sg;
  if (c4 < nq) {
    const int g0 = grp * G / kGroups, g1 = (grp + 1) * G / kGroups;
    for (int g = g0; g < g1; ++g) {
      const float4 a = reinterpret_cast<const float4*>(ws + static_cast<int64_t>(g) * 2 * h)[c4];
      const float4 b = reinterpret_cast<const float4*>(ws + static_cast<int64_t>(g) * 2 * h + h)[c4];
      sg.x += a.x; sg.y += a.y; sg.z += a.z; sg.w += a.w;
      sb.x += b.x; sb.y += b.y; sb.z += b.z; sb.w += b.w;
    }
  }
  part[0][grp][cq] = sg;
  part[1][grp][cq] = sb;
  __syncthreads();
  if (grp == 0 && c4 < nq) {
    float4 tg = part[0][0][cq], tb = part[1][0][cq];
    for (int i = 1; i < kGroups; ++i) {
      const float4 a = part[0][i][cq], b = part[1][i][cq];
      tg.x += a.x; tg.y += a.y; tg.z += a.z; tg.w += a.w;
      tb.x += b.x; tb.y += b.y; tb.z += b.z; tb.w += b.w;
    }
    reinterpret_cast<float4*>(dgamma)[c4] = tg;
    if (dbeta) reinterpret_cast<float4*>(dbeta)[c4] = tb;
  }
}

// VPT = 1 keeps two rows in flight per block; VPT = 2 (h above 8192 bf16 /
// 4096 f32) processes one row at a time to stay within 128 VGPRs at 1024
// threads.
template <class E>
hipError_t launch_rows(const BwdParams& p, const Shape& sh, hipStream_t stream) {
  constexpr int MAXBS = 1024;
  const dim3 grid(static_cast<unsigned>(p.G)), block(sh.threads);
  switch (sh.vpt) {
    case 1: hipLaunchKernelGGL((sp_region_bwd_rows_kernel<E, 1, 2, MAXBS>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((sp_region_bwd_rows_kernel<E, 2, 1, MAXBS>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Smallest VPT in {1, 2} giving at most 1024 threads (h = 8192 bf16 -> 1 x 1024).
Shape bwd_shape(int h, int dtype) {
  const int vec = dtype == 1 ? 8 : 4;
  const int nvec = h / vec;
  for (int vpt : {1, 2}) {
    const int need = (nvec + vpt - 1) / vpt;
    if (need <= 1024) return Shape{vpt, ((need + 63) / 64) * 64};
  }
  return Shape{0, 0};
}

hipError_t launch_bwd(const BwdParams& p, int dtype, hipStream_t stream) {
  if (p.G > 0) {
    const Shape sh = bwd_shape(p.h, dtype);
    const hipError_t e = dtype == 1 ? launch_rows<Bf16>(p, sh, stream) : launch_rows<F32>(p, sh, stream);
    if (e != hipSuccess) return e;
  }
  const int nq = p.h / 4;
  const dim3 grid((nq + kColQuads - 1) / kColQuads), block(kColQuads * kGroups);
  hipLaunchKernelGGL(sp_region_bwd_cols_kernel, grid, block, 0, stream, p.ws, p.G, p.h, p.dgamma, p.dbeta);
  return hipGetLastError();
}

}  // namespace spr

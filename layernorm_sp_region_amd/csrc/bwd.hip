// Backward of the region's normalisation (the adjoint of the forward, as
// hpc.payai.win lesson 7 section 3.B describes autograd): with
// xhat = (z - mean)*rstd (RMSNorm: z*rstd), g = dy*gamma,
// c1 = mean_j g, c2 = mean_j(g*xhat):
//   LayerNorm dx = rstd*(g - c1 - xhat*c2)     RMSNorm dx = rstd*(g - xhat*c2)
//   plus dres_in (the gradient reaching z through the residual stream);
//   dgamma_j = sum_i dy_ij*xhat_ij,  dbeta_j = sum_i dy_ij over the T rows.
//
// Through the dropout and the slab sum (the DROP variant, row-linear side of
// the same section): dpartial = dx * keep * scale with the forward's own
// mask, the gradient of every slab, and dbias_j = sum_i dpartial_ij.
//
// Stage 1 (sp_region_bwd_rows_kernel): G blocks, block b owns rows b, b + G,
// b + 2G, ... (interleaved, so the rows the G blocks read at one moment form
// one contiguous band of memory; contiguous runs of T/G rows per block put
// the concurrent reads T/G rows apart, a power-of-two stride at the usual
// shapes, which measured 2-9% slower).  Each thread owns a fixed set of columns, keeps
// their gamma and their dgamma/dbeta (/dbias) running sums in registers
// across rows, and the block writes one float32 partial per gradient to the
// workspace.  Rows stream through a ring of RING packed row buffers (RING
// rows in flight per block); each row's two sums take one block reduction.
//
// Stage 2 (sp_region_bwd_cols_kernel): each gradient = the G partials summed
// in ascending block order, split over 32 groups whose sums are combined in
// group order -- a fixed tree, so results are bitwise reproducible.

#include "spr_device.h"
#include "spr_internal.h"

namespace spr {
namespace {

#ifndef SPR_BWD_NT_STORE
#define SPR_BWD_NT_STORE 1        // nontemporal stores for dx (measured: the next kernel no longer
                                  // pays for writing back dirty dx lines)
#endif

__device__ __forceinline__ void st16_dx(void* p, u32x4 v) {
  if constexpr (SPR_BWD_NT_STORE) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else st16(p, v);
}

#ifndef SPR_WS_NT
#define SPR_WS_NT 0
#endif
__device__ __forceinline__ void st16_ws(void* p, u32x4 v) {
  if constexpr (SPR_WS_NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else st16(p, v);
}

// Packed loads of one row: VPT vectors of dy, z (and dres) per thread.
// The row's statistics travel with its data: every lane loads the same
// mean/rstd (one broadcast request per wave), so waiting for a ring slot
// never waits on loads issued after it (vmcnt completes in issue order).
template <int VPT, bool DRES>
struct RowBuf {
  u32x4 dy[VPT], z[VPT], dr[DRES ? VPT : 1];
  float mu, rs;
  uint32_t g_lo, g_hi;   // global token index of the row (dropout backward)
};

// Stage 1 for block blockIdx.x: dx of its rows (and, with DROP, dpartial =
// dx*keep*scale), and its partials of dgamma, dbeta (and dbias) in the
// workspace: slot j of block b at ws + b*ws_bstride + j*ws_sstride.
template <class E, int VPT, int RING, bool DRES, bool DROP>
__device__ __forceinline__ void rows_stage(const BwdParams& p) {
  constexpr int V = E::kVec;
  constexpr int EB = 16 / V;
  __shared__ float red[2][2 * 16];

  const int tid = threadIdx.x;
  const int bs = blockDim.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave, nwaves = bs / kWave;
  const int h = p.h;
  const int nvec = h / V;
  // Local row li of this block is global row blockIdx.x + li*G (G <= T, so
  // every block has at least one row).
  const int r0 = 0;
  const int r1 = static_cast<int>((p.T - blockIdx.x + p.G - 1) / p.G);
  const int bx = blockIdx.x, G = p.G;
  auto grow = [=](int li) { return bx + li * G; };
  const bool ln = p.norm == 0;
  const float inv_h = 1.0f / static_cast<float>(h);

  int vv[VPT];
  bool valid[VPT];
  float gam[VPT][V], dg[VPT][V], db[VPT][V];
  float dbs[DROP ? VPT : 1][V];   // dbias running sums
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * bs;
    valid[k] = v < nvec;
    vv[k] = valid[k] ? v : nvec - 1;   // clamped: loads stay in bounds
    unpack(E{}, ld16(static_cast<const char*>(p.gamma) + vv[k] * 16), gam[k]);
#pragma unroll
    for (int e = 0; e < V; ++e) dg[k][e] = db[k][e] = 0.0f;
    if constexpr (DROP) {
#pragma unroll
      for (int e = 0; e < V; ++e) dbs[k][e] = 0.0f;
    }
  }

  // Rows stream through a ring of RING row buffers: row r + RING is issued
  // as soon as row r has been consumed, so RING rows stay in flight.  The
  // loads are unconditional (no branch for the waitcnt pass to merge over,
  // which would force it to drain every outstanding load): past the block's
  // last row they read gamma instead, an in-bounds, L2-resident stand-in whose
  // values are never used.
  const char* stand_in = static_cast<const char*>(p.gamma);
  auto issue = [&](RowBuf<VPT, DRES>& b, int row) {
    const bool live = row < r1;   // block-uniform
    const int64_t off = static_cast<int64_t>(grow(row)) * h * EB;
    const char* dyp = live ? static_cast<const char*>(p.dy) + off : stand_in;
    const char* zp = live ? static_cast<const char*>(p.z) + off : stand_in;
    const char* drp = DRES && live ? static_cast<const char*>(p.dres) + off : stand_in;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      b.dy[k] = ld16_stream(dyp + vv[k] * 16);
      b.z[k] = ld16_stream(zp + vv[k] * 16);
      if constexpr (DRES) b.dr[k] = ld16_stream(drp + vv[k] * 16);
    }
    const int srow = grow(live ? row : r1 - 1);
    b.mu = ln ? p.mean[srow] : 0.0f;
    b.rs = p.rstd[srow];
    if constexpr (DROP) {
      // Scalar loads only (ragged offsets): no wait on the ring's vector loads.
      const uint64_t g = p.drop ? global_token_of(srow, p.T, p.t, p.rank, p.cu, p.nseq) : 0;
      b.g_lo = static_cast<uint32_t>(g);
      b.g_hi = static_cast<uint32_t>(g >> 32);
    }
  };

  int parity = 0;
  auto process = [&](const RowBuf<VPT, DRES>& b, int row) {
    if (row >= r1) return;   // block-uniform: every thread skips the barrier alike
    const float mu = b.mu;
    const float rs = b.rs;
    // xhat, g and dy of this row stay in registers between the two phases.
    float xh[VPT][V], gg[VPT][V], dyv[VPT][V];
    float part[2] = {0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float zv[V];
      unpack(E{}, b.z[k], zv);
      unpack(E{}, b.dy[k], dyv[k]);
      float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        xh[k][e] = (zv[e] - mu) * rs;
        gg[k][e] = dyv[k][e] * gam[k][e];
        p0 += gg[k][e];
        p1 = __builtin_fmaf(gg[k][e], xh[k][e], p1);
      }
      part[0] += valid[k] ? p0 : 0.0f;
      part[1] += valid[k] ? p1 : 0.0f;
    }
    // One barrier per row; the two LDS slots alternate, so a slot is only
    // rewritten after every wave has passed the barrier of the row between.
    float* slot = red[parity];
    parity ^= 1;
    wave_sum<2>(part);
    if (lane == 0) {
      slot[wave] = part[0];
      slot[16 + wave] = part[1];
    }
    __syncthreads();
    float s1 = slot[0], s2 = slot[16];
    for (int w = 1; w < nwaves; ++w) {   // wave order: the same total in every thread
      s1 += slot[w];
      s2 += slot[16 + w];
    }
    const float c1 = ln ? s1 * inv_h : 0.0f;
    const float c2 = s2 * inv_h;
    const int64_t off = static_cast<int64_t>(grow(row)) * h * EB;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (!valid[k]) continue;
      float dx[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        dx[e] = rs * __builtin_fmaf(-xh[k][e], c2, gg[k][e] - c1);
        dg[k][e] = __builtin_fmaf(dyv[k][e], xh[k][e], dg[k][e]);
        db[k][e] += dyv[k][e];
      }
      if constexpr (DRES) {
        float f[V];
        unpack(E{}, b.dr[k], f);
#pragma unroll
        for (int e = 0; e < V; ++e) dx[e] += f[e];
      }
      st16_dx(static_cast<char*>(p.dx) + off + vv[k] * 16, pack(E{}, dx));
      if constexpr (DROP) {
        // Through the dropout: kept channels times the forward's scale, the
        // forward's own mask (same seed, same global token).
        float dp[V];
        if (p.drop) {
          bool keep[V];
          dropout_keep<V>(static_cast<uint32_t>(vv[k]), b.g_lo, b.g_hi, p.key0, p.key1, p.thr, keep);
#pragma unroll
          for (int e = 0; e < V; ++e) dp[e] = keep[e] ? dx[e] * p.scale : 0.0f;
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) dp[e] = dx[e];
        }
#pragma unroll
        for (int e = 0; e < V; ++e) dbs[k][e] += dp[e];
        st16_dx(static_cast<char*>(p.dpartial) + off + vv[k] * 16, pack(E{}, dp));
      }
    }
  };

  RowBuf<VPT, DRES> ring[RING];
#pragma unroll
  for (int j = 0; j < RING; ++j) issue(ring[j], r0 + j);
  for (int r = r0; r < r1; r += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      process(ring[j], r + j);
      issue(ring[j], r + j + RING);
    }
  }

  // Partial slots: dgamma first, then dbeta and dbias where requested.
  float* ws = p.ws + static_cast<int64_t>(blockIdx.x) * p.ws_bstride;
  auto put = [&](float* dst, const float (&a)[V], int k) {
#pragma unroll
    for (int e0 = 0; e0 < V; e0 += 4)
      st16_ws(dst + vv[k] * V + e0, u32x4{__float_as_uint(a[e0]), __float_as_uint(a[e0 + 1]),
                                          __float_as_uint(a[e0 + 2]), __float_as_uint(a[e0 + 3])});
  };
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (!valid[k]) continue;
    put(ws, dg[k], k);
    if (p.slot_dbeta > 0) put(ws + p.slot_dbeta * p.ws_sstride, db[k], k);
    if constexpr (DROP) {
      if (p.slot_dbias > 0) put(ws + p.slot_dbias * p.ws_sstride, dbs[k], k);
    }
  }
}

template <class E, int VPT, int RING, bool DRES, bool DROP, int MAXBS>
__global__ __launch_bounds__(MAXBS) void sp_region_bwd_rows_kernel(const BwdParams p) {
  rows_stage<E, VPT, RING, DRES, DROP>(p);
}

// Stage 2: the G partials of each column are summed in a fixed tree: 32
// groups of consecutive partials, each summed in ascending block order, then
// the 32 group sums in group order.  The tree depends only on G.
#ifndef SPR_BWD_GROUPS
#define SPR_BWD_GROUPS 32   // 16 and 64 measured slower (latency-bound loads / half-line segments)
#endif
constexpr int kGroups = SPR_BWD_GROUPS;
static_assert(kBwdMaxBlocks % kGroups == 0, "groups must split the partials evenly");

// Column quads [q0, q1) of the NP partial slots (block b's slot j at
// ws + b*bstride + j*sstride) into out[j], cw = blockDim.x / kGroups quads at a
// time (cw <= CQMAX); thread (group, quad) = (threadIdx.x / cw,
// threadIdx.x % cw).  Every thread of the block calls this (it has barriers).
template <int CQMAX, int NP>
__device__ __forceinline__ void reduce_cols(const float* __restrict__ ws, int G, int64_t bstride, int64_t sstride,
                                            int q0, int q1, bool accumulate,
                                            float* const (&out)[NP]) {
  __shared__ float4 part[NP][kGroups][CQMAX];
  const int cw = static_cast<int>(blockDim.x) / kGroups;
  const int cq = threadIdx.x % cw;
  const int grp = threadIdx.x / cw;   // < kGroups since blockDim.x = kGroups * cw
  // At most kBwdMaxBlocks / kGroups partials per group: all loads in flight
  // together, then summed in ascending block order.
  constexpr int kPer = kBwdMaxBlocks / kGroups;
  const int g0 = grp * G / kGroups, g1 = (grp + 1) * G / kGroups;
  for (int qb = q0; qb < q1; qb += cw) {   // block-uniform
    const int c4 = qb + cq;
    float4 sum[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) sum[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (G > 0) {   // block-uniform; G == 0: no partials exist (the sums stay 0)
      // Every load is unconditional, from a clamped in-bounds address (a
      // load under a branch would make the waitcnt pass serialise them);
      // the bounds are applied by the selects below.
      const int cc = c4 < q1 ? c4 : q1 - 1;
      float4 a[NP][kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int gi = g0 + i < G ? g0 + i : G - 1;
#pragma unroll
        for (int j = 0; j < NP; ++j)
          a[j][i] = reinterpret_cast<const float4*>(ws + gi * bstride + j * sstride)[cc];
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool in = g0 + i < g1;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          sum[j].x = in ? sum[j].x + a[j][i].x : sum[j].x;
          sum[j].y = in ? sum[j].y + a[j][i].y : sum[j].y;
          sum[j].z = in ? sum[j].z + a[j][i].z : sum[j].z;
          sum[j].w = in ? sum[j].w + a[j][i].w : sum[j].w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) part[j][grp][cq] = sum[j];
    __syncthreads();
    if (grp == 0 && c4 < q1) {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        float4 tot = part[j][0][cq];
        for (int i = 1; i < kGroups; ++i) {
          const float4 x = part[j][i][cq];
          tot.x += x.x; tot.y += x.y; tot.z += x.z; tot.w += x.w;
        }
        if (accumulate) {   // main gradient: old + this call's sum, one rounding
          const float4 m = reinterpret_cast<const float4*>(out[j])[c4];
          tot.x = m.x + tot.x; tot.y = m.y + tot.y; tot.z = m.z + tot.z; tot.w = m.w + tot.w;
        }
        reinterpret_cast<float4*>(out[j])[c4] = tot;
      }
    }
    __syncthreads();   // part is rewritten by the next chunk
  }
}

#ifndef SPR_COLS_QPB
#define SPR_COLS_QPB 8    // column quads per block of stage 2: 128-byte segments of each partial
#endif
constexpr int kColQuads = SPR_COLS_QPB;

// Outputs of stage 2, slot order (dgamma, then dbeta / dbias where requested).
struct ColOut {
  float* p[3];
  int32_t accumulate;   // nonzero: out = old + sum
};

template <int NP>
__global__ __launch_bounds__(kColQuads * kGroups) void sp_region_bwd_cols_kernel(const float* __restrict__ ws, int G,
                                                                                 int h, int64_t bstride,
                                                                                 int64_t sstride, ColOut o) {
  const int nq = h / 4;
  const int q0 = blockIdx.x * kColQuads;
  float* out[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) out[j] = o.p[j];
  reduce_cols<kColQuads, NP>(ws, G, bstride, sstride, q0, q0 + kColQuads < nq ? q0 + kColQuads : nq,
                             o.accumulate != 0, out);
}

#ifndef SPR_BWD_MAX_THREADS
#define SPR_BWD_MAX_THREADS 512   // block size cap of the row stage
#endif
#ifndef SPR_BWD_RING
#define SPR_BWD_RING 4            // rows in flight per block
#endif

// Ring depth per vectors-per-thread, so the packed ring fits the VGPRs the
// block size leaves (wider rows keep fewer rows in flight).
template <int VPT, int MAXBS, bool DROP>
constexpr int ring_for() {
  return VPT == 1 ? SPR_BWD_RING : (VPT == 2 && MAXBS <= 512 ? SPR_BWD_RING : (VPT == 2 ? 2 : 1));
}

hipError_t launch_cols(const BwdParams& p, hipStream_t stream) {
  ColOut o{{p.dgamma, nullptr, nullptr}, p.accumulate};
  int np = 1;
  if (p.slot_dbeta > 0) o.p[np++] = p.dbeta;
  if (p.slot_dbias > 0) o.p[np++] = p.dbias;
  const int nq = p.h / 4;
  const dim3 grid((nq + kColQuads - 1) / kColQuads), block(kColQuads * kGroups);
  const KernelRole role = p.G > 0 ? KernelRole::kLast : KernelRole::kOnly;
  const float* ws = p.ws;
  switch (np) {
    case 1: launch_kernel(sp_region_bwd_cols_kernel<1>, grid, block, stream, role, ws, p.G, p.h, p.ws_bstride, p.ws_sstride, o); break;
    case 2: launch_kernel(sp_region_bwd_cols_kernel<2>, grid, block, stream, role, ws, p.G, p.h, p.ws_bstride, p.ws_sstride, o); break;
    default: launch_kernel(sp_region_bwd_cols_kernel<3>, grid, block, stream, role, ws, p.G, p.h, p.ws_bstride, p.ws_sstride, o); break;
  }
  return hipGetLastError();
}

template <class E, int VPT, bool DRES, bool DROP>
hipError_t launch_stages(const BwdParams& p, const Shape& sh, hipStream_t stream) {
  constexpr int MAXBS = SPR_BWD_MAX_THREADS;
  constexpr int RING = ring_for<VPT, MAXBS, DROP>();
  const dim3 grid(static_cast<unsigned>(p.G)), block(sh.threads);
  launch_kernel(sp_region_bwd_rows_kernel<E, VPT, RING, DRES, DROP, MAXBS>, grid, block, stream, KernelRole::kFirst, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_cols(p, stream);
}

template <class E, bool DROP>
hipError_t launch_rows(const BwdParams& p, const Shape& sh, hipStream_t stream) {
  const bool dres = p.dres != nullptr;
  switch (sh.vpt) {
    case 1: return dres ? launch_stages<E, 1, true, DROP>(p, sh, stream) : launch_stages<E, 1, false, DROP>(p, sh, stream);
    case 2: return dres ? launch_stages<E, 2, true, DROP>(p, sh, stream) : launch_stages<E, 2, false, DROP>(p, sh, stream);
    case 4: return dres ? launch_stages<E, 4, true, DROP>(p, sh, stream) : launch_stages<E, 4, false, DROP>(p, sh, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Smallest VPT in {1, 2, 4} within SPR_BWD_MAX_THREADS threads
// (h = 8192 bf16 -> 2 x 512 at the default cap of 512).
Shape bwd_shape(int h, int dtype) {
  const int vec = dtype == 1 ? 8 : 4;
  const int nvec = h / vec;
  for (int vpt : {1, 2, 4}) {
    const int need = (nvec + vpt - 1) / vpt;
    if (need <= SPR_BWD_MAX_THREADS) return Shape{vpt, ((need + 63) / 64) * 64};
  }
  return Shape{0, 0};
}

hipError_t launch_bwd(const BwdParams& params, int dtype, hipStream_t stream) {
  BwdParams p = params;
  p.ws_sstride = ws_slot_stride(p.h);
  p.ws_bstride = ws_block_stride(p.h, p.nparts);
  if (p.G > 0) {
    const Shape sh = bwd_shape(p.h, dtype);
    const bool drop = p.dpartial != nullptr;
    if (dtype == 1) return drop ? launch_rows<Bf16, true>(p, sh, stream) : launch_rows<Bf16, false>(p, sh, stream);
    return drop ? launch_rows<F32, true>(p, sh, stream) : launch_rows<F32, false>(p, sh, stream);
  }
  // No rows: every output is 0 (every group of partials is empty); an
  // accumulating call adds nothing and launches nothing.
  if (p.accumulate) return hipSuccess;
  return launch_cols(p, stream);
}

}  // namespace spr

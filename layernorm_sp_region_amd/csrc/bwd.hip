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
// Rows.  G blocks; block b owns rows b, b + G, b + 2G, ... (interleaved, so
// the rows the G blocks read at one moment form one contiguous band of
// memory).  Each thread owns a fixed set of columns: it keeps their gamma and
// their dgamma/dbeta (/dbias) running sums in registers across rows.  A
// block of at most R rows loads them all at once and takes ONE barrier for
// their row sums; longer blocks stream rows through a ring.  (At the 70B
// shard, 8 rows per block, the two forms measured the same, 24.5-25.0 us for
// the rows kernel against 24.3 us for a ring of 4 with a barrier per row
// (rocprofv3), before the row sums' LDS reads were batched (now 23.2 us); the
// one-barrier form is what the one-launch small-shard path is built on.)
//
// Column sums, in one fixed tree whatever the path, so results are bitwise
// reproducible: row block b's rows in row order; 32 groups of blocks (g,
// g + 32, ...), each summed in ascending block order; then the 32 group sums
// in group order.  Two ways to evaluate it:
//   * partials (any shard): every row block writes its column sums to the
//     workspace and a second kernel sums them down the tree;
//   * direct (small shards without the dropout, one launch): column blocks
//     beside the row blocks evaluate the same tree from dy, z, mean and rstd
//     themselves, so no partial is written and nothing waits on another
//     block.

#include <atomic>

#include "spr_device.h"
#include "spr_internal.h"

namespace spr {
namespace {

// One row of a [T][h] tensor as a buffer resource of `bytes` bytes (0 makes
// every load of it out of range: zeros, no memory access); loads are
// nontemporal (streamed once).
constexpr int kCpolNontemporal = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const char* row, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16_row(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kCpolNontemporal));
}

#ifndef SPR_BWD_MAX_THREADS
#define SPR_BWD_MAX_THREADS 512   // block size cap of the row stage
#endif

// Packed loads of N rows: VPT vectors of dy, z (and dres) per thread per
// row.  A row's statistics travel with its data: every lane loads the same
// mean/rstd (one broadcast request per wave), so waiting for a row never
// waits on loads issued after it (vmcnt completes in issue order).
template <int VPT, int N, bool DRES>
struct Rows {
  u32x4 dy[N][VPT], z[N][VPT], dr[DRES ? N : 1][DRES ? VPT : 1];
  float mu[N], rs[N];
  uint32_t g_lo[N], g_hi[N];   // global token index of each row (dropout backward)
};

// Column state of one block: the running sums of its columns (and their
// gamma, unpacked, when it fits the registers).
template <int VPT, int V, bool DROP>
struct ColSums {
  static constexpr bool kGammaLds = VPT >= 4;   // wide rows keep gamma packed in LDS
  int vv[VPT];       // vector index of slot k (clamped to the row)
  bool valid[VPT];   // slot k holds a vector of the row
  float gam[kGammaLds ? 1 : VPT][V], dg[VPT][V], db[VPT][V];
  float dbs[DROP ? VPT : 1][V];
};

// Rows of block b: local row li is global row b + li*G (G <= T, so every
// block has at least one row), r1 of them.
__device__ __forceinline__ int block_rows(const BwdParams& p) {
  return static_cast<int>((p.T - blockIdx.x + p.G - 1) / p.G);
}

template <class E, int VPT, bool DROP>
__device__ __forceinline__ void init_cols(const BwdParams& p, ColSums<VPT, E::kVec, DROP>& cs,
                                          u32x4 (*gl)[SPR_BWD_MAX_THREADS]) {
  constexpr int V = E::kVec;
  const int tid = threadIdx.x;
  const int nvec = p.h / V;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int v = tid + k * static_cast<int>(blockDim.x);
    cs.valid[k] = v < nvec;
    cs.vv[k] = cs.valid[k] ? v : nvec - 1;   // clamped: loads stay in bounds
    const u32x4 gv = ld16(static_cast<const char*>(p.gamma) + cs.vv[k] * 16);
    if constexpr (ColSums<VPT, V, DROP>::kGammaLds) gl[k][tid] = gv;
    else unpack(E{}, gv, cs.gam[k]);
#pragma unroll
    for (int e = 0; e < V; ++e) cs.dg[k][e] = cs.db[k][e] = 0.0f;
    if constexpr (DROP) {
#pragma unroll
      for (int e = 0; e < V; ++e) cs.dbs[k][e] = 0.0f;
    }
  }
}

template <class E, int VPT, bool DROP>
__device__ __forceinline__ void gamma_of(const ColSums<VPT, E::kVec, DROP>& cs, u32x4 (*gl)[SPR_BWD_MAX_THREADS],
                                         int k, float (&g)[E::kVec]) {
  if constexpr (ColSums<VPT, E::kVec, DROP>::kGammaLds) {
    unpack(E{}, gl[k][threadIdx.x], g);
  } else {
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) g[e] = cs.gam[k][e];
  }
}

// Issue the loads of local rows li0 .. li0+N-1.  Every load is unconditional
// (no branch for the waitcnt pass to merge over, which would make it drain
// every outstanding load): each row is read through a buffer resource based
// at the row, whose size is the row's for a row of the block and 0 past the
// block's last row -- those loads are out of range, so the hardware returns
// zeros without touching memory.
template <class E, int VPT, int N, bool DRES, bool DROP>
__device__ __forceinline__ void issue_rows(const BwdParams& p, const ColSums<VPT, E::kVec, DROP>& cs,
                                           Rows<VPT, N, DRES>& b, int li0, int r1) {
  constexpr int EB = 16 / E::kVec;
  const int h = p.h;
  const int bx = blockIdx.x, G = p.G;
  const bool ln = p.norm == 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int li = li0 + j;
    const bool live = li < r1;   // block-uniform
    const int lc = live ? li : r1 - 1;
    const int64_t off = static_cast<int64_t>(bx + static_cast<int64_t>(lc) * G) * h * EB;
    const int bytes = live ? h * EB : 0;
    const auto rdy = row_rsrc(static_cast<const char*>(p.dy) + off, bytes);
    const auto rz = row_rsrc(static_cast<const char*>(p.z) + off, bytes);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      b.dy[j][k] = ld16_row(rdy, cs.vv[k] * 16);
      b.z[j][k] = ld16_row(rz, cs.vv[k] * 16);
    }
    if constexpr (DRES) {
      const auto rdr = row_rsrc(static_cast<const char*>(p.dres) + off, bytes);
#pragma unroll
      for (int k = 0; k < VPT; ++k) b.dr[j][k] = ld16_row(rdr, cs.vv[k] * 16);
    }
    const int64_t srow = bx + static_cast<int64_t>(lc) * G;
    b.mu[j] = ln ? p.mean[srow] : 0.0f;
    b.rs[j] = p.rstd[srow];
    if constexpr (DROP) {
      // Scalar loads only (ragged offsets): no wait on the rows' vector loads.
      const uint64_t g = p.drop ? global_token_of(srow, p.T, p.t, p.rank, p.cu, p.nseq) : 0;
      b.g_lo[j] = static_cast<uint32_t>(g);
      b.g_hi[j] = static_cast<uint32_t>(g >> 32);
    }
  }
}

// Rows li0 .. li0+N-1 (those below r1): their N pairs of row sums (g,
// g*xhat) in one block reduction, then dx (and dpartial) stored and, with
// COLS, the column sums advanced, in row order.
// slot: LDS of 2*N*16 floats, alternated between consecutive calls by the
// caller (one barrier per call).
template <class E, int VPT, int N, bool DRES, bool DROP, bool COLS = true>
__device__ __forceinline__ void finish_rows(const BwdParams& p, ColSums<VPT, E::kVec, DROP>& cs,
                                            u32x4 (*gl)[SPR_BWD_MAX_THREADS], Rows<VPT, N, DRES>& b, int li0,
                                            int r1, float (*slot)[N][16]) {
  constexpr int V = E::kVec;
  constexpr int EB = 16 / V;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
  const int h = p.h;
  const bool ln = p.norm == 0;
  const float inv_h = 1.0f / static_cast<float>(h);
  float part[2 * N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    part[2 * j] = part[2 * j + 1] = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float zv[V], dyv[V], gm[V];
      unpack(E{}, b.z[j][k], zv);
      unpack(E{}, b.dy[j][k], dyv);
      gamma_of<E, VPT, DROP>(cs, gl, k, gm);
      float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = (zv[e] - b.mu[j]) * b.rs[j];
        const float gg = dyv[e] * gm[e];
        p0 += gg;
        p1 = __builtin_fmaf(gg, xh, p1);
      }
      part[2 * j] += cs.valid[k] ? p0 : 0.0f;
      part[2 * j + 1] += cs.valid[k] ? p1 : 0.0f;
    }
  }
  wave_sum<2 * N>(part);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      slot[0][j][wave] = part[2 * j];
      slot[1][j][wave] = part[2 * j + 1];
    }
  }
  __syncthreads();
  // Several rows: the packed rows are unpacked again below rather than kept
  // unpacked across the barrier (N rows of unpacked floats would not fit the
  // registers).  One row (the ring): the compiler may keep them unpacked.
  if constexpr (N > 1) {
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        asm volatile("" : "+v"(b.dy[j][k]));
        asm volatile("" : "+v"(b.z[j][k]));
      }
  }
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int li = li0 + j;
    if (li >= r1) continue;   // block-uniform
    // Wave order: the same total in every thread.  Every wave slot's LDS
    // read is issued before the adds (the slots past nwaves are read and
    // not added), rather than one read per add.
    constexpr int kMaxWaves = SPR_BWD_MAX_THREADS / kWave;
    float a1[kMaxWaves], a2[kMaxWaves];
#pragma unroll
    for (int w = 0; w < kMaxWaves; ++w) {
      a1[w] = slot[0][j][w];
      a2[w] = slot[1][j][w];
    }
    float s1 = a1[0], s2 = a2[0];
#pragma unroll
    for (int w = 1; w < kMaxWaves; ++w) {
      s1 = w < nwaves ? s1 + a1[w] : s1;
      s2 = w < nwaves ? s2 + a2[w] : s2;
    }
    const float c1 = ln ? s1 * inv_h : 0.0f;
    const float c2 = s2 * inv_h;
    const int64_t off = static_cast<int64_t>(blockIdx.x + static_cast<int64_t>(li) * p.G) * h * EB;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (!cs.valid[k]) continue;
      float zv[V], dyv[V], gm[V], dx[V];
      unpack(E{}, b.z[j][k], zv);
      unpack(E{}, b.dy[j][k], dyv);
      gamma_of<E, VPT, DROP>(cs, gl, k, gm);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = (zv[e] - b.mu[j]) * b.rs[j];
        const float gg = dyv[e] * gm[e];
        dx[e] = b.rs[j] * __builtin_fmaf(-xh, c2, gg - c1);
        if constexpr (COLS) {
          cs.dg[k][e] = __builtin_fmaf(dyv[e], xh, cs.dg[k][e]);
          cs.db[k][e] += dyv[e];
        }
      }
      if constexpr (DRES) {
        float f[V];
        unpack(E{}, b.dr[j][k], f);
#pragma unroll
        for (int e = 0; e < V; ++e) dx[e] += f[e];
      }
      // Nontemporal (measured: the next kernel no longer pays for writing
      // back dirty dx lines).
      st16_stream(static_cast<char*>(p.dx) + off + cs.vv[k] * 16, pack(E{}, dx));
      if constexpr (DROP) {
        // Through the dropout: kept channels times the forward's scale, the
        // forward's own mask (same seed, same global token).
        float dp[V];
        if (p.drop) {
          bool keep[V];
          dropout_keep<V>(static_cast<uint32_t>(cs.vv[k]), b.g_lo[j], b.g_hi[j], p.key0, p.key1, p.thr, keep);
#pragma unroll
          for (int e = 0; e < V; ++e) dp[e] = keep[e] ? dx[e] * p.scale : 0.0f;
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) dp[e] = dx[e];
        }
#pragma unroll
        for (int e = 0; e < V; ++e) cs.dbs[k][e] += dp[e];
        st16_stream(static_cast<char*>(p.dpartial) + off + cs.vv[k] * 16, pack(E{}, dp));
      }
    }
  }
}

// The rows of block blockIdx.x, R at a time (SHORT: the block has at most R
// rows, all loaded at once, one barrier -- straight-line code), or one at a
// time through a ring of R rows in flight (long shards).  dx (and dpartial)
// stored; then store_cols() with the block's column sums complete.
template <class E, int VPT, int R, bool SHORT, bool DRES, bool DROP, class Hook, bool COLS = true>
__device__ __forceinline__ void rows_phase(const BwdParams& p, ColSums<VPT, E::kVec, DROP>& cs,
                                           const Hook& store_cols) {
  __shared__ float red[2][2][SHORT ? R : 1][16];   // [parity][sum][row][wave]
  __shared__ u32x4 gam_lds[ColSums<VPT, E::kVec, DROP>::kGammaLds ? VPT : 1][SPR_BWD_MAX_THREADS];
  init_cols<E, VPT, DROP>(p, cs, gam_lds);
  const int r1 = block_rows(p);
  if constexpr (SHORT) {
    Rows<VPT, R, DRES> b;
    issue_rows<E, VPT, R, DRES, DROP>(p, cs, b, 0, r1);
    finish_rows<E, VPT, R, DRES, DROP, COLS>(p, cs, gam_lds, b, 0, r1, red[0]);
    if constexpr (COLS) store_cols();
  } else {
    // A ring of R single rows: row li + R is issued as soon as row li has
    // been consumed; one barrier per row, the two LDS slots alternating.
    Rows<VPT, 1, DRES> ring[R];
#pragma unroll
    for (int j = 0; j < R; ++j) issue_rows<E, VPT, 1, DRES, DROP>(p, cs, ring[j], j, r1);
    int parity = 0;
    for (int li = 0; li < r1; li += R) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        if (li + j < r1) {   // block-uniform
          finish_rows<E, VPT, 1, DRES, DROP, COLS>(p, cs, gam_lds, ring[j], li + j, r1, red[parity]);
          parity ^= 1;
        }
        issue_rows<E, VPT, 1, DRES, DROP>(p, cs, ring[j], li + j + R, r1);
      }
    }
    if constexpr (COLS) store_cols();
  }
}

// Block blockIdx.x's partial slots (dgamma first, then dbeta and dbias where
// requested) at ws + b*bstride + slot*sstride.
template <int VPT, int V, bool DROP>
__device__ __forceinline__ void store_partials(const BwdParams& p, const ColSums<VPT, V, DROP>& cs) {
  float* base = p.ws + static_cast<int64_t>(blockIdx.x) * p.ws_bstride;
  auto put = [&](int slot, const float (&a)[V], int k) {
    float* dst = base + slot * p.ws_sstride + cs.vv[k] * V;
#pragma unroll
    for (int e0 = 0; e0 < V; e0 += 4) {
      const u32x4 v{__float_as_uint(a[e0]), __float_as_uint(a[e0 + 1]), __float_as_uint(a[e0 + 2]),
                    __float_as_uint(a[e0 + 3])};
      st16(dst + e0, v);
    }
  };
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (!cs.valid[k]) continue;
    put(0, cs.dg[k], k);
    if (p.slot_dbeta > 0) put(p.slot_dbeta, cs.db[k], k);
    if constexpr (DROP) {
      if (p.slot_dbias > 0) put(p.slot_dbias, cs.dbs[k], k);
    }
  }
}

// The fixed tree's shape: 32 groups, group g holding the partials of blocks
// g, g + 32, g + 64, ... (blocks are dealt to the 8 XCDs round-robin, so a
// group's blocks share an XCD).  The tree depends only on G.
constexpr int kGroups = 32;
static_assert(kBwdMaxBlocks % kGroups == 0, "groups must split the partials evenly");
constexpr int kPerGroup = kBwdMaxBlocks / kGroups;   // partials per group, at most

// Outputs of the column sums, slot order (dgamma, then dbeta / dbias where requested).
struct ColOut {
  float* p[3];
  int32_t np;           // slots in use (1..3)
  int32_t accumulate;   // nonzero: out = old + sum
};

// Row block kernel of the partials path: dx (and dpartial), then the block's
// column sums to the workspace.
template <class E, int VPT, int R, bool SHORT, bool DRES, bool DROP, int MAXBS>
__global__ __launch_bounds__(MAXBS) void sp_region_bwd_rows_kernel(const BwdParams p) {
  ColSums<VPT, E::kVec, DROP> cs;
  rows_phase<E, VPT, R, SHORT, DRES, DROP>(p, cs, [&] { store_partials<VPT, E::kVec, DROP>(p, cs); });
}

// Second kernel of the partials path: column quads [q0, q0 + kColQuads) of
// the NP partial slots into o.p[j], thread (group, quad) = (threadIdx.x /
// kColQuads, threadIdx.x % kColQuads).  NP >= o.np is the compile-time slot
// count: slots o.np..NP-1 re-read slot 0 (the same addresses, no extra
// traffic) and are never stored.
#ifndef SPR_COLS_QPB
#define SPR_COLS_QPB 8    // column quads per block: 128-byte segments
#endif
constexpr int kColQuads = SPR_COLS_QPB;

template <int NP>
__global__ __launch_bounds__(kColQuads * kGroups) void sp_region_bwd_cols_kernel(const float* __restrict__ ws, int G,
                                                                                 int h, int64_t bstride,
                                                                                 int64_t sstride, ColOut o) {
  __shared__ float4 part[NP][kGroups][kColQuads];
  const int nq = h / 4;
  const int cq = threadIdx.x % kColQuads;
  const int grp = threadIdx.x / kColQuads;
  const int c4 = blockIdx.x * kColQuads + cq;
  int64_t soff[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) soff[j] = (j < o.np ? j : 0) * sstride;
  // Every load is unconditional, from a clamped in-bounds address (a load
  // under a branch would make the waitcnt pass serialise them); the bounds
  // are applied by the selects below.  G == 0: no partials (sums stay 0).
  const int cc = c4 < nq ? c4 : nq - 1;
  float4 a[NP][kPerGroup];
#pragma unroll
  for (int i = 0; i < kPerGroup; ++i) {
    const int b = grp + i * kGroups;
    const int gi = b < G ? b : (G > 0 ? G - 1 : 0);
#pragma unroll
    for (int j = 0; j < NP; ++j) a[j][i] = reinterpret_cast<const float4*>(ws + gi * bstride + soff[j] + 4 * cc)[0];
  }
  float4 sum[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) sum[j] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < kPerGroup; ++i) {
    const bool in = grp + i * kGroups < G;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      sum[j].x = in ? sum[j].x + a[j][i].x : sum[j].x;
      sum[j].y = in ? sum[j].y + a[j][i].y : sum[j].y;
      sum[j].z = in ? sum[j].z + a[j][i].z : sum[j].z;
      sum[j].w = in ? sum[j].w + a[j][i].w : sum[j].w;
    }
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) part[j][grp][cq] = sum[j];
  __syncthreads();
  // Group row j of the threads sums slot j over the 32 groups, in group
  // order: all 32 LDS reads issued first, then the chain of adds (read by
  // read, each add waited on its read: 1.5 us at the 70B shard).
  if (grp < NP && grp < o.np && c4 < nq) {
    const int j = grp;
    float4 x[kGroups];
#pragma unroll
    for (int i = 0; i < kGroups; ++i) x[i] = part[j][i][cq];
    float4 tot = x[0];
#pragma unroll
    for (int i = 1; i < kGroups; ++i) {
      tot.x += x[i].x; tot.y += x[i].y; tot.z += x[i].z; tot.w += x[i].w;
    }
    float* out = j == 0 ? o.p[0] : (j == 1 ? o.p[1] : o.p[2]);
    if (o.accumulate) {   // main gradient: old + this call's sum, one rounding
      const float4 m = reinterpret_cast<const float4*>(out)[c4];
      tot.x = m.x + tot.x; tot.y = m.y + tot.y; tot.z = m.z + tot.z; tot.w = m.w + tot.w;
    }
    reinterpret_cast<float4*>(out)[c4] = tot;
  }
}

// The direct path (small shards, no dropout): the same launch holds the G
// row blocks, which store dx and keep no column sums, and column blocks,
// each of which sums dgamma/dbeta for kDirectLanes vectors of columns straight
// from dy, z, mean and rstd.  No partials leave the block, so there is no
// workspace, flag or second launch -- and the column blocks reproduce the
// partials path's tree exactly (row block b's rows in order, from 0; the 32
// groups of blocks g, g + 32, ... in order, from 0; then the groups in
// order), so the result is bitwise the same whichever path runs.
#ifndef SPR_BWD_DIRECT_LANES
#define SPR_BWD_DIRECT_LANES 4
#endif
constexpr int kDirectLanes = SPR_BWD_DIRECT_LANES;   // 16-byte vectors per row segment of a column block
constexpr int kDirectMaxBlocks = 128;   // row blocks the column blocks' LDS holds

// Column slice of column block c (a bijection on the column blocks).  Within
// each run of 16 column blocks, blocks c and c + 8 take the two adjacent
// slices that share each row's 128-byte line; under round-robin dispatch over
// the 8 XCDs the two blocks sit on one XCD, so the second read of the line
// hits its L2 (measured at 512 x 4096 bf16: 9.2 -> 7.7 us, where consecutive
// slices on consecutive blocks fetched every line twice).  Which block sums
// which slice does not change any sum's order, so placement never changes
// the bits.  Blocks past the last full run keep their own slice.
__device__ __forceinline__ int col_slice(int c, int ncb) {
  if (c >= ncb / 16 * 16) return c;
  const int r = c % 16;
  return c - r + (r < 8 ? 2 * r : 2 * (r - 8) + 1);
}

template <class E, int R>
__device__ __forceinline__ void col_block(const BwdParams& p, const ColOut& o, int cb) {
  constexpr int V = E::kVec, EB = 16 / V, L = kDirectLanes, W = L * V;
  __shared__ float sb[2][kDirectMaxBlocks][W];   // [dgamma|dbeta][row block][column]
  __shared__ float grp[2][kGroups][W];
  const int G = p.G, h = p.h, nvec = h / V;
  const int c = col_slice(cb, (nvec + L - 1) / L);
  const int t = threadIdx.x, nt = static_cast<int>(blockDim.x);
  const int lc = t % L, rl = t / L, RL = nt / L;
  const int v = c * L + lc;
  const int64_t voff = static_cast<int64_t>(v < nvec ? v : nvec - 1) * 16;
  const bool ln = p.norm == 0;
  // Row block b's sums, one row block per row lane at a time: its (at most
  // R) rows loaded together (rows past the block's last re-read that row and
  // are not summed), then summed in row order.  The rows differ across the
  // lanes of a wave, so these are plain per-lane loads.
  for (int b = rl; b < G; b += RL) {
    const int r1 = static_cast<int>((p.T - b + G - 1) / G);
    u32x4 dy[R], z[R];
    float mu[R], rs[R];
#pragma unroll
    for (int li = 0; li < R; ++li) {
      const int64_t row = b + static_cast<int64_t>(li < r1 ? li : r1 - 1) * G;
      const int64_t off = row * h * EB + voff;
      // Ordinary loads: the line stays in L2 for the partner block.
      dy[li] = ld16(static_cast<const char*>(p.dy) + off);
      z[li] = ld16(static_cast<const char*>(p.z) + off);
      mu[li] = ln ? p.mean[row] : 0.0f;
      rs[li] = p.rstd[row];
    }
    float dg[V], db[V];
#pragma unroll
    for (int e = 0; e < V; ++e) dg[e] = db[e] = 0.0f;
#pragma unroll
    for (int li = 0; li < R; ++li) {
      if (li >= r1) break;
      float zv[V], dyv[V];
      unpack(E{}, z[li], zv);
      unpack(E{}, dy[li], dyv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = (zv[e] - mu[li]) * rs[li];
        dg[e] = __builtin_fmaf(dyv[e], xh, dg[e]);
        db[e] += dyv[e];
      }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      sb[0][b][lc * V + e] = dg[e];
      sb[1][b][lc * V + e] = db[e];
    }
  }
  __syncthreads();
  // The LDS reads of each sum are issued before its chain of adds (blocks
  // past G read block 0's slot and add nothing).
  for (int q = t; q < kGroups * W; q += nt) {
    const int g = q / W, col = q % W;
    float x0[kPerGroup], x1[kPerGroup];
#pragma unroll
    for (int i = 0; i < kPerGroup; ++i) {
      const int b = g + i * kGroups;
      x0[i] = sb[0][b < G ? b : 0][col];
      x1[i] = sb[1][b < G ? b : 0][col];
    }
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < kPerGroup; ++i) {
      const bool in = g + i * kGroups < G;
      s0 = in ? s0 + x0[i] : s0;
      s1 = in ? s1 + x1[i] : s1;
    }
    grp[0][g][col] = s0;
    grp[1][g][col] = s1;
  }
  __syncthreads();
  for (int q = t; q < W * o.np; q += nt) {
    const int j = q / W, col = q % W;
    const int64_t gc = static_cast<int64_t>(c) * W + col;
    if (gc >= h) continue;
    float x[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) x[g] = grp[j][g][col];
    float tot = x[0];
#pragma unroll
    for (int g = 1; g < kGroups; ++g) tot += x[g];
    float* out = j == 0 ? o.p[0] : o.p[1];
    if (o.accumulate) tot = out[gc] + tot;
    out[gc] = tot;
  }
}

// Blocks [0, G): rows (SHORT, at most R each, no column sums; with DROP they
// also write dpartial); blocks [G, G + ceil(h / (kDirectLanes * V))):
// columns, dgamma and dbeta only (dbias needs the row sums, so a call that
// wants it takes the partials path).  Nothing waits on another block.
template <class E, int VPT, int R, bool DRES, bool DROP, int MAXBS>
__global__ __launch_bounds__(MAXBS) void sp_region_bwd_direct_kernel(const BwdParams p, const ColOut o) {
  if (static_cast<int>(blockIdx.x) >= p.G) {
    col_block<E, R>(p, o, static_cast<int>(blockIdx.x) - p.G);
    return;
  }
  ColSums<VPT, E::kVec, DROP> cs;
  rows_phase<E, VPT, R, true, DRES, DROP, int, false>(p, cs, 0);
}

// Rows in flight for VPT vectors per thread: the packed rows take at most
// 128 VGPRs; 96 with dres, 64 at 4 vectors per thread or for the dropout
// backward's extra state, 32 for both (beyond those budgets the kernels
// spill).  A block of at most that many rows runs straight-line code (all
// its rows loaded at once, one barrier); longer ones stream their rows
// through a ring of at most 4.
#ifndef SPR_BWD_MAX_R
#define SPR_BWD_MAX_R 8
#endif

template <int VPT, bool DRES, bool DROP>
constexpr int rows_in_flight() {
  constexpr int budget = DROP ? (VPT >= 4 ? 32 : 64) : (DRES ? 96 : (VPT >= 4 ? 64 : 128));
  constexpr int per_row = VPT * (DRES ? 3 : 2) * 4;
  constexpr int r = budget / per_row;
  return r < 1 ? 1 : (r > SPR_BWD_MAX_R ? SPR_BWD_MAX_R : r);
}
template <int VPT, bool DRES, bool DROP>
constexpr int ring_rows() {
  constexpr int r = rows_in_flight<VPT, DRES, DROP>();
  return r > 4 ? 4 : r;
}

hipError_t launch_cols(const BwdParams& p, const ColOut& o, int np, hipStream_t stream) {
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

std::atomic<int> g_max_launches{1};   // sp_region_set_bwd_launches

// Compute units of the device that runs `stream`, cached per device (0 if
// unknown: the partials path is then taken).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus(hipStream_t stream) {
  int dev = 0;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return 0;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return 0;
  }
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <class E, int VPT, bool DRES, bool DROP>
hipError_t launch_rows(const BwdParams& p, const ColOut& o, int np, const Shape& sh, hipStream_t stream) {
  constexpr int MAXBS = SPR_BWD_MAX_THREADS;
  constexpr int RS = rows_in_flight<VPT, DRES, DROP>();
  constexpr int RR = ring_rows<VPT, DRES, DROP>();
  const dim3 grid(static_cast<unsigned>(p.G)), block(sh.threads);
  const int64_t rows_per_block = (p.T + p.G - 1) / p.G;
  {
    // The direct path when the row blocks are short enough, every block of
    // the launch can be resident at once, and no dbias is wanted (measured at
    // s = h = 4096, t = 8, 512 local tokens: 128 row + 128 column blocks,
    // 7.8-8.3 us against 15.9 us for the partials path; the dropout backward
    // 8.7 against 16.8 us).
    constexpr int RD = RS < 4 ? RS : 4;
    const int gcols = (p.h / E::kVec + kDirectLanes - 1) / kDirectLanes;
    const bool no_dbias = !DROP || p.slot_dbias == 0;
    if (no_dbias && g_max_launches.load(std::memory_order_relaxed) == 1 && rows_per_block <= RD &&
        p.G <= kDirectMaxBlocks && p.G + gcols <= device_cus(stream)) {
      launch_kernel(sp_region_bwd_direct_kernel<E, VPT, RD, DRES, DROP, MAXBS>,
                    dim3(static_cast<unsigned>(p.G + gcols)), block, stream, KernelRole::kOnly, p, o);
      return hipGetLastError();
    }
  }
  if (rows_per_block <= RS)
    launch_kernel(sp_region_bwd_rows_kernel<E, VPT, RS, true, DRES, DROP, MAXBS>, grid, block, stream,
                  KernelRole::kFirst, p);
  else
    launch_kernel(sp_region_bwd_rows_kernel<E, VPT, RR, false, DRES, DROP, MAXBS>, grid, block, stream,
                  KernelRole::kFirst, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_cols(p, o, np, stream);
}

template <class E, bool DROP>
hipError_t launch_e(const BwdParams& p, const ColOut& o, int np, const Shape& sh, hipStream_t stream) {
  const bool dres = p.dres != nullptr;
  switch (sh.vpt) {
    case 1: return dres ? launch_rows<E, 1, true, DROP>(p, o, np, sh, stream) : launch_rows<E, 1, false, DROP>(p, o, np, sh, stream);
    case 2: return dres ? launch_rows<E, 2, true, DROP>(p, o, np, sh, stream) : launch_rows<E, 2, false, DROP>(p, o, np, sh, stream);
    case 4: return dres ? launch_rows<E, 4, true, DROP>(p, o, np, sh, stream) : launch_rows<E, 4, false, DROP>(p, o, np, sh, stream);
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
    if (need <= SPR_BWD_MAX_THREADS) {
      // At least kGroups * 2 threads: the reduction's (group, quad) layout.
      const int t = ((need + 63) / 64) * 64;
      return Shape{vpt, t < kGroups * 2 ? kGroups * 2 : t};
    }
  }
  return Shape{0, 0};
}

void set_bwd_launches(int n) { g_max_launches.store(n, std::memory_order_relaxed); }

hipError_t launch_bwd(const BwdParams& params, int dtype, hipStream_t stream) {
  BwdParams p = params;
  p.ws_sstride = ws_slot_stride(p.h);
  p.ws_bstride = ws_block_stride(p.h, p.nparts);
  ColOut o{{p.dgamma, nullptr, nullptr}, 1, p.accumulate};
  if (p.slot_dbeta > 0) o.p[o.np++] = p.dbeta;
  if (p.slot_dbias > 0) o.p[o.np++] = p.dbias;
  const int np = o.np;
  if (p.G == 0) {
    // No rows: every output is 0 (every group of partials is empty); an
    // accumulating call adds nothing and launches nothing.
    if (p.accumulate) return hipSuccess;
    return launch_cols(p, o, np, stream);
  }
  const Shape sh = bwd_shape(p.h, dtype);
  if (sh.vpt == 0) return hipErrorInvalidValue;
  const bool drop = p.dpartial != nullptr;
  if (dtype == 1) return drop ? launch_e<Bf16, true>(p, o, np, sh, stream) : launch_e<Bf16, false>(p, o, np, sh, stream);
  return drop ? launch_e<F32, true>(p, o, np, sh, stream) : launch_e<F32, false>(p, o, np, sh, stream);
}

}  // namespace spr

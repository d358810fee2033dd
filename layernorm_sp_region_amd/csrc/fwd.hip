// Forward of the sequence-parallel region: WPR wavefronts per local token row.
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
// Memory plan.  Lane l of wave w of the row owns the 16-byte vectors
// v = l + 64*(w + WPR*k), k < VPL, so every load instruction of a wave reads
// 1 KB of contiguous row.  The row is streamed in chunks of C vectors per
// lane: the t slab vectors and the residual vector of chunk c+1 are in
// flight while chunk c is summed, masked and stored, and the rounded z stays
// packed in registers (h*2/(64*WPR) bytes per lane in bf16).  Statistics are
// wave butterflies, combined through LDS when WPR > 1 (one row per block, so
// a barrier only couples the row's own waves).  With WPR = 1 waves never
// wait for each other; WPR = 2 halves the registers per wave, doubling the
// waves per SIMD that hide the dropout hash and conversions behind HBM.
// Slabs and residual are streamed with a nontemporal hint; gamma, beta and
// bias (read by every row) use ordinary cached loads.
#include "spr_device.h"
#include "spr_internal.h"

namespace spr {
namespace {

// Tuning knobs (defaults are the measured best on MI355X).
#ifndef SPR_FWD_WAVES_PER_ROW
#define SPR_FWD_WAVES_PER_ROW 1   // waves per row for rows of at least 512 vectors
#endif
#ifndef SPR_FWD_CHUNK
#define SPR_FWD_CHUNK 1           // vectors per lane per streamed chunk
#endif
#ifndef SPR_FWD_NT_STORE
#define SPR_FWD_NT_STORE 0        // nontemporal stores for z and y
#endif
constexpr int kRowsPerBlockW1 = 4;   // WPR = 1: four independent rows per block

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

// Loads of one chunk: C vectors x (NS slabs + residual) per lane.
__device__ __forceinline__ void st16_out(void* p, u32x4 v) {
  if constexpr (SPR_FWD_NT_STORE) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else st16(p, v);
}

template <int NS, int C>
struct Chunk {
  u32x4 s[C][NS];
  u32x4 r[C];
  u32x4 b[C];
};

// gamma/beta of the y phase are fetched kGB slots at a time, one group ahead.
constexpr int kGB = 4;

template <class E, int NS, int VPL, int C, int WPR>
__global__ __launch_bounds__(WPR == 1 ? 64 * kRowsPerBlockW1 : 64 * WPR) void sp_region_fwd_kernel(const FwdParams p) {
  constexpr int V = E::kVec;
  constexpr int EB = 16 / V;
  constexpr int NCH = VPL / C;
  static_assert(VPL % C == 0, "chunk must divide the vectors per lane");
  __shared__ float red[2][WPR];

  const int lane = threadIdx.x & 63;
  const int wv = WPR == 1 ? 0 : threadIdx.x / 64;
  const int64_t row = WPR == 1 ? static_cast<int64_t>(blockIdx.x) * kRowsPerBlockW1 + threadIdx.x / 64
                               : static_cast<int64_t>(blockIdx.x);
  if (row >= p.T) return;   // the whole wave (WPR = 1) or block (WPR > 1) leaves

  const int h = p.h;
  const int nvec = h / V;
  const int64_t row_off = row * static_cast<int64_t>(h) * EB;   // bytes
  const int64_t slab_bytes = p.slab_stride * EB;
  const char* prow = static_cast<const char*>(p.partials) + row_off;
  const char* rrow = static_cast<const char*>(p.residual) + row_off;
  const bool has_res = p.residual != nullptr;

  // Vector owned by slot k, clamped so that loads stay in bounds.
  auto vec_of = [&](int k) {
    const int v = lane + 64 * (wv + WPR * k);
    return v < nvec ? v : nvec - 1;
  };
  auto valid = [&](int k) { return lane + 64 * (wv + WPR * k) < nvec; };

  const bool has_bias = p.bias != nullptr;
  auto issue = [&](Chunk<NS, C>& ch, int c) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int64_t o = static_cast<int64_t>(vec_of(c * C + i)) * 16;
#pragma unroll
      for (int s = 0; s < NS; ++s) ch.s[i][s] = ld16_stream(prow + s * slab_bytes + o);
      if (has_res) ch.r[i] = ld16_stream(rrow + o);
      if (has_bias) ch.b[i] = ld16(static_cast<const char*>(p.bias) + o);
    }
  };

  const uint64_t g = p.drop ? global_token(p, row) : 0;
  const uint32_t g_lo = static_cast<uint32_t>(g), g_hi = static_cast<uint32_t>(g >> 32);

  u32x4 zs[VPL];   // rounded z, packed
  float zsum = 0.0f;   // LayerNorm: sum of the rounded z, accumulated while streaming
  Chunk<NS, C> buf[2];
  issue(buf[0], 0);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c + 1 < NCH) issue(buf[(c + 1) & 1], c + 1);
    Chunk<NS, C>& ch = buf[c & 1];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int k = c * C + i;
      const int v = vec_of(k);
      float acc[V];
      unpack(E{}, ch.s[i][0], acc);
#pragma unroll
      for (int s = 1; s < NS; ++s) {
        float f[V];
        unpack(E{}, ch.s[i][s], f);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = acc[e] + f[e];
      }
      if (has_bias) {
        float f[V];
        unpack(E{}, ch.b[i], f);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = acc[e] + f[e];
      }
      uint8_t keep[V];
#pragma unroll
      for (int e = 0; e < V; ++e) keep[e] = 1;
      if (p.drop) {
#pragma unroll
        for (int b4 = 0; b4 < V / 4; ++b4) {
          const uint32_t blk = static_cast<uint32_t>(v * (V / 4) + b4);   // channel / 4
          const Philox4 r = philox4x32_10(blk, g_lo, g_hi, 0u, p.key0, p.key1);
#pragma unroll
          for (int w = 0; w < 4; ++w) keep[b4 * 4 + w] = r.w[w] >= p.thr;
        }
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = keep[e] ? acc[e] * p.scale : 0.0f;
      }
      if (has_res) {
        float f[V];
        unpack(E{}, ch.r[i], f);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = f[e] + acc[e];
      }
      zs[k] = pack(E{}, acc);
      if (valid(k)) {
        if (p.norm == 0) {
          float f[V];
          rounded_values(E{}, zs[k], f);
#pragma unroll
          for (int e = 0; e < V; ++e) zsum += f[e];
        }
        st16_out(static_cast<char*>(p.z) + row_off + v * 16, zs[k]);
        if (p.mask) {
          uint8_t* m = p.mask + row * static_cast<int64_t>(h) + v * V;
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
  }

  // gamma/beta of the first kGB slots: in flight during the statistics.
  u32x4 gb[2][kGB][2];
  auto issue_gb = [&](int grp) {
#pragma unroll
    for (int j = 0; j < kGB; ++j) {
      const int k = grp * kGB + j;
      if (k < VPL) {
        const int64_t o = static_cast<int64_t>(vec_of(k)) * 16;
        gb[grp & 1][j][0] = ld16(static_cast<const char*>(p.gamma) + o);
        if (p.beta) gb[grp & 1][j][1] = ld16(static_cast<const char*>(p.beta) + o);
      }
    }
  };
  issue_gb(0);

  // ---- statistics over the full h (from the rounded z) --------------------
  const float inv_h = 1.0f / static_cast<float>(h);
  float mean = 0.0f, q = 0.0f;
  if (p.norm == 0) {
    mean = row_total<WPR>(zsum, red[0]) * inv_h;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if (valid(k)) {
        float f[V];
        rounded_values(E{}, zs[k], f);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float d = f[e] - mean;
          q = __builtin_fmaf(d, d, q);
        }
      }
  } else {
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if (valid(k)) {
        float f[V];
        rounded_values(E{}, zs[k], f);
#pragma unroll
        for (int e = 0; e < V; ++e) q = __builtin_fmaf(f[e], f[e], q);
      }
  }
  const float rstd = 1.0f / __builtin_sqrtf(row_total<WPR>(q, red[1]) * inv_h + p.eps);
  if (threadIdx.x % (64 * WPR) == 0) {
    if (p.mean) p.mean[row] = mean;
    p.rstd[row] = rstd;
  }

  // ---- y -------------------------------------------------------------------
  constexpr int NG = (VPL + kGB - 1) / kGB;
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    if (grp + 1 < NG) issue_gb(grp + 1);
#pragma unroll
    for (int j = 0; j < kGB; ++j) {
      const int k = grp * kGB + j;
      if (k >= VPL || !valid(k)) continue;
      float zf[V], gm[V], bt[V], yv[V];
      rounded_values(E{}, zs[k], zf);
      unpack(E{}, gb[grp & 1][j][0], gm);
      if (p.beta) unpack(E{}, gb[grp & 1][j][1], bt);
      else {
#pragma unroll
        for (int e = 0; e < V; ++e) bt[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < V; ++e) yv[e] = __builtin_fmaf((zf[e] - mean) * rstd, gm[e], bt[e]);
      st16_out(static_cast<char*>(p.y) + row_off + vec_of(k) * 16, pack(E{}, yv));
    }
  }
}

template <class E, int VPL, int WPR>
hipError_t launch_ns(const FwdParams& p, hipStream_t stream) {
  constexpr int C = VPL % SPR_FWD_CHUNK == 0 ? SPR_FWD_CHUNK : 1;
  const dim3 grid(static_cast<unsigned>(WPR == 1 ? (p.T + kRowsPerBlockW1 - 1) / kRowsPerBlockW1 : p.T));
  const dim3 block(WPR == 1 ? 64 * kRowsPerBlockW1 : 64 * WPR);
  switch (p.t) {
#define SPR_NS(N) \
  case N: hipLaunchKernelGGL((sp_region_fwd_kernel<E, N, VPL, C, WPR>), grid, block, 0, stream, p); break;
    SPR_NS(1) SPR_NS(2) SPR_NS(3) SPR_NS(4) SPR_NS(5) SPR_NS(6) SPR_NS(7) SPR_NS(8)
#undef SPR_NS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class E>
hipError_t launch_e(const FwdParams& p, const Shape& sh, hipStream_t stream) {
  constexpr int W2 = SPR_FWD_WAVES_PER_ROW;
  if (sh.threads == 64) {
    switch (sh.vpt) {
      case 1: return launch_ns<E, 1, 1>(p, stream);
      case 2: return launch_ns<E, 2, 1>(p, stream);
      case 4: return launch_ns<E, 4, 1>(p, stream);
      case 8: return launch_ns<E, 8, 1>(p, stream);
      default:
        if constexpr (W2 == 1) {
          if (sh.vpt == 16) return launch_ns<E, 16, 1>(p, stream);
          if (sh.vpt == 32) return launch_ns<E, 32, 1>(p, stream);
        }
        return hipErrorInvalidValue;
    }
  }
  if constexpr (W2 > 1) {
    switch (sh.vpt) {
      case 4: return launch_ns<E, 4, W2>(p, stream);
      case 8: return launch_ns<E, 8, W2>(p, stream);
      case 16: return launch_ns<E, 16, W2>(p, stream);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Waves per row and vectors per lane.  Rows of fewer than 512 vectors get one
// wave (threads = 64) and the smallest power-of-two VPL covering them; longer
// rows get SPR_FWD_WAVES_PER_ROW waves (threads = 64*WPR).
// (h = 8192 bf16 -> 2 waves x 8; h = 5120 -> 2 x 8 with 3 slots predicated off;
//  h = 512 f32 -> 1 x 2.)
Shape fwd_shape(int h, int dtype) {
  const int vec = dtype == 1 ? 8 : 4;
  const int nvec = h / vec;
  constexpr int W2 = SPR_FWD_WAVES_PER_ROW;
  if (nvec < 512 || W2 == 1) {
    for (int vpl : {1, 2, 4, 8, 16, 32})
      if (nvec <= 64 * vpl) return Shape{vpl, 64};
    return Shape{0, 0};
  }
  for (int vpl : {4, 8, 16})
    if (nvec <= 64 * W2 * vpl) return Shape{vpl, 64 * W2};
  return Shape{0, 0};
}

hipError_t launch_fwd(const FwdParams& p, int dtype, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const Shape sh = fwd_shape(p.h, dtype);
  return dtype == 1 ? launch_e<Bf16>(p, sh, stream) : launch_e<F32>(p, sh, stream);
}

}  // namespace spr

// Device helpers of the SP-region kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spr {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Storage element traits.  Every global access is a 16-byte vector: 8 bf16 or
// 4 float32 channels.
// ---------------------------------------------------------------------------
struct Bf16 {
  static constexpr int kVec = 8;
};
struct F32 {
  static constexpr int kVec = 4;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte access
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Streamed-once data: nontemporal hint keeps it from displacing reused lines.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Output no kernel of this library reads back: nontemporal, so its lines
// stream to memory instead of filling the caches with dirty data.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// 16 bytes -> float32 channels (bf16 widening is exact: the 16 bits become
// the high half of the float32 pattern).
__device__ __forceinline__ void unpack(Bf16, u32x4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f[2 * m] = __uint_as_float(w[m] << 16);
    f[2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack(F32, u32x4 v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

// float32 channels -> 16 bytes; bf16 uses the hardware round-to-nearest-even
// conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ u32x4 pack(Bf16, const float* f) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
               pack_bf16x2(f[6], f[7])};
}
__device__ __forceinline__ u32x4 pack(F32, const float* f) {
  return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
               __float_as_uint(f[3])};
}

// Value of a packed-and-rounded channel as float32 (what a reader of z sees).
__device__ __forceinline__ void rounded_values(Bf16, u32x4 v, float* f) { unpack(Bf16{}, v, f); }
__device__ __forceinline__ void rounded_values(F32, u32x4 v, float* f) { unpack(F32{}, v, f); }

// ---------------------------------------------------------------------------
// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11, section 4): per round the
// counter words 0 and 2 are multiplied by two odd constants, both halves of
// each 64-bit product are kept, and the words are permuted with the key
// xor-ed in; the key advances by the golden-ratio and sqrt(3) Weyl constants
// between rounds.  The 32x32->64 products map to v_mad_u64_u32.
// ---------------------------------------------------------------------------
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// Keep decisions of the V channels of 16-byte vector v of the row with global
// token index g: channel j is kept iff word (j mod 4) of Philox-4x32-10 with
// counter (j div 4, lo32 g, hi32 g, 0) and key (k0, k1) is >= thr.
template <int V>
__device__ __forceinline__ void dropout_keep(uint32_t v, uint32_t g_lo, uint32_t g_hi, uint32_t k0, uint32_t k1,
                                             uint32_t thr, bool* keep) {
#pragma unroll
  for (int b4 = 0; b4 < V / 4; ++b4) {
    const Philox4 r = philox4x32_10(v * (V / 4) + b4, g_lo, g_hi, 0u, k0, k1);
#pragma unroll
    for (int w = 0; w < 4; ++w) keep[b4 * 4 + w] = r.w[w] >= thr;
  }
}

// Global token index of local row `row` (its row in the unsharded [s*b][h]
// view): rank*T + row for a uniform shard; for a packed ragged batch with
// local offsets cu[0..nseq], row i of sequence q is token
// t*cu[q] + rank*(cu[q+1]-cu[q]) + (i-cu[q]).  The offsets are read through
// the constant address space, so the lookups are scalar loads: they are
// counted apart from the vector-memory stream and never make a wait on them
// drain the prefetched rows.
__device__ __forceinline__ uint64_t global_token_of(int64_t row, int64_t T, int t, int rank, const int32_t* cu,
                                                    int nseq) {
  if (cu == nullptr) return static_cast<uint64_t>(rank) * static_cast<uint64_t>(T) + row;
  typedef const __attribute__((address_space(4))) int32_t* const_i32p;
  const const_i32p c = (const_i32p)(cu);   // address-space cast (generic -> constant)
  // Largest q in [0, nseq) with cu[q] <= row (empty sequences are skipped).
  int lo = 0, hi = nseq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (c[mid] <= row) lo = mid; else hi = mid;
  }
  const int64_t start = c[lo];
  const int64_t len = static_cast<int64_t>(c[lo + 1]) - start;
  return static_cast<uint64_t>(t * start + rank * len + (row - start));
}

// ---------------------------------------------------------------------------
// Reductions.  Wave sums use DPP row steps plus readlane (below), and the
// cross-wave stage sums the per-wave totals in wave order, so a block's
// result is deterministic and uniform across its threads.
// ---------------------------------------------------------------------------
// DPP row operations of GFX9 (operand permutations inside each row of 16
// lanes, applied by the VALU itself: no LDS round trip).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over each row of 16 lanes: after the two quad steps every lane holds
// its quad's sum, after the half mirror its 8-lane group's, after the mirror
// its row's.  Each step adds the same two values in both partner lanes, so
// all lanes of a row hold bit-identical totals.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}

// Wave total, uniform (scalar) and deterministic: the four row sums are
// combined in row order.
__device__ __forceinline__ float wave_total(float x) {
  x = row16_sum(x);
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return ((r0 + r1) + r2) + r3;
}

template <int N>
__device__ __forceinline__ void wave_sum(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_total(v[i]);
}

// Block-wide sum of N values per thread (blocks of at most 16 waves).  `slot`
// is LDS of N * 16 floats; callers alternate two slots between consecutive
// reductions so that one barrier per reduction suffices: a slot is rewritten
// only after every wave has passed the barrier of the reduction in between.
template <int N>
__device__ __forceinline__ void block_sum(float (&v)[N], float* slot) {
  wave_sum<N>(v);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = (blockDim.x + kWave - 1) / kWave;
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) slot[i * 16 + wave] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float s = slot[i * 16];
    for (int w = 1; w < nwaves; ++w) s += slot[i * 16 + w];
    v[i] = s;
  }
}

}  // namespace spr

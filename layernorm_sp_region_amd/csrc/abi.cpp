// C ABI of the SP-region library: argument validation, then dispatch to the
// kernel launchers.  Every check runs before any HIP call, so an invalid call
// launches nothing and leaves the outputs untouched.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "sp_region.h"
#include "spr_internal.h"

namespace spr {
thread_local LaunchEvents g_launch_events = {nullptr, nullptr};
}  // namespace spr

namespace {

thread_local int g_last_hip_error = 0;

// The hook applies to one region call; cleared on every exit path.
struct ClearLaunchEvents {
  ~ClearLaunchEvents() { spr::g_launch_events = {nullptr, nullptr}; }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned16_or_null(const void* p) { return p == nullptr || aligned16(p); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SPR_OK;
  g_last_hip_error = static_cast<int>(e);
  return SPR_ERR_HIP;
}

// Shared shape checks of fwd and bwd; on success sets T.
int check_shape(int64_t b, int64_t s, int64_t h, int32_t t, int32_t norm, int32_t dtype, int64_t* T) {
  if (t < 1 || b < 1 || s < 0 || h <= 0) return SPR_ERR_INVALID_ARG;
  if (dtype != SPR_F32 && dtype != SPR_BF16) return SPR_ERR_INVALID_ARG;
  if (norm != SPR_LAYERNORM && norm != SPR_RMSNORM) return SPR_ERR_INVALID_ARG;
  if (s % t != 0) return SPR_ERR_INVALID_ARG;
  if (t > SPR_MAX_T_SLABS) return SPR_ERR_UNSUPPORTED;
  const int64_t vec = dtype == SPR_BF16 ? 8 : 4;
  const int64_t hmax = dtype == SPR_BF16 ? SPR_MAX_H_BF16 : SPR_MAX_H_F32;
  if (h % vec != 0 || h > hmax) return SPR_ERR_UNSUPPORTED;
  const int64_t per_rank = s / t;
  if (per_rank > 0 && b > INT64_MAX / per_rank) return SPR_ERR_INVALID_ARG;
  *T = b * per_rank;
  if (*T > INT32_MAX) return SPR_ERR_UNSUPPORTED;   // grid.x limit of one row per block
  return SPR_OK;
}

}  // namespace

extern "C" {

int sp_region_abi_version(void) { return SP_REGION_ABI_VERSION; }

const char* sp_region_strerror(int status) {
  switch (status) {
    case SPR_OK: return "ok";
    case SPR_ERR_INVALID_ARG: return "invalid argument";
    case SPR_ERR_UNSUPPORTED: return "unsupported shape (t, h or dtype outside the compiled kernels)";
    case SPR_ERR_ALIGNMENT: return "pointer or slab stride not 16-byte aligned";
    case SPR_ERR_HIP: return "HIP launch error (see sp_region_last_hip_error)";
    case SPR_ERR_SCRATCH:
      return "shard needs more workspace than sp_region_bwd_noalloc's static scratch (SPR_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int sp_region_last_hip_error(void) { return g_last_hip_error; }

int sp_region_time_next_call(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return SPR_ERR_INVALID_ARG;
  spr::g_launch_events = {static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  return SPR_OK;
}

}  // extern "C"

namespace {

// The forward's checks and parameters, shared by the strided and the
// pointer-table entry points; slabs[k] is slab k's device pointer.
int run_fwd(int64_t b, int64_t s, int64_t h, int32_t t, float eps, float p_drop, const void* gamma,
            const void* beta, int32_t norm, int32_t dtype, int32_t rank, uint64_t seed, const void* const* slabs,
            const void* bias, const void* residual, const int32_t* cu_seqlens, int32_t nseq, void* z, void* y,
            float* mean, float* rstd, uint8_t* mask_out, void* stream) {
  for (int32_t k = 0; k < t && k < SPR_MAX_T_SLABS; ++k) {
    if (slabs[k] == nullptr) return SPR_ERR_INVALID_ARG;
    if (!aligned16(slabs[k])) return SPR_ERR_ALIGNMENT;
  }
  const bool ln = norm == SPR_LAYERNORM;
  if (!gamma || !z || !y || !rstd) return SPR_ERR_INVALID_ARG;
  if (ln != (mean != nullptr)) return SPR_ERR_INVALID_ARG;
  if (!ln && beta != nullptr) return SPR_ERR_INVALID_ARG;
  for (const void* ptr : {gamma, static_cast<const void*>(z), static_cast<const void*>(y),
                          static_cast<const void*>(rstd)})
    if (!aligned16(ptr)) return SPR_ERR_ALIGNMENT;
  for (const void* ptr : {beta, bias, residual, static_cast<const void*>(mean), static_cast<const void*>(mask_out)})
    if (!aligned16_or_null(ptr)) return SPR_ERR_ALIGNMENT;
  if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return SPR_ERR_ALIGNMENT;

  spr::FwdParams p{};
  for (int32_t k = 0; k < t; ++k) p.slab[k] = slabs[k];
  p.bias = bias;
  p.residual = residual;
  p.gamma = gamma;
  p.beta = beta;
  p.cu = cu_seqlens;
  p.nseq = nseq;
  p.z = z;
  p.y = y;
  p.mean = mean;
  p.rstd = rstd;
  p.mask = mask_out;
  p.T = b * (s / t);
  p.h = static_cast<int32_t>(h);
  p.t = t;
  p.rank = rank;
  p.norm = norm;
  p.eps = eps;
  const double pd = static_cast<double>(p_drop);
  p.drop = p_drop > 0.0f ? 1 : 0;
  p.scale = static_cast<float>(1.0 / (1.0 - pd));
  p.thr = static_cast<uint32_t>(std::floor(pd * 4294967296.0));
  p.key0 = static_cast<uint32_t>(seed);
  p.key1 = static_cast<uint32_t>(seed >> 32);
  return hip_status(spr::launch_fwd(p, dtype, static_cast<hipStream_t>(stream)));
}

// Scalar checks common to both forward entry points; sets T.
int check_fwd_scalars(int64_t b, int64_t s, int64_t h, int32_t t, float eps, float p_drop, int32_t norm,
                      int32_t dtype, int32_t rank, const int32_t* cu_seqlens, int32_t nseq, int64_t* T) {
  const int st = check_shape(b, s, h, t, norm, dtype, T);
  if (st != SPR_OK) return st;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return SPR_ERR_INVALID_ARG;
  if (!(p_drop >= 0.0f && p_drop < 1.0f)) return SPR_ERR_INVALID_ARG;
  if (rank < 0 || rank >= t) return SPR_ERR_INVALID_ARG;
  if (cu_seqlens != nullptr && (nseq < 1 || b != 1)) return SPR_ERR_INVALID_ARG;
  if (nseq < 0) return SPR_ERR_INVALID_ARG;
  return SPR_OK;
}

}  // namespace

extern "C" {

int sp_region_fwd(int64_t b, int64_t s, int64_t h, int32_t t, float eps, float p_drop,
                  const void* gamma, const void* beta,
                  int32_t norm, int32_t dtype, int32_t rank, uint64_t seed,
                  const void* partials, int64_t slab_stride,
                  const void* bias, const void* residual,
                  const int32_t* cu_seqlens, int32_t nseq,
                  void* z, void* y, float* mean, float* rstd,
                  uint8_t* mask_out,
                  void* stream) {
  ClearLaunchEvents clear_hook;
  int64_t T = 0;
  const int st = check_fwd_scalars(b, s, h, t, eps, p_drop, norm, dtype, rank, cu_seqlens, nseq, &T);
  if (st != SPR_OK) return st;
  if (T == 0) return SPR_OK;
  if (!partials) return SPR_ERR_INVALID_ARG;
  if (slab_stride < T * h) return SPR_ERR_INVALID_ARG;
  const int64_t eb = dtype == SPR_BF16 ? 2 : 4;
  if ((slab_stride * eb) % 16 != 0) return SPR_ERR_ALIGNMENT;
  const void* slabs[SPR_MAX_T_SLABS];
  for (int32_t k = 0; k < t; ++k) slabs[k] = static_cast<const char*>(partials) + k * slab_stride * eb;
  return run_fwd(b, s, h, t, eps, p_drop, gamma, beta, norm, dtype, rank, seed, slabs, bias, residual, cu_seqlens,
                 nseq, z, y, mean, rstd, mask_out, stream);
}

int sp_region_fwd_slabs(int64_t b, int64_t s, int64_t h, int32_t t, float eps, float p_drop,
                        const void* gamma, const void* beta,
                        int32_t norm, int32_t dtype, int32_t rank, uint64_t seed,
                        const void* const* slabs,
                        const void* bias, const void* residual,
                        const int32_t* cu_seqlens, int32_t nseq,
                        void* z, void* y, float* mean, float* rstd,
                        uint8_t* mask_out,
                        void* stream) {
  ClearLaunchEvents clear_hook;
  int64_t T = 0;
  const int st = check_fwd_scalars(b, s, h, t, eps, p_drop, norm, dtype, rank, cu_seqlens, nseq, &T);
  if (st != SPR_OK) return st;
  if (T == 0) return SPR_OK;
  if (slabs == nullptr) return SPR_ERR_INVALID_ARG;
  return run_fwd(b, s, h, t, eps, p_drop, gamma, beta, norm, dtype, rank, seed, slabs, bias, residual, cu_seqlens,
                 nseq, z, y, mean, rstd, mask_out, stream);
}

int64_t sp_region_partials_stride(int64_t n_local_tokens, int64_t h, int32_t dtype) {
  if (n_local_tokens <= 0 || h <= 0 || (dtype != SPR_F32 && dtype != SPR_BF16)) return 0;
  const int64_t eb = dtype == SPR_BF16 ? 2 : 4;
  const int64_t bytes = n_local_tokens * h * eb;
  return ((bytes + 2047) / 2048 * 2048 + 1024) / eb;
}

size_t sp_region_bwd_workspace_bytes(int64_t n_local_tokens, int64_t h) {
  if (n_local_tokens <= 0 || h <= 0) return 0;
  return static_cast<size_t>(spr::ws_total_bytes(spr::bwd_blocks(n_local_tokens, h), h, 2));
}

size_t sp_region_bwd_dropout_workspace_bytes(int64_t n_local_tokens, int64_t h) {
  if (n_local_tokens <= 0 || h <= 0) return 0;
  return static_cast<size_t>(spr::ws_total_bytes(spr::bwd_blocks(n_local_tokens, h), h, 3));
}

}  // extern "C"

namespace {

// Checks shared by both backward entry points; fills the normalisation part
// of the parameters.
int prepare_bwd(int64_t b, int64_t s, int64_t h, int32_t t, const void* gamma, int32_t norm, int32_t dtype,
                const void* dy, const void* z, const float* mean, const float* rstd, const void* dres_in, void* dx,
                float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes, bool with_dropout,
                spr::BwdParams* p) {
  int64_t T = 0;
  const int st = check_shape(b, s, h, t, norm, dtype, &T);
  if (st != SPR_OK) return st;
  const size_t need = with_dropout ? sp_region_bwd_dropout_workspace_bytes(T, h) : sp_region_bwd_workspace_bytes(T, h);
  const bool ln = norm == SPR_LAYERNORM;
  if (!gamma || !dgamma) return SPR_ERR_INVALID_ARG;
  if (!ln && dbeta != nullptr) return SPR_ERR_INVALID_ARG;
  if (workspace_bytes < need || (need > 0 && workspace == nullptr)) return SPR_ERR_INVALID_ARG;
  if (T > 0) {
    if (!dy || !z || !rstd || !dx) return SPR_ERR_INVALID_ARG;
    if (ln != (mean != nullptr)) return SPR_ERR_INVALID_ARG;
  }
  for (const void* ptr : {gamma, dy, z, static_cast<const void*>(mean), static_cast<const void*>(rstd), dres_in,
                          static_cast<const void*>(dx), static_cast<const void*>(dgamma),
                          static_cast<const void*>(dbeta), static_cast<const void*>(workspace)})
    if (!aligned16_or_null(ptr)) return SPR_ERR_ALIGNMENT;
  *p = spr::BwdParams{};
  p->dy = dy;
  p->z = z;
  p->mean = mean;
  p->rstd = rstd;
  p->gamma = gamma;
  p->dres = dres_in;
  p->dx = dx;
  p->ws = static_cast<float*>(workspace);
  p->dgamma = dgamma;
  p->dbeta = dbeta;
  p->T = T;
  p->h = static_cast<int32_t>(h);
  p->norm = norm;
  p->G = static_cast<int32_t>(spr::bwd_blocks(T, h));
  p->nparts = 1;
  if (dbeta) p->slot_dbeta = p->nparts++;
  return SPR_OK;
}

// The forward's dropout arguments as the backward takes them (same checks).
int check_dropout_args(int64_t b, int32_t t, float p_drop, int32_t rank, const int32_t* cu_seqlens, int32_t nseq) {
  if (!(p_drop >= 0.0f && p_drop < 1.0f)) return SPR_ERR_INVALID_ARG;
  if (rank < 0 || rank >= t) return SPR_ERR_INVALID_ARG;
  if (cu_seqlens != nullptr && (nseq < 1 || b != 1)) return SPR_ERR_INVALID_ARG;
  if (nseq < 0) return SPR_ERR_INVALID_ARG;
  if (cu_seqlens != nullptr && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return SPR_ERR_ALIGNMENT;
  return SPR_OK;
}

// Gradient through the dropout and the slab sum: dpartial (rows kernel) and
// the dbias partials, with the mask parameters the forward used.
void set_dropout(spr::BwdParams* p, int32_t t, float p_drop, int32_t rank, uint64_t seed,
                 const int32_t* cu_seqlens, int32_t nseq, void* dpartial, float* dbias) {
  if (p->T > 0) p->dpartial = dpartial;
  p->dbias = dbias;
  if (dbias) p->slot_dbias = p->nparts++;
  p->cu = cu_seqlens;
  p->nseq = nseq;
  p->t = t;
  p->rank = rank;
  const double pd = static_cast<double>(p_drop);
  p->drop = p_drop > 0.0f ? 1 : 0;
  p->scale = static_cast<float>(1.0 / (1.0 - pd));
  p->thr = static_cast<uint32_t>(std::floor(pd * 4294967296.0));
  p->key0 = static_cast<uint32_t>(seed);
  p->key1 = static_cast<uint32_t>(seed >> 32);
}

}  // namespace

extern "C" {

int sp_region_bwd(int64_t b, int64_t s, int64_t h, int32_t t,
                  const void* gamma, int32_t norm, int32_t dtype,
                  const void* dy, const void* z, const float* mean, const float* rstd,
                  const void* dres_in,
                  void* dx, float* dgamma, float* dbeta,
                  void* workspace, size_t workspace_bytes,
                  void* stream) {
  ClearLaunchEvents clear_hook;
  spr::BwdParams p;
  const int st = prepare_bwd(b, s, h, t, gamma, norm, dtype, dy, z, mean, rstd, dres_in, dx, dgamma, dbeta,
                             workspace, workspace_bytes, false, &p);
  if (st != SPR_OK) return st;
  return hip_status(spr::launch_bwd(p, dtype, static_cast<hipStream_t>(stream)));
}

int sp_region_bwd_dropout(int64_t b, int64_t s, int64_t h, int32_t t,
                          const void* gamma, int32_t norm, int32_t dtype,
                          const void* dy, const void* z, const float* mean, const float* rstd,
                          const void* dres_in,
                          float p_drop, int32_t rank, uint64_t seed,
                          const int32_t* cu_seqlens, int32_t nseq,
                          void* dx, void* dpartial, float* dgamma, float* dbeta, float* dbias,
                          void* workspace, size_t workspace_bytes,
                          void* stream) {
  ClearLaunchEvents clear_hook;
  spr::BwdParams p;
  int st = prepare_bwd(b, s, h, t, gamma, norm, dtype, dy, z, mean, rstd, dres_in, dx, dgamma, dbeta,
                       workspace, workspace_bytes, true, &p);
  if (st != SPR_OK) return st;
  st = check_dropout_args(b, t, p_drop, rank, cu_seqlens, nseq);
  if (st != SPR_OK) return st;
  if (p.T > 0 && dpartial == nullptr) return SPR_ERR_INVALID_ARG;
  if (!aligned16_or_null(dpartial) || !aligned16_or_null(dbias)) return SPR_ERR_ALIGNMENT;
  set_dropout(&p, t, p_drop, rank, seed, cu_seqlens, nseq, dpartial, dbias);
  return hip_status(spr::launch_bwd(p, dtype, static_cast<hipStream_t>(stream)));
}

int sp_region_bwd_accumulate(int64_t b, int64_t s, int64_t h, int32_t t,
                             const void* gamma, int32_t norm, int32_t dtype,
                             const void* dy, const void* z, const float* mean, const float* rstd,
                             const void* dres_in,
                             float p_drop, int32_t rank, uint64_t seed,
                             const int32_t* cu_seqlens, int32_t nseq,
                             void* dx, void* dpartial, float* dgamma, float* dbeta, float* dbias,
                             void* workspace, size_t workspace_bytes,
                             void* stream) {
  ClearLaunchEvents clear_hook;
  const bool with_dropout = dpartial != nullptr;
  spr::BwdParams p;
  int st = prepare_bwd(b, s, h, t, gamma, norm, dtype, dy, z, mean, rstd, dres_in, dx, dgamma, dbeta,
                       workspace, workspace_bytes, with_dropout, &p);
  if (st != SPR_OK) return st;
  st = check_dropout_args(b, t, p_drop, rank, cu_seqlens, nseq);
  if (st != SPR_OK) return st;
  if (p.T > 0 && !with_dropout && dbias != nullptr) return SPR_ERR_INVALID_ARG;   // dbias needs dpartial
  if (!aligned16_or_null(dpartial) || !aligned16_or_null(dbias)) return SPR_ERR_ALIGNMENT;
  if (with_dropout) set_dropout(&p, t, p_drop, rank, seed, cu_seqlens, nseq, dpartial, dbias);
  p.accumulate = 1;
  return hip_status(spr::launch_bwd(p, dtype, static_cast<hipStream_t>(stream)));
}

int sp_region_set_bwd_launches(int32_t launches) {
  if (launches != 1 && launches != 2) return SPR_ERR_INVALID_ARG;
  spr::set_bwd_launches(launches);
  return SPR_OK;
}

int sp_region_hbm_copy(const void* src, void* dst, size_t nbytes, void* stream) {
  if (nbytes % 16 != 0) return SPR_ERR_INVALID_ARG;
  if (nbytes == 0) return SPR_OK;
  if (!src || !dst) return SPR_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(dst)) return SPR_ERR_ALIGNMENT;
  return hip_status(spr::launch_copy(src, dst, nbytes, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free backward.  Its workspace is this file-scope device array,
// one copy per GPU.  In host code `scratch` names a host-side stand-in, not
// the GPU's copy, so it is never passed to a kernel or a copy: the GPU's
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept in g_scratch.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SPR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Address of `scratch` on the GPU that runs `stream` (the current device for
// the null stream).
int scratch_for_stream(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e);
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_status(e);
  }
  if (dev < 0 || dev >= kMaxDevices) return SPR_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t e2 = dev != cur ? hipSetDevice(cur) : hipSuccess;
      if (e != hipSuccess) return hip_status(e);
      if (e2 != hipSuccess) return hip_status(e2);
      if (p == nullptr) return SPR_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SPR_OK;
}

}  // namespace

extern "C" int sp_region_bwd_noalloc(int64_t b, int64_t s, int64_t h, int32_t t,
                                     const void* gamma, int32_t norm, int32_t dtype,
                                     const void* dy, const void* z, const float* mean, const float* rstd,
                                     const void* dres_in,
                                     void* dx, float* dgamma, float* dbeta,
                                     void* stream) {
  ClearLaunchEvents clear_hook;
  int64_t T = 0;
  int st = check_shape(b, s, h, t, norm, dtype, &T);
  if (st != SPR_OK) return st;
  if (sp_region_bwd_workspace_bytes(T, h) > SPR_NOALLOC_SCRATCH_BYTES) return SPR_ERR_SCRATCH;
  // Every argument check first, against an aligned stand-in for the scratch
  // address; the real address replaces it once the call is known valid.
  spr::BwdParams p;
  st = prepare_bwd(b, s, h, t, gamma, norm, dtype, dy, z, mean, rstd, dres_in, dx, dgamma, dbeta,
                   reinterpret_cast<void*>(uintptr_t{256}), SPR_NOALLOC_SCRATCH_BYTES, false, &p);
  if (st != SPR_OK) return st;
  void* ws = nullptr;
  st = scratch_for_stream(static_cast<hipStream_t>(stream), &ws);
  if (st != SPR_OK) return st;
  p.ws = static_cast<float*>(ws);
  return hip_status(spr::launch_bwd(p, dtype, static_cast<hipStream_t>(stream)));
}

/*
 * sp_region.h -- C ABI of the fused sequence-parallel region for MI355X (gfx950).
 *
 * The region is the non-tensor-parallel part of a Megatron TP+SP transformer
 * block, on one rank's sequence shard [s/t][b][h]:
 *
 *   forward   z = residual + dropout(sum_{k<t} P_k + bias)
 *             y = LayerNorm(z) or RMSNorm(z), per token over the full h
 *   backward  dx = dL/dz (+ dres_in), dgamma, dbeta
 *
 * P_k is this rank's [T][h] slice of TP rank k's row-parallel-linear partial
 * output, so the sum is the arithmetic of the g* reduce-scatter done locally
 * (hpc.payai.win lesson 7 "Sequence parallelism", section 3.A: g* sums the
 * row-linear partial outputs and leaves each rank its s/t slice).  LayerNorm
 * is the formula of section 2 of that lesson (mean and population variance
 * over h, eps inside the square root, then gamma and beta).  Dropout masks
 * are a pure function of (seed, global token, channel), so every rank draws
 * the same mask for the same token, as the lesson's answer to question 1
 * requires; the (b, s, h, t, eps, p, gamma, beta) argument set follows the
 * lesson's statement of the problem.
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless stated; `stream` is a hipStream_t
 *     passed as void* (NULL = the default stream).
 *   - T = b * s / t local rows; every [T][h] tensor is row-major, contiguous,
 *     row i at element offset i*h.  A packed ragged batch is passed as b = 1
 *     and s = total packed length, with cu_seqlens giving local row offsets.
 *   - dtype SPR_BF16: activations, gamma, beta and bias are bfloat16;
 *     SPR_F32: all float32.  mean, rstd, dgamma, dbeta are always float32.
 *   - The caller owns every buffer (the backward workspace included).  The
 *     library allocates nothing, keeps no mutable global state (except the
 *     static device scratch of sp_region_bwd_noalloc), launches
 *     asynchronously on `stream`, never synchronises and never reads device
 *     memory on the host.  Outputs are overwritten, not accumulated.
 *   - Errors: a nonzero status is returned BEFORE any launch and leaves every
 *     output untouched.  Argument checks: see each function.  A failed launch
 *     returns SPR_ERR_HIP; sp_region_last_hip_error() then gives the raw
 *     hipError_t of this thread.  Nothing prints, aborts or throws.
 *   - Every device pointer must be 16-byte aligned.
 */
#ifndef SP_REGION_H_
#define SP_REGION_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SP_REGION_ABI_VERSION 4   /* 2 sp_region_bwd_accumulate; 3 sp_region_bwd_noalloc; 4 sp_region_set_bwd_launches */

enum sp_region_status {
  SPR_OK = 0,
  SPR_ERR_INVALID_ARG = 1,  /* argument outside its documented domain */
  SPR_ERR_UNSUPPORTED = 2,  /* valid, but not compiled for (h, t, dtype) */
  SPR_ERR_ALIGNMENT = 3,    /* pointer or slab stride not 16-byte aligned */
  SPR_ERR_HIP = 4,          /* kernel launch failed (see sp_region_last_hip_error) */
  SPR_ERR_SCRATCH = 5       /* sp_region_bwd_noalloc: the shard needs more than its static scratch */
};

enum sp_region_dtype { SPR_F32 = 0, SPR_BF16 = 1 };
enum sp_region_norm { SPR_LAYERNORM = 0, SPR_RMSNORM = 1 };

/* Limits of the compiled kernels. */
#define SPR_MAX_T_SLABS 8      /* tensor-parallel degree t: 1..8 */
#define SPR_MAX_H_BF16 16384   /* h % 8 == 0 */
#define SPR_MAX_H_F32 8192     /* h % 4 == 0 */

/* Returns SP_REGION_ABI_VERSION of the built library. */
int sp_region_abi_version(void);

/* Static string naming a status code (never NULL). */
const char* sp_region_strerror(int status);

/* hipError_t of this thread's last SPR_ERR_HIP (0 if none). */
int sp_region_last_hip_error(void);

/*
 * Profiling hook.  The next sp_region_fwd, sp_region_bwd or
 * sp_region_bwd_dropout call on this thread records start_event when its
 * first kernel starts and stop_event when its last kernel ends: timestamps
 * carried by the kernels' own dispatch packets (hipExtLaunchKernel), so no
 * extra packets are placed on the stream.  The events are hipEvent_t passed
 * as void*, created by the caller with timing enabled.  The hook applies to
 * exactly one call (whatever its status) and is then cleared; both NULL clears
 * it.  Returns SPR_ERR_INVALID_ARG if exactly one of them is NULL.
 */
int sp_region_time_next_call(void* start_event, void* stop_event);

/*
 * Recommended slab_stride, in elements, for the forward's t partial slabs of
 * T = n_local_tokens rows of h channels of `dtype`: the smallest stride
 * >= T*h whose size in bytes is 1 KiB more than a multiple of 2 KiB.  The
 * forward reads row i of every slab at the same time; slabs whose starts are
 * congruent modulo 2 KiB (contiguous slabs of 32 MiB, say) send those reads to
 * the same HBM channels, which measured about 5% slower on MI355X.  Any
 * stride the forward accepts gives identical results.  A pure function;
 * returns 0 for T <= 0, h <= 0 or an unknown dtype.
 */
int64_t sp_region_partials_stride(int64_t n_local_tokens, int64_t h, int32_t dtype);

/*
 * Forward of the region on one rank's shard.
 *
 *   b, s, t      micro-batch, global sequence length, TP degree (1..8);
 *                s % t == 0; T = b*s/t.  Ragged: b must be 1.
 *   h            hidden size; bf16: h % 8 == 0, h <= SPR_MAX_H_BF16;
 *                f32: h % 4 == 0, h <= SPR_MAX_H_F32.
 *   eps          > 0 and finite; added to the variance (LayerNorm) or to the
 *                mean square (RMSNorm) inside the square root.
 *   p_drop       dropout probability in [0, 1).  Element (i, j) is kept iff
 *                word (j mod 4) of Philox-4x32-10(counter = (j div 4,
 *                lo32 g_i, hi32 g_i, 0), key = (lo32 seed, hi32 seed)) is
 *                >= floor(p_drop * 2^32); kept values are scaled by the
 *                float32 value of 1/(1 - p_drop).  p_drop == 0 skips the hash.
 *                (Philox: Salmon et al., "Parallel random numbers: as easy as
 *                1, 2, 3", SC'11.)
 *   gamma        [h], required.  beta: [h] or NULL (no shift); must be NULL
 *                for RMSNorm.
 *   norm, dtype  enum values above.
 *   rank         this rank's index in the TP group, 0 <= rank < t.
 *   seed         dropout seed, identical on every rank.
 *   partials     t slabs, slab k at element offset k*slab_stride, each [T][h];
 *                slab_stride >= T*h and slab_stride*elem_size % 16 == 0
 *                (sp_region_partials_stride gives the fastest layout).
 *   bias         [h] or NULL, added to the slab sum before dropout.
 *   residual     [T][h] or NULL, added after dropout.
 *   cu_seqlens   NULL for a uniform shard: the global token of local row i is
 *                g_i = rank*T + i.  Otherwise int32 [nseq+1] local row offsets
 *                (cu[0] = 0, cu[nseq] = T, non-decreasing; the caller
 *                guarantees this, it is not checked on the device): row i of
 *                sequence q has g_i = t*cu[q] + rank*(cu[q+1]-cu[q]) + (i-cu[q]).
 *   z            out [T][h]: round_to_dtype(residual + dropout(sum + bias)),
 *                summed in float32 in ascending k with no fused multiply-add.
 *   y            out [T][h]: the normalised z (statistics from the rounded z).
 *   mean, rstd   out float32 [T]; mean must be NULL for RMSNorm.
 *   mask_out     NULL, or out uint8 [T][h] (1 = kept) for inspection.
 *
 * T == 0 is a no-op returning SPR_OK.
 */
int sp_region_fwd(int64_t b, int64_t s, int64_t h, int32_t t, float eps, float p_drop,
                  const void* gamma, const void* beta,
                  int32_t norm, int32_t dtype, int32_t rank, uint64_t seed,
                  const void* partials, int64_t slab_stride,
                  const void* bias, const void* residual,
                  const int32_t* cu_seqlens, int32_t nseq,
                  void* z, void* y, float* mean, float* rstd,
                  uint8_t* mask_out,
                  void* stream);

/*
 * sp_region_fwd with the t partial slabs given as a HOST array slabs[0..t) of
 * device pointers, each to a row-major [T][h] slab, 16-byte aligned: the
 * slabs may live in separate buffers (receive buffers of a reduce-scatter,
 * say) or, peer-mapped, in other GPUs' memory -- each is read through its own
 * base address, in the same order and with the same results as the strided
 * form.  The array is read during the call only.  Every other argument,
 * check and result as in sp_region_fwd; a NULL array or slab pointer returns
 * SPR_ERR_INVALID_ARG, a misaligned slab SPR_ERR_ALIGNMENT.
 */
int sp_region_fwd_slabs(int64_t b, int64_t s, int64_t h, int32_t t, float eps, float p_drop,
                        const void* gamma, const void* beta,
                        int32_t norm, int32_t dtype, int32_t rank, uint64_t seed,
                        const void* const* slabs,
                        const void* bias, const void* residual,
                        const int32_t* cu_seqlens, int32_t nseq,
                        void* z, void* y, float* mean, float* rstd,
                        uint8_t* mask_out,
                        void* stream);

/*
 * Bytes of device workspace sp_region_bwd needs for n_local_tokens = T rows of
 * h channels: float32 dgamma/dbeta partial sums of G = min(ceil(T/4), 256) row
 * blocks (at least 4 rows per block on shards of fewer than 1024 rows),
 * two slots of h per block.  Slots and blocks sit at strides 1 KiB past a
 * multiple of 2 KiB (slot: round_up(h, 512) + 256 floats; block:
 * round_up(2*slot, 512) + 256 floats), so the blocks' simultaneous partial
 * writes spread over the HBM channels.  A pure function (no device query).
 * Returns 0 for T <= 0 or h <= 0.
 */
size_t sp_region_bwd_workspace_bytes(int64_t n_local_tokens, int64_t h);

/*
 * Backward of the normalisation (the adjoint of the forward's last step):
 * hpc.payai.win lesson 7 "Sequence parallelism", section 3.B (the backward of
 * each forward step is its adjoint, computed on the same s/t token slice),
 * applied to the LayerNorm of section 2 (mean and population variance over
 * the full h, eps inside the square root) and to RMSNorm.
 *
 *   b, s, t, h, norm, dtype   as in sp_region_fwd (T = b*s/t).
 *   gamma        [h].
 *   dy           [T][h] upstream gradient of y.
 *   z            [T][h] the forward's z.
 *   mean, rstd   the forward's float32 statistics (mean NULL for RMSNorm).
 *   dres_in      [T][h] or NULL: extra gradient arriving on z (z is also the
 *                next residual stream); added to dx.
 *   dx           out [T][h]: with xhat = (z - mean)*rstd (RMS: z*rstd),
 *                g = dy*gamma, c1 = mean_j g, c2 = mean_j(g*xhat):
 *                LayerNorm dx = rstd*(g - c1 - xhat*c2) (+ dres_in),
 *                RMSNorm   dx = rstd*(g - xhat*c2)      (+ dres_in).
 *   dgamma       out float32 [h]: sum over this rank's T rows of dy*xhat.
 *   dbeta        out float32 [h] or NULL: sum over the T rows of dy
 *                (must be NULL for RMSNorm).
 *   workspace    >= sp_region_bwd_workspace_bytes(T, h) bytes, 16-byte aligned
 *                (may be NULL when that is 0).  Contents on entry do not
 *                matter; calls that share a workspace must be ordered.
 *
 * dgamma/dbeta are reduced in one fixed order (row block b = rows b, b + G,
 * ... in order; 32 groups of blocks g, g + 32, ... in order; the groups in
 * order), so results are bitwise reproducible for a given (T, h), whichever
 * launch path runs.  Small shards (at most 4 rows per row block, G <= 128,
 * and the row and column blocks together no more than the device's compute
 * units: T <= 512 at h = 4096) take one kernel launch, in which column blocks
 * sum dgamma/dbeta from dy and z themselves and the workspace is not used;
 * otherwise the row blocks write partial sums to the workspace and a second
 * launch reduces them.  T == 0 writes zeros to dgamma/dbeta.
 */
int sp_region_bwd(int64_t b, int64_t s, int64_t h, int32_t t,
                  const void* gamma, int32_t norm, int32_t dtype,
                  const void* dy, const void* z, const float* mean, const float* rstd,
                  const void* dres_in,
                  void* dx, float* dgamma, float* dbeta,
                  void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * sp_region_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Every argument, check and result is that of sp_region_bwd (same kernels,
 * bit for bit the same outputs); the workspace is not passed: the partial
 * sums live in a static device array of SPR_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on, until the process ends.  The call
 * allocates nothing and frees nothing.
 *
 *   Limit: sp_region_bwd_workspace_bytes(T, h) <= SPR_NOALLOC_SCRATCH_BYTES
 *   (32 MiB: every shard up to h = 8192, and up to 1000 rows at h = 16384),
 *   else SPR_ERR_SCRATCH before any launch, outputs untouched.
 *   Races: every call on one GPU uses that GPU's one array, which keeps the
 *   last call's contents (the kernels need no particular contents on entry).
 *   Calls that can overlap on one GPU -- on different streams, or from
 *   different threads without ordering -- race on it and give wrong
 *   results; order them (one stream, or events).
 *   The array's address on the GPU that runs `stream` is looked up on the
 *   first call there (hipGetSymbolAddress) and kept.
 */
#define SPR_NOALLOC_SCRATCH_BYTES (32u << 20)
int sp_region_bwd_noalloc(int64_t b, int64_t s, int64_t h, int32_t t,
                          const void* gamma, int32_t norm, int32_t dtype,
                          const void* dy, const void* z, const float* mean, const float* rstd,
                          const void* dres_in,
                          void* dx, float* dgamma, float* dbeta,
                          void* stream);

/*
 * Bytes of device workspace sp_region_bwd_dropout needs for T rows of h
 * channels: as sp_region_bwd_workspace_bytes with three slots per block
 * (dgamma, dbeta and dbias partials; block stride round_up(3*slot, 512) + 256
 * floats).  A pure function; 0 for T <= 0 or h <= 0.
 */
size_t sp_region_bwd_dropout_workspace_bytes(int64_t n_local_tokens, int64_t h);

/*
 * Backward of the whole region below the normalisation: everything
 * sp_region_bwd computes, plus the gradients through the dropout and the g*
 * sum (hpc.payai.win lesson 7 "Sequence parallelism", section 3.B: the
 * backward of each step is its adjoint, and g*'s backward is an all-gather
 * that hands every TP rank the same gradient of its row-linear output).
 *
 *   b, s, h, t, gamma, norm, dtype, dy, z, mean, rstd, dres_in, dx, dgamma,
 *   dbeta        as in sp_region_bwd (dx includes dres_in).
 *   p_drop, rank, seed, cu_seqlens, nseq
 *                the forward's dropout arguments, with the same meaning and
 *                checks as in sp_region_fwd: the mask is recomputed from them,
 *                never stored.
 *   dpartial     out [T][h], the gradient of the slab sum sum_k P_k (the same
 *                for every slab k) and of the pre-dropout activation:
 *                dx * keep * float32(1/(1-p_drop)), computed from the float32
 *                dx before its rounding and rounded once; p_drop == 0 gives
 *                dpartial = dx.  Required when T > 0.
 *   dbias        out float32 [h] or NULL: sum of dpartial over the T rows, in
 *                the same fixed order as dgamma/dbeta.
 *   workspace    >= sp_region_bwd_dropout_workspace_bytes(T, h) bytes,
 *                16-byte aligned.  Contents are scratch.
 *
 * Results are bitwise reproducible for a given (T, h); dx, dgamma and dbeta
 * are bitwise those of sp_region_bwd on the same inputs.  Without dbias,
 * small shards take sp_region_bwd's one-launch path (its row blocks also
 * write dpartial); a call that wants dbias always takes the partials path.
 */
int sp_region_bwd_dropout(int64_t b, int64_t s, int64_t h, int32_t t,
                          const void* gamma, int32_t norm, int32_t dtype,
                          const void* dy, const void* z, const float* mean, const float* rstd,
                          const void* dres_in,
                          float p_drop, int32_t rank, uint64_t seed,
                          const int32_t* cu_seqlens, int32_t nseq,
                          void* dx, void* dpartial, float* dgamma, float* dbeta, float* dbias,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Backward with the parameter gradients accumulated into float32 main-grad
 * buffers, for gradient accumulation over micro-batches: the step's gradient
 * of gamma, beta and the bias sums over the tokens of every micro-batch, so
 * each micro-batch's backward adds its own sums into buffers that persist
 * across them.  The pages do not describe this step; float32 main-grad
 * buffers are the usual convention of mixed-precision training.
 *
 *   All arguments as in sp_region_bwd_dropout, except:
 *   dpartial     out [T][h] or NULL.  NULL: no gradient through the dropout
 *                and the slab sum (dbias must then be NULL too when T > 0);
 *                the dropout arguments are still checked but otherwise
 *                unused, and the call is sp_region_bwd with accumulation.
 *   dgamma, dbeta, dbias
 *                in/out float32 [h] (dbeta and dbias may be NULL): element j
 *                becomes float32(old_j + sum_j), where sum_j is, bit for bit,
 *                what sp_region_bwd_dropout (dpartial given) or sp_region_bwd
 *                (dpartial NULL) writes for the same inputs.
 *   workspace    >= sp_region_bwd_dropout_workspace_bytes(T, h) bytes when
 *                dpartial is given, else >= sp_region_bwd_workspace_bytes(T, h).
 *
 * dx and dpartial are overwritten, as in the other calls.  T == 0 launches
 * nothing and leaves every buffer as it was.  The buffers are read and
 * written by the call's last kernel, so calls that accumulate into the same
 * buffers must be ordered (one stream, or events between streams).
 */
int sp_region_bwd_accumulate(int64_t b, int64_t s, int64_t h, int32_t t,
                             const void* gamma, int32_t norm, int32_t dtype,
                             const void* dy, const void* z, const float* mean, const float* rstd,
                             const void* dres_in,
                             float p_drop, int32_t rank, uint64_t seed,
                             const int32_t* cu_seqlens, int32_t nseq,
                             void* dx, void* dpartial, float* dgamma, float* dbeta, float* dbias,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * Host-side batch planning (no device work; pointers are HOST pointers).
 *
 * coreui.cn, "Why Sequence Parallel saves memory but makes throughput
 * jitter: from reduce-scatter to the LayerNorm boundary", section "stabilise
 * the shapes first, then define the LayerNorm shard contract": the step
 * function buckets the batch by length with a length coefficient of
 * variation (CV) of at most 0.15 and runs a bucket with tensor parallelism
 * alone when its CV exceeds 0.18 or the reduce-scatter wait share exceeds
 * 0.22.  CV = population standard deviation / mean of the sequence lengths
 * (0 for an empty or all-zero set).  CV thresholds are integers in basis
 * points (1500 = 0.15), and "CV <= c" is decided exactly in integer
 * arithmetic:  1e8 * (n*sum(x^2) - sum(x)^2) <= c_bp^2 * sum(x)^2.
 * Limits: n <= 2^20 sequences, 0 <= length <= 2^24, 0 <= c_bp <= 100000.
 * Arguments outside them, or NULL outputs, return SPR_ERR_INVALID_ARG and
 * write nothing.
 * ------------------------------------------------------------------------ */
#define SPR_MAX_CV_BP 1500          /* bucket_by_tokens(max_cv = 0.15) */
#define SPR_GATE_CV_BP 1800         /* TP alone above a bucket length CV of 0.18 */
#define SPR_GATE_RS_WAIT 0.22       /* ... or above a reduce-scatter wait share of 0.22 */

/* *within = 1 iff CV(lengths[0..n)) <= cv_bp / 10^4. */
int sp_region_cv_within(const int32_t* lengths, int32_t n, int32_t cv_bp, int32_t* within);

/*
 * Length buckets: the batch sorted by (length, index) and cut greedily, the
 * next sequence joining the current bucket while the bucket's CV stays
 * <= max_cv_bp and, if max_tokens > 0, its token total stays <= max_tokens;
 * the first sequence of a bucket always joins it.
 *   order         out [n]: sequence indices, bucket by bucket.
 *   bucket_start  out [n+1]: bucket k is order[bucket_start[k] ..
 *                 bucket_start[k+1]); entries 0..*n_buckets are written.
 *   n_buckets     out.
 */
int sp_region_bucket_by_tokens(const int32_t* lengths, int32_t n, int32_t max_cv_bp, int64_t max_tokens,
                               int32_t* order, int32_t* bucket_start, int32_t* n_buckets);

/*
 * SP gate of one bucket: *use_sp = 1 iff CV(lengths) <= max_cv_bp / 10^4 and
 * rs_wait_share <= max_rs_wait_share (SPR_GATE_CV_BP and SPR_GATE_RS_WAIT are
 * the page's values); 0 means run the bucket with tensor parallelism alone.
 * NaN shares are invalid.
 */
int sp_region_sp_gate(const int32_t* lengths, int32_t n, double rs_wait_share, int32_t max_cv_bp,
                      double max_rs_wait_share, int32_t* use_sp);

/*
 * Packed shard layout of a bucket for TP degree t (1..SPR_MAX_T_SLABS): each
 * sequence is padded up to a multiple of t (padded[q]); rank r holds the
 * r-th of the t equal slices of every sequence, so every rank has the same
 * T = sum(padded)/t local rows, and cu_local [n+1] are the local row offsets
 * that sp_region_fwd / sp_region_bwd_dropout take as cu_seqlens (with b = 1,
 * s = sum(padded)).  T beyond INT32_MAX returns SPR_ERR_UNSUPPORTED.
 */
int sp_region_shard_layout(const int32_t* lengths, int32_t n, int32_t t, int32_t* padded, int32_t* cu_local,
                           int64_t* n_local_tokens);

/*
 * Launch path of the backward calls (sp_region_bwd and its accumulating and
 * allocation-free forms), process-wide: 1 (default) = one launch on small
 * shards as sp_region_bwd describes, 2 = always the row launch followed by
 * the column-reduction launch.  Results are bitwise identical; the setting
 * exists for tests and measurements.  Returns SPR_ERR_INVALID_ARG for other
 * values.
 */
int sp_region_set_bwd_launches(int32_t launches);

/*
 * Calibration kernel: copies nbytes (a multiple of 16) from src to dst with
 * 16-byte loads and stores, for measuring the achievable HBM copy rate and for
 * scaling hardware traffic counters.  Not part of the region's computation.
 */
int sp_region_hbm_copy(const void* src, void* dst, size_t nbytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SP_REGION_H_ */

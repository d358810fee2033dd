/*
 * A plain C99 client of libsp_region: the library used through
 * include/sp_region.h alone, with the HIP runtime's own allocator and stream,
 * no Python and no torch.  The tests run it and compare what it prints or
 * writes with the CPU oracle.
 *
 *   sp_region_client host T_TP LEN...
 *       Host-only entry points (no device is touched): the ABI version, the
 *       slab stride and workspace sizes of a 2048 x 8192 bf16 shard, the
 *       length-CV test, the SP gate, the length buckets and the shard layout
 *       of the given sequence lengths for TP degree T_TP, and the status of a
 *       rejected forward call.  One "key values..." line each.
 *
 *   sp_region_client gpu DIR
 *       Reads DIR/params.txt ("key value" lines: b s h t rank seed p_drop eps
 *       dtype norm bias residual) and the raw little-endian arrays
 *       DIR/partials.bin [t][T][h], gamma.bin, beta.bin (LayerNorm), bias.bin
 *       and residual.bin (when enabled) and dy.bin, all in the storage dtype;
 *       runs sp_region_fwd and sp_region_bwd_dropout on one HIP stream and
 *       writes z y mean rstd dx dpartial dgamma dbeta dbias (.bin) to DIR.
 *
 * Exit status 0 on success; any failing call prints its name and status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sp_region.h"

static int fail(const char* what, int code) {
  fprintf(stderr, "sp_region_client: %s failed (%d)\n", what, code);
  return 1;
}

#define HIP_OK(call)                                       \
  do {                                                     \
    hipError_t e_ = (call);                                \
    if (e_ != hipSuccess) return fail(#call, (int)e_);     \
  } while (0)

#define SPR_OK_(call)                                                        \
  do {                                                                       \
    int s_ = (call);                                                         \
    if (s_ != SPR_OK) {                                                      \
      fprintf(stderr, "sp_region_client: %s -> %s (last hip error %d)\n",    \
              #call, sp_region_strerror(s_), sp_region_last_hip_error());    \
      return 1;                                                              \
    }                                                                        \
  } while (0)

static int run_host(int argc, char** argv) {
  if (argc < 4) return fail("usage: host T_TP LEN...", 2);
  const int32_t t = (int32_t)atoi(argv[2]);
  const int32_t n = (int32_t)(argc - 3);
  int32_t* len = calloc((size_t)n, sizeof *len);
  int32_t* order = calloc((size_t)n, sizeof *order);
  int32_t* starts = calloc((size_t)n + 1, sizeof *starts);
  int32_t* padded = calloc((size_t)n, sizeof *padded);
  int32_t* cu = calloc((size_t)n + 1, sizeof *cu);
  if (!len || !order || !starts || !padded || !cu) return fail("calloc", 0);
  for (int32_t i = 0; i < n; ++i) len[i] = (int32_t)atoi(argv[3 + i]);

  printf("abi %d\n", sp_region_abi_version());
  printf("stride %lld\n", (long long)sp_region_partials_stride(2048, 8192, SPR_BF16));
  printf("workspace %zu %zu\n", sp_region_bwd_workspace_bytes(2048, 8192),
         sp_region_bwd_dropout_workspace_bytes(2048, 8192));

  int32_t within = -1, use_sp = -1, nb = -1;
  int64_t T = -1;
  SPR_OK_(sp_region_cv_within(len, n, SPR_MAX_CV_BP, &within));
  printf("cv_within %d\n", within);
  SPR_OK_(sp_region_sp_gate(len, n, 0.1, SPR_GATE_CV_BP, SPR_GATE_RS_WAIT, &use_sp));
  printf("sp_gate %d\n", use_sp);
  SPR_OK_(sp_region_bucket_by_tokens(len, n, SPR_MAX_CV_BP, 0, order, starts, &nb));
  printf("bucket_starts");
  for (int32_t k = 0; k <= nb; ++k) printf(" %d", starts[k]);
  printf("\nbucket_order");
  for (int32_t i = 0; i < n; ++i) printf(" %d", order[i]);
  SPR_OK_(sp_region_shard_layout(len, n, t, padded, cu, &T));
  printf("\nlayout_T %lld\nlayout_padded", (long long)T);
  for (int32_t i = 0; i < n; ++i) printf(" %d", padded[i]);
  printf("\nlayout_cu");
  for (int32_t i = 0; i <= n; ++i) printf(" %d", cu[i]);
  /* t = 0 is outside the forward's domain: a status, and no launch. */
  printf("\nreject_t0 %d\n", sp_region_fwd(1, 8, 64, 0, 1e-5f, 0.0f, NULL, NULL, SPR_LAYERNORM, SPR_BF16, 0, 0,
                                            NULL, 0, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL));
  free(len); free(order); free(starts); free(padded); free(cu);
  return 0;
}

/* ---- gpu mode ---------------------------------------------------------- */

typedef struct {
  long long b, s, h, t, rank, dtype, norm, bias, residual;
  unsigned long long seed;
  double p_drop, eps;
} Params;

static int read_params(const char* dir, Params* p) {
  char path[4096];
  snprintf(path, sizeof path, "%s/params.txt", dir);
  FILE* f = fopen(path, "r");
  if (!f) return fail("open params.txt", 0);
  char key[64], val[128];
  memset(p, 0, sizeof *p);
  while (fscanf(f, "%63s %127s", key, val) == 2) {
    const long long v = strtoll(val, NULL, 10);
    if (!strcmp(key, "b")) p->b = v;
    else if (!strcmp(key, "s")) p->s = v;
    else if (!strcmp(key, "h")) p->h = v;
    else if (!strcmp(key, "t")) p->t = v;
    else if (!strcmp(key, "rank")) p->rank = v;
    else if (!strcmp(key, "seed")) p->seed = strtoull(val, NULL, 10);   /* all 64 bits */
    else if (!strcmp(key, "dtype")) p->dtype = v;
    else if (!strcmp(key, "norm")) p->norm = v;
    else if (!strcmp(key, "bias")) p->bias = v;
    else if (!strcmp(key, "residual")) p->residual = v;
    else if (!strcmp(key, "p_drop")) p->p_drop = strtod(val, NULL);
    else if (!strcmp(key, "eps")) p->eps = strtod(val, NULL);
  }
  fclose(f);
  return 0;
}

/* Reads DIR/name into a new device buffer of exactly `bytes` bytes. */
static int load(const char* dir, const char* name, size_t bytes, void** dev) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return fail(path, 0);
  void* host = malloc(bytes ? bytes : 1);
  if (!host) return fail("malloc", 0);
  const size_t got = fread(host, 1, bytes, f);
  fclose(f);
  if (got != bytes) return fail(path, (int)got);
  HIP_OK(hipMalloc(dev, bytes ? bytes : 16));
  HIP_OK(hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice));
  free(host);
  return 0;
}

static int save(const char* dir, const char* name, const void* dev, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  void* host = malloc(bytes ? bytes : 1);
  if (!host) return fail("malloc", 0);
  HIP_OK(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
  FILE* f = fopen(path, "wb");
  if (!f) return fail(path, 0);
  const size_t put = fwrite(host, 1, bytes, f);
  fclose(f);
  free(host);
  return put == bytes ? 0 : fail(path, (int)put);
}

static int run_gpu(const char* dir) {
  Params p;
  if (read_params(dir, &p)) return 1;
  if (p.t < 1 || p.b < 1 || p.s < 0 || p.h < 1) return fail("params.txt shape", 0);
  const long long T = p.b * p.s / p.t;
  const size_t eb = p.dtype == SPR_BF16 ? 2 : 4;
  const size_t row = (size_t)p.h * eb, act = (size_t)T * row, vec = (size_t)p.h * eb, f32h = (size_t)p.h * 4;
  const int ln = p.norm == SPR_LAYERNORM;

  void *P = NULL, *gamma = NULL, *beta = NULL, *bias = NULL, *res = NULL, *dy = NULL;
  if (load(dir, "partials.bin", (size_t)p.t * act, &P) || load(dir, "gamma.bin", vec, &gamma) ||
      load(dir, "dy.bin", act, &dy))
    return 1;
  if (ln && load(dir, "beta.bin", vec, &beta)) return 1;
  if (p.bias && load(dir, "bias.bin", vec, &bias)) return 1;
  if (p.residual && load(dir, "residual.bin", act, &res)) return 1;

  void *z, *y, *dx, *dpart, *ws;
  float *mean = NULL, *rstd, *dgamma, *dbeta = NULL, *dbias;
  const size_t wsb = sp_region_bwd_dropout_workspace_bytes(T, p.h);
  HIP_OK(hipMalloc(&z, act ? act : 16));
  HIP_OK(hipMalloc(&y, act ? act : 16));
  HIP_OK(hipMalloc(&dx, act ? act : 16));
  HIP_OK(hipMalloc(&dpart, act ? act : 16));
  HIP_OK(hipMalloc((void**)&rstd, (size_t)T * 4 + 16));
  if (ln) HIP_OK(hipMalloc((void**)&mean, (size_t)T * 4 + 16));
  HIP_OK(hipMalloc((void**)&dgamma, f32h));
  if (ln) HIP_OK(hipMalloc((void**)&dbeta, f32h));
  HIP_OK(hipMalloc((void**)&dbias, f32h));
  HIP_OK(hipMalloc(&ws, wsb ? wsb : 16));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  SPR_OK_(sp_region_fwd(p.b, p.s, p.h, (int32_t)p.t, (float)p.eps, (float)p.p_drop, gamma, beta, (int32_t)p.norm,
                        (int32_t)p.dtype, (int32_t)p.rank, (uint64_t)p.seed, P, (int64_t)(T * p.h), bias, res,
                        NULL, 0, z, y, mean, rstd, NULL, stream));
  SPR_OK_(sp_region_bwd_dropout(p.b, p.s, p.h, (int32_t)p.t, gamma, (int32_t)p.norm, (int32_t)p.dtype, dy, z, mean,
                                rstd, NULL, (float)p.p_drop, (int32_t)p.rank, (uint64_t)p.seed, NULL, 0, dx, dpart,
                                dgamma, dbeta, dbias, ws, wsb, stream));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipStreamDestroy(stream));

  if (save(dir, "z.bin", z, act) || save(dir, "y.bin", y, act) || save(dir, "rstd.bin", rstd, (size_t)T * 4) ||
      save(dir, "dx.bin", dx, act) || save(dir, "dpartial.bin", dpart, act) ||
      save(dir, "dgamma.bin", dgamma, f32h) || save(dir, "dbias.bin", dbias, f32h))
    return 1;
  if (ln && (save(dir, "mean.bin", mean, (size_t)T * 4) || save(dir, "dbeta.bin", dbeta, f32h))) return 1;

  void* bufs[] = {P, gamma, beta, bias, res, dy, z, y, dx, dpart, mean, rstd, dgamma, dbeta, dbias, ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) HIP_OK(hipFree(bufs[i]));
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && !strcmp(argv[1], "host")) return run_host(argc, argv);
  if (argc == 3 && !strcmp(argv[1], "gpu")) return run_gpu(argv[2]);
  fprintf(stderr, "usage: sp_region_client host T_TP LEN... | gpu DIR\n");
  return 2;
}

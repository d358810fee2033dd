// Host-side batch planning around the SP region (no device work): length
// buckets, the SP gate and the packed shard layout of a ragged batch.
//
// The step function of coreui.cn's "Why Sequence Parallel saves memory but
// makes throughput jitter" (section "stabilise the shapes first, then define
// the LayerNorm shard contract") buckets the batch by length with a length
// coefficient of variation of at most 0.15, and falls back to tensor
// parallelism alone when a bucket's CV exceeds 0.18 or the reduce-scatter
// wait share exceeds 0.22.  The page names the steps only; the readings
// taken here: CV is the population standard deviation over the mean; a
// bucket is a greedy run of the batch sorted by (length, index); "CV <= c"
// is decided exactly in integers with c in basis points:
//     1e8 * (n * sum(x^2) - sum(x)^2) <= c_bp^2 * sum(x)^2,
// which is population variance <= c^2 * mean^2 scaled by n^2 * 1e8.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "sp_region.h"

namespace {

constexpr int32_t kMaxSeqs = 1 << 20;     // sequences per call
constexpr int32_t kMaxLen = 1 << 24;      // tokens per sequence
constexpr int32_t kMaxCvBp = 100000;      // CV thresholds up to 10.0

// n <= 2^20 and x <= 2^24 keep every product below 2^123.
struct Moments {
  int64_t n = 0;
  __int128 s1 = 0, s2 = 0;
  void add(int64_t x) {
    ++n;
    s1 += x;
    s2 += static_cast<__int128>(x) * x;
  }
};

bool within(const Moments& m, int32_t cv_bp) {
  const __int128 lhs = static_cast<__int128>(100000000) * (static_cast<__int128>(m.n) * m.s2 - m.s1 * m.s1);
  const __int128 rhs = static_cast<__int128>(cv_bp) * cv_bp * m.s1 * m.s1;
  return lhs <= rhs;
}

int check_lengths(const int32_t* lengths, int32_t n) {
  if (n < 0 || n > kMaxSeqs) return SPR_ERR_INVALID_ARG;
  if (n > 0 && lengths == nullptr) return SPR_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (lengths[i] < 0 || lengths[i] > kMaxLen) return SPR_ERR_INVALID_ARG;
  return SPR_OK;
}

}  // namespace

extern "C" {

int sp_region_cv_within(const int32_t* lengths, int32_t n, int32_t cv_bp, int32_t* out_within) {
  const int st = check_lengths(lengths, n);
  if (st != SPR_OK) return st;
  if (cv_bp < 0 || cv_bp > kMaxCvBp || out_within == nullptr) return SPR_ERR_INVALID_ARG;
  Moments m;
  for (int32_t i = 0; i < n; ++i) m.add(lengths[i]);
  *out_within = within(m, cv_bp) ? 1 : 0;
  return SPR_OK;
}

int sp_region_bucket_by_tokens(const int32_t* lengths, int32_t n, int32_t max_cv_bp, int64_t max_tokens,
                               int32_t* order, int32_t* bucket_start, int32_t* n_buckets) {
  const int st = check_lengths(lengths, n);
  if (st != SPR_OK) return st;
  if (max_cv_bp < 0 || max_cv_bp > kMaxCvBp || max_tokens < 0) return SPR_ERR_INVALID_ARG;
  if (n_buckets == nullptr || bucket_start == nullptr || (n > 0 && order == nullptr)) return SPR_ERR_INVALID_ARG;
  std::vector<int32_t> idx(static_cast<size_t>(n));
  std::iota(idx.begin(), idx.end(), 0);
  std::sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) {
    return lengths[a] != lengths[b] ? lengths[a] < lengths[b] : a < b;
  });
  int32_t nb = 0;
  Moments cur;
  for (int32_t pos = 0; pos < n; ++pos) {
    const int64_t x = lengths[idx[pos]];
    Moments cand = cur;
    cand.add(x);
    const bool fits = within(cand, max_cv_bp) && (max_tokens == 0 || cand.s1 <= max_tokens);
    if (cur.n == 0 || !fits) {   // the first sequence of a bucket always joins it
      bucket_start[nb++] = pos;
      cur = Moments{};
      cur.add(x);
    } else {
      cur = cand;
    }
    order[pos] = idx[pos];
  }
  bucket_start[nb] = n;
  *n_buckets = nb;
  return SPR_OK;
}

int sp_region_sp_gate(const int32_t* lengths, int32_t n, double rs_wait_share, int32_t max_cv_bp,
                      double max_rs_wait_share, int32_t* use_sp) {
  const int st = check_lengths(lengths, n);
  if (st != SPR_OK) return st;
  if (max_cv_bp < 0 || max_cv_bp > kMaxCvBp || use_sp == nullptr) return SPR_ERR_INVALID_ARG;
  if (std::isnan(rs_wait_share) || std::isnan(max_rs_wait_share)) return SPR_ERR_INVALID_ARG;
  Moments m;
  for (int32_t i = 0; i < n; ++i) m.add(lengths[i]);
  *use_sp = (within(m, max_cv_bp) && !(rs_wait_share > max_rs_wait_share)) ? 1 : 0;
  return SPR_OK;
}

int sp_region_shard_layout(const int32_t* lengths, int32_t n, int32_t t, int32_t* padded, int32_t* cu_local,
                           int64_t* n_local_tokens) {
  const int st = check_lengths(lengths, n);
  if (st != SPR_OK) return st;
  if (t < 1 || t > SPR_MAX_T_SLABS || cu_local == nullptr || n_local_tokens == nullptr ||
      (n > 0 && padded == nullptr))
    return SPR_ERR_INVALID_ARG;
  int64_t T = 0;
  for (int32_t q = 0; q < n; ++q) {
    const int64_t p = (static_cast<int64_t>(lengths[q]) + t - 1) / t * t;
    if (T + p / t > INT32_MAX) return SPR_ERR_UNSUPPORTED;   // cu_seqlens are int32
    T += p / t;
  }
  T = 0;
  cu_local[0] = 0;
  for (int32_t q = 0; q < n; ++q) {
    const int64_t p = (static_cast<int64_t>(lengths[q]) + t - 1) / t * t;
    padded[q] = static_cast<int32_t>(p);
    T += p / t;
    cu_local[q + 1] = static_cast<int32_t>(T);
  }
  *n_local_tokens = T;
  return SPR_OK;
}

}  // extern "C"

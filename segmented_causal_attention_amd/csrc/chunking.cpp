// Host planner: workload-balanced chunking of a packed variable-length batch
// (InfiniPipe, section III-B "Sequence Processor", Algorithm 1; the time of a
// slice is the computation cost of section III-A2, eq. (1)).
//
//   cost     a slice of s tokens after a context of C tokens costs
//            alpha1 ((C + s)^2 - C^2) + alpha2 s; a chunk the sum over its
//            slices (the factor 1/N and the per-chunk constant of eq. (1)
//            are the same for every chunk on one device and are left out).
//   mesh     the longest sequence L cut into K slices of equal cost: inner
//            boundary i is the integer b minimising |K f(b) - i f(L)| with
//            f(b) = alpha1 b^2 + alpha2 b, ties to the smaller b.
//   split    every sequence is cut at the inner mesh boundaries that lie
//            inside it: the pieces before the last cut are split chunks,
//            the last piece is a tail slice; a sequence without a cut is
//            short.
//   pack     best-fit-decreasing: one bucket per tail slice, ordered by
//            time / tokens ascending; short sequences, longest first, join
//            the first bucket within the time threshold T_t (initially one
//            mesh slice's cost) and the token threshold T_m (the caller's
//            token capacity); a sequence no bucket can take within T_m opens
//            a new bucket, and one that only misses T_t loosens it to the
//            least bucket time plus its own over the buckets within T_m.
//   output   split chunks, then the buckets in the order they were opened
//            (hybrid chunks: a tail plus short sequences; batched chunks:
//            short sequences only), each slice as a work item.
//
// The float64 operations are written out one by one and uncontracted, so
// their rounding is fixed and reproducible.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "segattn.h"
#include "status.h"

#pragma clang fp contract(off)

namespace {

constexpr int64_t kMaxTokens = 0x7fffffffLL;

struct Piece {
  int32_t seq;
  int64_t ctx, len;
};

struct Bucket {
  int32_t id;
  double time;
  int64_t tokens;
  bool tail;
  std::vector<Piece> members;
};

double piece_time(int64_t ctx, int64_t s, double a1, double a2) {
  const int64_t quad = s * (2 * ctx + s);  // (ctx + s)^2 - ctx^2, exact below 2^63
  const double q = a1 * (double)quad;
  const double l = a2 * (double)s;
  return q + l;
}

double mesh_f(int64_t b, double a1, double a2) {
  const double q = a1 * (double)(b * b);
  const double l = a2 * (double)b;
  return q + l;
}

// Boundaries 0 = b_0 < ... < b_K = L.
std::vector<int64_t> make_mesh(int64_t L, int32_t K, double a1, double a2) {
  std::vector<int64_t> b{0};
  const double total = mesh_f(L, a1, a2);
  for (int32_t i = 1; i < K; ++i) {
    const double goal = (double)i * total;
    const double t = goal / (double)K;
    const double disc = a2 * a2 + 4.0 * a1 * t;
    const double root = (-a2 + std::sqrt(disc)) / (2.0 * a1);
    const int64_t lo = b.back() + 1, hi = L - (K - i);
    const int64_t fl = (int64_t)std::floor(root);
    int64_t best = -1;
    double best_err = 0.0;
    for (int64_t c = fl - 1; c <= fl + 2; ++c) {
      const int64_t x = std::min(std::max(c, lo), hi);
      const double err = std::fabs((double)K * mesh_f(x, a1, a2) - goal);
      if (best < 0 || err < best_err || (err == best_err && x < best)) {
        best = x;
        best_err = err;
      }
    }
    b.push_back(best);
  }
  b.push_back(L);
  return b;
}

}  // namespace

extern "C" int segattn_chunk_varlen(const int64_t *cu, int32_t nseq, int32_t K, double alpha1, double alpha2,
                                    int64_t token_cap, segattn_item *items, int32_t *chunk_of, int32_t cap,
                                    int32_t *n_items, int32_t *n_chunks, double *time_threshold) {
  using segattn::fail;
  segattn::clear_error();
  static const char *fn = "segattn_chunk_varlen";
  if (!cu || !n_items || !n_chunks) return fail(SEGATTN_E_INVALID, "%s: NULL pointer", fn);
  if (nseq < 1) return fail(SEGATTN_E_INVALID, "%s: nseq = %d < 1", fn, nseq);
  if (K < 1) return fail(SEGATTN_E_INVALID, "%s: K = %d < 1", fn, K);
  if (!(alpha1 > 0.0) || !(alpha1 < 1e300) || !(alpha2 >= 0.0) || !(alpha2 < 1e300))
    return fail(SEGATTN_E_INVALID, "%s: need finite alpha1 > 0 and alpha2 >= 0", fn);
  if (token_cap < 1) return fail(SEGATTN_E_INVALID, "%s: token_cap < 1", fn);
  if (cap < 0 || (cap > 0 && !items)) return fail(SEGATTN_E_INVALID, "%s: bad items/cap", fn);
  if (cu[0] != 0) return fail(SEGATTN_E_INVALID, "%s: cu_seqlens[0] != 0", fn);
  int64_t L = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    if (cu[s + 1] < cu[s]) return fail(SEGATTN_E_INVALID, "%s: cu_seqlens decreases at %d", fn, s);
    L = std::max(L, cu[s + 1] - cu[s]);
  }
  if (cu[nseq] > kMaxTokens) return fail(SEGATTN_E_RANGE, "%s: %lld tokens > 2^31-1", fn, (long long)cu[nseq]);
  if (L == 0) return fail(SEGATTN_E_INVALID, "%s: every sequence is empty", fn);

  // The mesh and the thresholds.
  const int32_t Km = (int32_t)std::min<int64_t>(K, L);
  const std::vector<int64_t> mesh = make_mesh(L, Km, alpha1, alpha2);
  double t_t = mesh_f(L, alpha1, alpha2) / (double)Km;
  const int64_t t_m = token_cap;

  // Cut every sequence by the inner mesh boundaries inside it.
  std::vector<Piece> split_chunks, tails, shorts;
  for (int32_t s = 0; s < nseq; ++s) {
    const int64_t len = cu[s + 1] - cu[s];
    if (len == 0) continue;
    int64_t start = 0;
    bool cut = false;
    for (int32_t i = 1; i < Km; ++i) {
      if (mesh[i] >= len) break;
      split_chunks.push_back({s, start, mesh[i] - start});
      start = mesh[i];
      cut = true;
    }
    if (cut) tails.push_back({s, start, len - start});
    else shorts.push_back({s, 0, len});
  }

  // Best-fit-decreasing packing.
  std::vector<Bucket> buckets;
  for (const Piece &p : tails)
    buckets.push_back({(int32_t)buckets.size(), piece_time(p.ctx, p.len, alpha1, alpha2), p.len, true, {p}});
  std::vector<double> stime(shorts.size());
  for (size_t i = 0; i < shorts.size(); ++i) stime[i] = piece_time(0, shorts[i].len, alpha1, alpha2);
  std::vector<size_t> order(shorts.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](size_t a, size_t b) {
    if (stime[a] != stime[b]) return stime[a] > stime[b];
    return shorts[a].seq < shorts[b].seq;
  });
  std::vector<size_t> by_metric;
  for (size_t oi : order) {
    const Piece &p = shorts[oi];
    const double t = stime[oi];
    const int64_t n = p.len;
    for (;;) {
      int64_t fewest = INT64_MAX;
      for (const Bucket &b : buckets) fewest = std::min(fewest, b.tokens);
      if (buckets.empty() || fewest + n > t_m) {
        buckets.push_back({(int32_t)buckets.size(), t, n, false, {p}});
        break;
      }
      by_metric.resize(buckets.size());
      for (size_t i = 0; i < buckets.size(); ++i) by_metric[i] = i;
      std::sort(by_metric.begin(), by_metric.end(), [&](size_t a, size_t b) {
        const double ma = buckets[a].time / (double)buckets[a].tokens;
        const double mb = buckets[b].time / (double)buckets[b].tokens;
        if (ma != mb) return ma < mb;
        return buckets[a].id < buckets[b].id;
      });
      bool placed = false;
      for (size_t bi : by_metric) {
        Bucket &b = buckets[bi];
        if (b.time + t <= t_t && b.tokens + n <= t_m) {
          b.time = b.time + t;
          b.tokens += n;
          b.members.push_back(p);
          placed = true;
          break;
        }
      }
      if (placed) break;
      // Loosen T_t to the least time the sequence could join at, over the
      // buckets within T_m (the check above guarantees there is one).
      bool first = true;
      for (const Bucket &b : buckets)
        if (b.tokens + n <= t_m) {
          const double v = b.time + t;
          if (first || v < t_t) t_t = v;
          first = false;
        }
    }
  }

  // Items of the split chunks, then of the buckets.
  int64_t needed = (int64_t)split_chunks.size();
  for (const Bucket &b : buckets) needed += (int64_t)b.members.size();
  const int64_t nch = (int64_t)split_chunks.size() + (int64_t)buckets.size();
  if (needed > 0x7fffffff) return fail(SEGATTN_E_RANGE, "%s: too many items", fn);
  if (needed > cap) {
    *n_items = (int32_t)needed;
    return fail(SEGATTN_E_CAPACITY, "%s: %lld items needed, capacity %d", fn, (long long)needed, cap);
  }
  int64_t w = 0, c = 0;
  auto put = [&](const Piece &p) {
    const int64_t hi = p.ctx + p.len;
    items[w] = segattn_item{cu[p.seq], p.ctx, hi, 0, hi};
    if (chunk_of) chunk_of[w] = (int32_t)c;
    ++w;
  };
  for (const Piece &p : split_chunks) {
    put(p);
    ++c;
  }
  for (const Bucket &b : buckets) {
    for (const Piece &p : b.members) put(p);
    ++c;
  }
  *n_items = (int32_t)needed;
  *n_chunks = (int32_t)nch;
  if (time_threshold) *time_threshold = t_t;
  return SEGATTN_OK;
}

// Host planner: FLOPs-balanced segment boundaries, variable-length slicing and
// ring-order work items.  Integer arithmetic only (128-bit products), so the
// results are exact and reproducible bit for bit.
//
// SPPO (Adaptive Sequence Pipeline Parallel Offloading), section 3.2: the
// FLOPs-based policy keeps the attention work of every subsequence equal,
// which under the causal mask makes earlier subsequences longer; section 5.2
// takes such a FLOPs-optimized partition s0..sN as given.  InfiniPipe eq. (1)
// prices a slice s with context C by the quadratic term (C+s)^2 - C^2; with
// the diagonal counted, the prefix of length b holds T(b) = b(b+1)/2 visible
// (query, key) pairs, and boundary i is the integer b nearest (in work) to
// i/N of T(S).
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "segattn.h"
#include "status.h"

namespace segattn {

namespace {
thread_local std::string g_error;
}

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

void clear_error() { g_error.clear(); }

const char *last_error() { return g_error.c_str(); }

namespace {

using i128 = __int128;
constexpr int64_t kMaxTokens = 0x7fffffffLL;

inline i128 tri(int64_t x) { return (i128)x * (i128)(x + 1) / 2; }

inline i128 iabs(i128 x) { return x < 0 ? -x : x; }

// Integer b in [0, S] minimising |n*T(b) - goal|, ties to the smaller b.
// T is strictly increasing, so the least b with n*T(b) >= goal and its
// predecessor are the only candidates.
int64_t nearest_boundary(i128 goal, int64_t n, int64_t S) {
  int64_t lo = 0, hi = S;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if ((i128)n * tri(mid) >= goal)
      hi = mid;
    else
      lo = mid + 1;
  }
  if (lo > 0 && iabs((i128)n * tri(lo - 1) - goal) <= iabs((i128)n * tri(lo) - goal)) return lo - 1;
  return lo;
}

// Boundaries of an N-way FLOPs-balanced partition of S tokens into out[0..N].
int partition_into(int64_t S, int64_t N, int64_t *out) {
  const i128 total = tri(S);
  out[0] = 0;
  for (int64_t i = 1; i < N; ++i) out[i] = nearest_boundary((i128)i * total, N, S);
  out[N] = S;
  for (int64_t i = 0; i < N; ++i)
    if (out[i + 1] <= out[i])
      return fail(SEGATTN_E_RANGE, "segment %lld of a %lld-way partition of %lld tokens is empty",
                  (long long)i, (long long)N, (long long)S);
  return SEGATTN_OK;
}

// First (longest) slice of the n-way partition of L tokens.
int64_t first_slice(int64_t L, int64_t n) { return nearest_boundary(tri(L), n, L); }

}  // namespace
}  // namespace segattn

using namespace segattn;

extern "C" int segattn_partition(int64_t S, int32_t N, int64_t *bounds) {
  clear_error();
  if (!bounds) return fail(SEGATTN_E_INVALID, "segattn_partition: bounds is NULL");
  if (N < 1) return fail(SEGATTN_E_INVALID, "segattn_partition: N = %d < 1", N);
  if (S < N) return fail(SEGATTN_E_RANGE, "segattn_partition: S = %lld < N = %d", (long long)S, N);
  if (S > kMaxTokens) return fail(SEGATTN_E_RANGE, "segattn_partition: S = %lld > 2^31-1", (long long)S);
  // Work in a local copy so nothing is written on error.
  int64_t local_small[65];
  int64_t *tmp = local_small;
  std::string heap;
  if (N + 1 > 65) {
    heap.resize(sizeof(int64_t) * (size_t)(N + 1));
    tmp = reinterpret_cast<int64_t *>(&heap[0]);
  }
  int rc = partition_into(S, N, tmp);
  if (rc) return rc;
  std::memcpy(bounds, tmp, sizeof(int64_t) * (size_t)(N + 1));
  return SEGATTN_OK;
}

extern "C" int segattn_partition_varlen(const int64_t *cu, int32_t nseq, int64_t max_slice,
                                        segattn_item *items, int32_t cap, int32_t *n_items) {
  clear_error();
  if (!cu || !n_items) return fail(SEGATTN_E_INVALID, "segattn_partition_varlen: NULL pointer");
  if (nseq < 0) return fail(SEGATTN_E_INVALID, "segattn_partition_varlen: nseq = %d < 0", nseq);
  if (max_slice < 1) return fail(SEGATTN_E_INVALID, "segattn_partition_varlen: max_slice < 1");
  if (cap < 0 || (cap > 0 && !items)) return fail(SEGATTN_E_INVALID, "segattn_partition_varlen: bad items/cap");
  if (cu[0] != 0) return fail(SEGATTN_E_INVALID, "segattn_partition_varlen: cu_seqlens[0] != 0");
  for (int32_t s = 0; s < nseq; ++s)
    if (cu[s + 1] < cu[s])
      return fail(SEGATTN_E_INVALID, "segattn_partition_varlen: cu_seqlens decreases at %d", s);
  if (cu[nseq] > kMaxTokens)
    return fail(SEGATTN_E_RANGE, "segattn_partition_varlen: %lld tokens > 2^31-1", (long long)cu[nseq]);

  // Pass 1: slice counts (and validity); pass 2: write.
  int64_t needed = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    const int64_t L = cu[s + 1] - cu[s];
    if (L == 0) continue;
    if (L <= max_slice) {
      needed += 1;
      continue;
    }
    // first_slice(L, n) is non-increasing in n: bisect the least n >= 2 with
    // a first slice no longer than max_slice.
    int64_t lo = 2, hi = L;
    while (lo < hi) {
      int64_t mid = lo + (hi - lo) / 2;
      if (first_slice(L, mid) <= max_slice)
        hi = mid;
      else
        lo = mid + 1;
    }
    if (first_slice(L, lo) > max_slice)
      return fail(SEGATTN_E_RANGE, "segattn_partition_varlen: cannot slice length %lld", (long long)L);
    needed += lo;
    if (needed > 0x7fffffff) return fail(SEGATTN_E_RANGE, "segattn_partition_varlen: too many items");
  }
  // Validate every multi-slice partition (pass 0) before reporting the
  // capacity or writing anything (pass 1): a capacity query then fails the
  // same way the call that writes would.
  std::string scratch;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1 && needed > cap) {
      *n_items = (int32_t)needed;
      return fail(SEGATTN_E_CAPACITY, "segattn_partition_varlen: %lld items needed, capacity %d",
                  (long long)needed, cap);
    }
    int64_t w = 0;
    for (int32_t s = 0; s < nseq; ++s) {
      const int64_t off = cu[s], L = cu[s + 1] - cu[s];
      if (L == 0) continue;
      if (L <= max_slice) {
        if (pass) items[w] = segattn_item{off, 0, L, 0, L};
        ++w;
        continue;
      }
      int64_t lo = 2, hi = L;
      while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (first_slice(L, mid) <= max_slice)
          hi = mid;
        else
          lo = mid + 1;
      }
      scratch.resize(sizeof(int64_t) * (size_t)(lo + 1));
      int64_t *b = reinterpret_cast<int64_t *>(&scratch[0]);
      int rc = partition_into(L, lo, b);
      if (rc) return rc;
      for (int64_t i = 0; i < lo; ++i) {
        if (pass) items[w] = segattn_item{off, b[i], b[i + 1], 0, b[i + 1]};
        ++w;
      }
    }
  }
  *n_items = (int32_t)needed;
  return SEGATTN_OK;
}

extern "C" int segattn_ring_items(const int64_t *bounds, int32_t N, int64_t block, segattn_item *items,
                                  int32_t cap, int32_t *n_items) {
  clear_error();
  if (!bounds || !n_items) return fail(SEGATTN_E_INVALID, "segattn_ring_items: NULL pointer");
  if (N < 1) return fail(SEGATTN_E_INVALID, "segattn_ring_items: N = %d < 1", N);
  if (block < 1) return fail(SEGATTN_E_INVALID, "segattn_ring_items: block < 1");
  if (cap < 0 || (cap > 0 && !items)) return fail(SEGATTN_E_INVALID, "segattn_ring_items: bad items/cap");
  if (bounds[0] != 0) return fail(SEGATTN_E_INVALID, "segattn_ring_items: bounds[0] != 0");
  for (int32_t i = 0; i < N; ++i)
    if (bounds[i + 1] <= bounds[i])
      return fail(SEGATTN_E_INVALID, "segattn_ring_items: bounds not strictly increasing at %d", i);
  if (bounds[N] > kMaxTokens) return fail(SEGATTN_E_RANGE, "segattn_ring_items: > 2^31-1 tokens");
  int64_t needed = 0;
  for (int32_t i = 0; i < N; ++i) needed += (bounds[i + 1] + block - 1) / block;
  if (needed > 0x7fffffff) return fail(SEGATTN_E_RANGE, "segattn_ring_items: too many items");
  if (needed > cap) {
    *n_items = (int32_t)needed;
    return fail(SEGATTN_E_CAPACITY, "segattn_ring_items: %lld items needed, capacity %d",
                (long long)needed, cap);
  }
  int64_t w = 0;
  for (int32_t i = 0; i < N; ++i) {
    const int64_t lo = bounds[i], hi = bounds[i + 1];
    for (int64_t j = (hi + block - 1) / block - 1; j >= 0; --j) {
      const int64_t klo = j * block, khi = (j + 1) * block < hi ? (j + 1) * block : hi;
      items[w++] = segattn_item{0, lo, hi, klo, khi};
    }
  }
  *n_items = (int32_t)needed;
  return SEGATTN_OK;
}

// Offload plan: SPPO section 5.2 (sequence-aware offloading).  Every stage
// moves the same volume, alpha_i A_i = threshold, so that the transfer takes
// as long as one balanced computation step; the GPU memory after stage i is
// M_i = M_{i-1} + A_i - alpha_{i-1} A_{i-1}.  The double operations below are
// kept separate and uncontracted so their rounding is fixed.
#pragma clang fp contract(off)
extern "C" int segattn_offload_plan(const int64_t *rows, const int64_t *row_bytes, int32_t n,
                                    double threshold_bytes, double *alpha, int64_t *rows_moved,
                                    double *mem_bytes, double *peak_bytes) {
  segattn::clear_error();
  using segattn::fail;
  if (!rows || !row_bytes || !alpha || !rows_moved || !mem_bytes)
    return fail(SEGATTN_E_INVALID, "segattn_offload_plan: NULL array");
  if (n < 1) return fail(SEGATTN_E_INVALID, "segattn_offload_plan: n = %d < 1", n);
  if (!(threshold_bytes > 0.0) || !(threshold_bytes < 1e308))
    return fail(SEGATTN_E_INVALID, "segattn_offload_plan: threshold must be finite and > 0");
  for (int32_t i = 0; i < n; ++i) {
    if (rows[i] < 0 || row_bytes[i] < 0)
      return fail(SEGATTN_E_INVALID, "segattn_offload_plan: negative size at %d", i);
    if (row_bytes[i] > 0 && rows[i] > INT64_MAX / row_bytes[i])
      return fail(SEGATTN_E_INVALID, "segattn_offload_plan: rows * row_bytes overflows at %d", i);
  }
  double m = 0.0, peak = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    const double a = (double)(rows[i] * row_bytes[i]);
    double r = 0.0;
    if (a != 0.0) {
      r = threshold_bytes / a;
      if (r > 1.0) r = 1.0;
    }
    alpha[i] = r;
    const double moved_rows = r * (double)rows[i];
    int64_t k = (int64_t)moved_rows;  // floor: moved_rows >= 0
    if (k > rows[i]) k = rows[i];
    rows_moved[i] = k;
    if (i == 0) {
      m = a;
    } else {
      const double moved = alpha[i - 1] * (double)(rows[i - 1] * row_bytes[i - 1]);
      m = m + a;
      m = m - moved;
    }
    mem_bytes[i] = m;
    if (i == 0 || m > peak) peak = m;
  }
  if (peak_bytes) *peak_bytes = peak;
  return SEGATTN_OK;
}
#pragma clang fp contract(on)

extern "C" const char *segattn_status_string(int status) {
  switch (status) {
    case SEGATTN_OK: return "SEGATTN_OK";
    case SEGATTN_E_INVALID: return "SEGATTN_E_INVALID";
    case SEGATTN_E_UNSUPPORTED: return "SEGATTN_E_UNSUPPORTED";
    case SEGATTN_E_RANGE: return "SEGATTN_E_RANGE";
    case SEGATTN_E_CAPACITY: return "SEGATTN_E_CAPACITY";
    case SEGATTN_E_WORKSPACE: return "SEGATTN_E_WORKSPACE";
    case SEGATTN_E_DEVICE: return "SEGATTN_E_DEVICE";
    default: return "SEGATTN_E_UNKNOWN";
  }
}

extern "C" const char *segattn_last_error(void) { return segattn::last_error(); }

extern "C" const char *segattn_version(void) { return "segattn 0.1.0 (gfx950)"; }

// C-ABI entry points of the attention path: argument validation (all of it
// on the host, before anything is launched), work-table construction, the
// table upload into the caller's workspace, and the kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <queue>
#include <vector>

#include "kernels.h"
#include "segattn.h"
#include "status.h"

using namespace segattn;

namespace {

constexpr int64_t kMaxTokens = 0x7fffffffLL;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptr(const void *p, const char *fn, const char *name) {
  if (!p) return fail(SEGATTN_E_INVALID, "%s: %s is NULL", fn, name);
  if (!aligned16(p)) return fail(SEGATTN_E_INVALID, "%s: %s is not 16-byte aligned", fn, name);
  return SEGATTN_OK;
}

int check_shape(const segattn_shape *s, const char *fn) {
  if (!s) return fail(SEGATTN_E_INVALID, "%s: shape is NULL", fn);
  if (s->tokens < 1 || s->tokens > kMaxTokens)
    return fail(SEGATTN_E_RANGE, "%s: tokens = %lld outside [1, 2^31-1]", fn, (long long)s->tokens);
  if (s->hq < 1 || s->hkv < 1) return fail(SEGATTN_E_INVALID, "%s: hq, hkv must be >= 1", fn);
  if (s->hq % s->hkv) return fail(SEGATTN_E_UNSUPPORTED, "%s: hq %% hkv != 0 (%d, %d)", fn, s->hq, s->hkv);
  if (s->d != 64 && s->d != 128) return fail(SEGATTN_E_UNSUPPORTED, "%s: d = %d not in {64, 128}", fn, s->d);
  if (s->in_dtype != SEGATTN_BF16 && s->in_dtype != SEGATTN_F32)
    return fail(SEGATTN_E_INVALID, "%s: in_dtype %d unknown", fn, s->in_dtype);
  if (!(std::isfinite(s->scale) && s->scale > 0.f)) return fail(SEGATTN_E_INVALID, "%s: scale must be finite and > 0", fn);
  // Element offsets are 64-bit in the kernels; rows times heads must stay
  // within int64 comfortably (always true below 2^31 tokens and 2^16 heads).
  if (s->hq > 65536 || s->hkv > 65536) return fail(SEGATTN_E_RANGE, "%s: too many heads", fn);
  return SEGATTN_OK;
}

// Per-item ranges.  Sequence-local indices must fit int32 once offset.
int check_items(const segattn_shape *s, const segattn_item *items, int32_t n, const char *fn) {
  if (!items) return fail(SEGATTN_E_INVALID, "%s: items is NULL", fn);
  if (n < 1) return fail(SEGATTN_E_INVALID, "%s: n_items = %d < 1", fn, n);
  for (int32_t i = 0; i < n; ++i) {
    const segattn_item &it = items[i];
    if (it.seq_off < 0 || it.q_lo < 0 || it.k_lo < 0)
      return fail(SEGATTN_E_RANGE, "%s: item %d has a negative index", fn, i);
    if (it.q_hi <= it.q_lo) return fail(SEGATTN_E_RANGE, "%s: item %d has an empty query range", fn, i);
    if (it.k_hi <= it.k_lo) return fail(SEGATTN_E_RANGE, "%s: item %d has an empty key range", fn, i);
    if (it.k_hi > it.q_hi)
      return fail(SEGATTN_E_RANGE, "%s: item %d: k_hi %lld > q_hi %lld (keys no query of the item can see)", fn, i,
                  (long long)it.k_hi, (long long)it.q_hi);
    if (it.seq_off > s->tokens || it.q_hi > s->tokens - it.seq_off)
      return fail(SEGATTN_E_RANGE, "%s: item %d reaches beyond tokens = %lld", fn, i, (long long)s->tokens);
  }
  return SEGATTN_OK;
}

struct Range {
  int64_t lo, hi;  // global, half-open
  int32_t idx;
};

// Forward items must have pairwise disjoint global query ranges.
int check_disjoint_q(const segattn_item *items, int32_t n, const char *fn) {
  std::vector<Range> r(n);
  for (int32_t i = 0; i < n; ++i) r[i] = {items[i].seq_off + items[i].q_lo, items[i].seq_off + items[i].q_hi, i};
  std::sort(r.begin(), r.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
  for (int32_t i = 1; i < n; ++i)
    if (r[i].lo < r[i - 1].hi)
      return fail(SEGATTN_E_INVALID, "%s: items %d and %d have overlapping query rows", fn, r[i - 1].idx, r[i].idx);
  return SEGATTN_OK;
}

int device_error(hipError_t e, const char *fn) {
  return fail(SEGATTN_E_DEVICE, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
}

// ------------------------------------------------------------ forward table
// Items sorted by the cost of their heaviest work unit (keys visible to the
// last row of a query tile, divided among its key pieces), heaviest first;
// each item's tiles run from its last rows to its first, so the whole unit
// order is heaviest-first for a single sequence.
//
// Key pieces (SEGATTN_SPLIT_KEYS): the key tiles of each query tile of an
// item are cut into P contiguous pieces, one workgroup each, whose partials
// (O, LSE) a second kernel on the stream combines with the log-sum-exp
// merge.  (Combining them inside the forward -- the last piece to finish,
// found with an atomic ticket -- needed device-scope fences, which write
// back and invalidate L2 across the XCDs: 6-12 us per launch, more than the
// split saved.)
//
// P is chosen per launch from a longest-first schedule of its work units on
// the GPU (kSlots workgroups at a time: one forward workgroup per CU), in
// 64-key tile steps: a workgroup costs its key tiles plus kUnitOverhead,
// and a split launch adds kMergeOverhead for the merge kernel (from the
// small-launch kernel trace: about 4 us per workgroup, 0.8 us per key tile,
// 2 us for the merge).  Candidates are P = 1, 2, 3, 4, 6, 8, capped per item
// so that a piece keeps at least kMinPieceTiles key tiles, and limited to
// kSplitMaxPartialBytes of partials; the least makespan wins (ties to fewer
// pieces).  Launches of kSplitGrid or more units are never split: they fill
// the GPU many times over.
constexpr int64_t kSlots = 256;
constexpr int64_t kSplitGrid = 4 * kSlots;
constexpr int64_t kMinPieceTiles = 2;
constexpr int64_t kMaxPieces = kFwdMaxPieces;
constexpr int64_t kUnitOverhead = 5;
constexpr int64_t kMergeOverhead = 3;
constexpr int64_t kSplitMaxPartialBytes = int64_t(512) << 20;

struct FwdPlan {
  std::vector<int32_t> words;
  std::vector<int32_t> split_tiles;  // kSplitTileWords per split query tile
  int32_t n_units = 0;
  int64_t n_parts = 0;  // partial results of split query tiles (per head)
};

int64_t fwd_tiles(const segattn_item &it) { return (it.q_hi - it.q_lo + kFwdBM - 1) / kFwdBM; }
int64_t fwd_key_tiles(const segattn_item &it) {
  return (std::min(it.k_hi, it.q_hi) - it.k_lo + kFwdBN - 1) / kFwdBN;
}
// Key tiles of query tile t of an item (t = 0: its last rows).
int64_t fwd_unit_key_tiles(const segattn_item &it, int64_t t) {
  const int64_t ke = std::min(it.k_hi, it.q_hi - t * kFwdBM);
  return ke > it.k_lo ? (ke - it.k_lo + kFwdBN - 1) / kFwdBN : 0;
}

// Longest-first list schedule of `costs` on kSlots workgroup slots.
int64_t lpt_makespan(std::vector<int64_t> costs) {
  std::sort(costs.begin(), costs.end(), std::greater<int64_t>());
  std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> load;
  for (int64_t i = 0; i < kSlots; ++i) load.push(0);
  int64_t span = 0;
  for (int64_t c : costs) {
    const int64_t l = load.top() + c;
    load.pop();
    load.push(l);
    span = std::max(span, l);
  }
  return span;
}

// Pieces per item (all 1 unless a split applies).
std::vector<int64_t> fwd_pieces(const segattn_item *items, int32_t n, int32_t hq, int32_t d, bool split) {
  std::vector<int64_t> best(n, 1);
  int64_t grid = 0;
  for (int32_t i = 0; i < n; ++i) grid += fwd_tiles(items[i]) * hq;
  if (!split || grid >= kSplitGrid) return best;
  auto makespan = [&](const std::vector<int64_t> &P, int64_t *parts) {
    std::vector<int64_t> costs;
    *parts = 0;
    for (int32_t i = 0; i < n; ++i)
      for (int64_t t = 0; t < fwd_tiles(items[i]); ++t) {
        const int64_t c = fwd_unit_key_tiles(items[i], t);
        for (int64_t p = 0; p < P[i]; ++p) {
          const int64_t cp = (p + 1) * c / P[i] - p * c / P[i] + kUnitOverhead;
          for (int32_t h = 0; h < hq; ++h) costs.push_back(cp);
        }
        if (P[i] > 1) *parts += P[i];
      }
    return lpt_makespan(costs) + (*parts ? kMergeOverhead : 0);
  };
  int64_t parts = 0;
  int64_t best_span = makespan(best, &parts);
  for (int64_t pc : {2, 3, 4, 6, 8}) {
    if (pc > kMaxPieces) break;
    std::vector<int64_t> P(n);
    for (int32_t i = 0; i < n; ++i) P[i] = std::max<int64_t>(1, std::min(pc, fwd_key_tiles(items[i]) / kMinPieceTiles));
    const int64_t span = makespan(P, &parts);
    if ((int64_t)hq * parts * kFwdBM * (d + 1) * 4 > kSplitMaxPartialBytes) continue;
    if (span < best_span) {
      best_span = span;
      best = P;
    }
  }
  return best;
}

void build_fwd_plan(const segattn_item *items, int32_t n, int32_t hq, int32_t d, bool split, FwdPlan &p) {
  const std::vector<int64_t> P = fwd_pieces(items, n, hq, d, split);
  std::vector<int32_t> order(n);
  for (int32_t i = 0; i < n; ++i) order[i] = i;
  auto cost = [&](int32_t i) { return (fwd_key_tiles(items[i]) + P[i] - 1) / P[i]; };
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return cost(a) > cost(b); });
  p.words.assign((size_t)n * kItemWords, 0);
  int64_t unit = 0, part = 0;
  for (int32_t r = 0; r < n; ++r) {
    const segattn_item &it = items[order[r]];
    int32_t *w = &p.words[(size_t)r * kItemWords];
    w[0] = (int32_t)it.seq_off;
    w[1] = (int32_t)it.q_lo;
    w[2] = (int32_t)it.q_hi;
    w[3] = (int32_t)it.k_lo;
    w[4] = (int32_t)it.k_hi;
    w[5] = (int32_t)unit;
    w[6] = (int32_t)P[order[r]];
    w[7] = (int32_t)(P[order[r]] > 1 ? part : 0);
    unit += fwd_tiles(it) * P[order[r]];
    if (P[order[r]] > 1) {
      for (int64_t t = 0; t < fwd_tiles(it); ++t) {  // query tile t: rows [r0, r1), last rows first
        const int64_t r1 = it.q_hi - t * kFwdBM, r0 = std::max(it.q_lo, r1 - kFwdBM);
        p.split_tiles.insert(p.split_tiles.end(), {(int32_t)it.seq_off, (int32_t)r0, (int32_t)r1,
                                                   (int32_t)P[order[r]], (int32_t)(part + t * P[order[r]])});
      }
      part += fwd_tiles(it) * P[order[r]];
    }
  }
  p.n_units = (int32_t)unit;
  p.n_parts = part;
}

// Workspace: the item table and the split-tile table (one upload), then
// (split plans only) the partial LSEs [part][head][kFwdBM] and the partial
// O [part][head][kFwdBM][d] (fp32).
struct FwdLayout {
  size_t split_tiles = 0, part_lse = 0, part_o = 0, bytes = 0;
};

FwdLayout fwd_layout(int32_t n, const FwdPlan &p, int32_t hq, int32_t d) {
  FwdLayout L;
  L.split_tiles = (size_t)n * kItemWords * sizeof(int32_t);
  const size_t np = (size_t)p.n_parts * hq;
  L.part_lse = align_up(L.split_tiles + p.split_tiles.size() * sizeof(int32_t));
  L.part_o = align_up(L.part_lse + np * kFwdBM * sizeof(float));
  L.bytes = p.n_parts ? align_up(L.part_o + np * kFwdBM * (size_t)d * sizeof(float)) : align_up(L.split_tiles);
  return L;
}

// ----------------------------------------------------------- backward table
struct BwdPlan {
  std::vector<int32_t> items, kvg, qg;
  int32_t n_kv_units = 0, n_q_units = 0;
  // longest walk of each role in tile steps: a dQ workgroup's 64-key tiles,
  // a dK/dV workgroup's 64-row tiles per query head of its group
  int64_t kv_walk = 0, q_walk = 0;
};

int build_bwd_plan(const segattn_item *items, int32_t n, BwdPlan &p, const char *fn) {
  // q groups: runs of adjacent items with identical query ranges.
  struct QG {
    int32_t first, count;
    int64_t lo, hi;  // global rows
    int64_t cost;
  };
  std::vector<QG> qgs;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t lo = items[i].seq_off + items[i].q_lo, hi = items[i].seq_off + items[i].q_hi;
    if (!qgs.empty() && qgs.back().lo == lo && qgs.back().hi == hi &&
        items[qgs.back().first].seq_off == items[i].seq_off) {
      qgs.back().count++;
    } else {
      qgs.push_back({i, 1, lo, hi, 0});
    }
  }
  {
    std::vector<Range> r(qgs.size());
    for (size_t i = 0; i < qgs.size(); ++i) r[i] = {qgs[i].lo, qgs[i].hi, qgs[i].first};
    std::sort(r.begin(), r.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
    for (size_t i = 1; i < r.size(); ++i)
      if (r[i].lo < r[i - 1].hi)
        return fail(SEGATTN_E_INVALID,
                    "%s: items %d and %d overlap in query rows without being adjacent items of one query range", fn,
                    r[i - 1].idx, r[i].idx);
  }
  // kv groups: per sequence, the union of the items' key ranges as disjoint
  // intervals (rows outside every key range are never written).
  struct KG {
    int64_t seq_off, kb, ke, qmax;
  };
  std::vector<KG> kgs;
  {
    std::vector<int32_t> idx(n);
    for (int32_t i = 0; i < n; ++i) idx[i] = i;
    std::sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) {
      if (items[a].seq_off != items[b].seq_off) return items[a].seq_off < items[b].seq_off;
      return items[a].k_lo < items[b].k_lo;
    });
    for (int32_t t = 0; t < n; ++t) {
      const segattn_item &it = items[idx[t]];
      if (!kgs.empty() && kgs.back().seq_off == it.seq_off && it.k_lo <= kgs.back().ke) {
        kgs.back().ke = std::max(kgs.back().ke, it.k_hi);
        kgs.back().qmax = std::max(kgs.back().qmax, it.q_hi);
      } else {
        kgs.push_back({it.seq_off, it.k_lo, it.k_hi, it.q_hi});
      }
    }
    // A key interval of one sequence also bounds the query rows that matter
    // to it: the latest q_hi among the sequence's items.
    for (auto &g : kgs) {
      int64_t qm = 0;
      for (int32_t i = 0; i < n; ++i)
        if (items[i].seq_off == g.seq_off) qm = std::max(qm, items[i].q_hi);
      g.qmax = qm;
    }
  }
  // Heaviest work first: kv groups by the rows that can see their first key,
  // q groups by the keys visible to their last row.
  std::stable_sort(kgs.begin(), kgs.end(), [](const KG &a, const KG &b) { return a.qmax - a.kb > b.qmax - b.kb; });
  for (auto &q : qgs) {
    int64_t c = 0;
    for (int32_t i = q.first; i < q.first + q.count; ++i) c += std::min(items[i].k_hi, items[i].q_hi) - items[i].k_lo;
    q.cost = c;
  }
  std::stable_sort(qgs.begin(), qgs.end(), [](const QG &a, const QG &b) { return a.cost > b.cost; });

  p.items.assign((size_t)n * kItemWords, 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t *w = &p.items[(size_t)i * kItemWords];
    w[0] = (int32_t)items[i].seq_off;
    w[1] = (int32_t)items[i].q_lo;
    w[2] = (int32_t)items[i].q_hi;
    w[3] = (int32_t)items[i].k_lo;
    w[4] = (int32_t)items[i].k_hi;
  }
  p.kvg.clear();
  int64_t u = 0;
  for (auto &g : kgs) {
    p.kvg.insert(p.kvg.end(), {(int32_t)g.seq_off, (int32_t)g.kb, (int32_t)g.ke, (int32_t)u});
    u += (g.ke - g.kb + kBwdKvBN - 1) / kBwdKvBN;
  }
  p.n_kv_units = (int32_t)u;
  // a dK/dV workgroup walks, per query head of its group, the 64-row tiles
  // of every item that sees its keys; the first key tile of a group sees
  // the most
  for (auto &g : kgs) {
    int64_t walk = 0;
    for (int32_t i = 0; i < n; ++i) {
      const segattn_item &it = items[i];
      if (it.seq_off == g.seq_off && it.k_lo < g.kb + kBwdKvBN && it.k_hi > g.kb && it.q_hi > g.kb)
        walk += (it.q_hi - std::max(it.q_lo, g.kb) + kBwdKvBM - 1) / kBwdKvBM;
    }
    p.kv_walk = std::max(p.kv_walk, walk);
  }
  p.qg.clear();
  u = 0;
  for (auto &q : qgs) {
    p.qg.insert(p.qg.end(), {q.first, q.count, (int32_t)u, 0});
    u += (q.hi - q.lo + kBwdQBM - 1) / kBwdQBM;
  }
  p.n_q_units = (int32_t)u;
  for (auto &q : qgs) p.q_walk = std::max(p.q_walk, (q.cost + kBwdQBN - 1) / kBwdQBN);
  return SEGATTN_OK;
}

size_t bwd_delta_bytes(const segattn_shape *s) { return align_up((size_t)s->hq * (size_t)s->tokens * sizeof(float)); }

size_t bwd_ws_bytes(const segattn_shape *s, const BwdPlan &p) {
  return bwd_delta_bytes(s) + align_up(p.items.size() * 4) + align_up(p.kvg.size() * 4) + align_up(p.qg.size() * 4);
}

// Device copies of the plan tables, after D in the workspace.
struct BwdTables {
  int32_t *items, *kvg, *qg;
};

// Places the three tables in the workspace and uploads them (one
// stream-ordered upload; they are contiguous).
hipError_t upload_bwd_tables(const segattn_shape *shape, const BwdPlan &plan, void *workspace, hipStream_t s,
                             BwdTables &t) {
  char *ws = static_cast<char *>(workspace);
  size_t off = bwd_delta_bytes(shape);
  t.items = reinterpret_cast<int32_t *>(ws + off);
  off += align_up(plan.items.size() * 4);
  t.kvg = reinterpret_cast<int32_t *>(ws + off);
  off += align_up(plan.kvg.size() * 4);
  t.qg = reinterpret_cast<int32_t *>(ws + off);
  std::vector<int32_t> words((size_t)(t.qg - t.items) + plan.qg.size(), 0);
  std::copy(plan.items.begin(), plan.items.end(), words.begin());
  std::copy(plan.kvg.begin(), plan.kvg.end(), words.begin() + (t.kvg - t.items));
  std::copy(plan.qg.begin(), plan.qg.end(), words.begin() + (t.qg - t.items));
  return launch_upload(t.items, words.data(), (int64_t)words.size(), s);
}

PreArgs pre_args(const segattn_shape *shape, const BwdPlan &plan, const void *o, const void *d_o, float *delta,
                 const BwdTables &t) {
  return PreArgs{o, d_o, delta, t.items, t.qg, (int32_t)(plan.qg.size() / 4), plan.n_q_units, shape->tokens,
                 shape->hq};
}

}  // namespace

// ================================================================== forward

extern "C" int segattn_fwd_workspace(const segattn_shape *shape, const segattn_item *items, int32_t n_items,
                                     size_t *bytes) {
  clear_error();
  static const char *fn = "segattn_fwd_workspace";
  if (!bytes) return fail(SEGATTN_E_INVALID, "%s: bytes is NULL", fn);
  if (int rc = check_shape(shape, fn)) return rc;
  if (int rc = check_items(shape, items, n_items, fn)) return rc;
  // enough for the call with or without SEGATTN_SPLIT_KEYS
  FwdPlan plan;
  build_fwd_plan(items, n_items, shape->hq, shape->d, true, plan);
  *bytes = fwd_layout(n_items, plan, shape->hq, shape->d).bytes;
  return SEGATTN_OK;
}

extern "C" int segattn_fwd(const segattn_shape *shape, const void *q, const void *k, const void *v,
                           const segattn_item *items, int32_t n_items, void *o, int32_t o_dtype, float *lse,
                           uint32_t flags, void *workspace, size_t ws_bytes, void *stream) {
  clear_error();
  static const char *fn = "segattn_fwd";
  if (int rc = check_shape(shape, fn)) return rc;
  if (int rc = check_ptr(q, fn, "q")) return rc;
  if (int rc = check_ptr(k, fn, "k")) return rc;
  if (int rc = check_ptr(v, fn, "v")) return rc;
  if (int rc = check_ptr(o, fn, "o")) return rc;
  if (int rc = check_ptr(lse, fn, "lse")) return rc;
  if (o_dtype != SEGATTN_BF16 && o_dtype != SEGATTN_F32) return fail(SEGATTN_E_INVALID, "%s: o_dtype %d unknown", fn, o_dtype);
  if (flags & ~(SEGATTN_MERGE_INTO | SEGATTN_SPLIT_KEYS)) return fail(SEGATTN_E_INVALID, "%s: unknown flags 0x%x", fn, flags);
  if ((flags & SEGATTN_MERGE_INTO) && o_dtype != SEGATTN_F32)
    return fail(SEGATTN_E_INVALID, "%s: SEGATTN_MERGE_INTO needs an fp32 output", fn);
  if (int rc = check_items(shape, items, n_items, fn)) return rc;
  if (int rc = check_disjoint_q(items, n_items, fn)) return rc;
  FwdPlan plan;
  build_fwd_plan(items, n_items, shape->hq, shape->d, (flags & SEGATTN_SPLIT_KEYS) != 0, plan);
  const FwdLayout lay = fwd_layout(n_items, plan, shape->hq, shape->d);
  const size_t need = lay.bytes;
  if (!workspace || ws_bytes < need)
    return fail(SEGATTN_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? ws_bytes : 0);
  if (!aligned16(workspace)) return fail(SEGATTN_E_INVALID, "%s: workspace is not 16-byte aligned", fn);

  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  int32_t *table = reinterpret_cast<int32_t *>(ws);
  const int32_t n_split = (int32_t)(plan.split_tiles.size() / kSplitTileWords);
  // Small tables travel in the kernel arguments; larger ones (the item
  // table, then the split-tile table) are uploaded into the workspace.
  const bool inline_tables = n_items <= kInlineItems && n_split <= kInlineSplitTiles;
  if (!inline_tables) {
    std::vector<int32_t> words = plan.words;
    words.insert(words.end(), plan.split_tiles.begin(), plan.split_tiles.end());
    if (hipError_t e = launch_upload(table, words.data(), (int64_t)words.size(), s)) return device_error(e, fn);
  }

  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.items = inline_tables ? nullptr : table;
  if (inline_tables) std::copy(plan.words.begin(), plan.words.end(), a.inline_items);
  a.n_items = n_items;
  a.n_units = plan.n_units;
  a.tokens = shape->tokens;
  a.hq = shape->hq;
  a.hkv = shape->hkv;
  a.scale_log2 = shape->scale * 1.4426950408889634f;
  a.merge = (flags & SEGATTN_MERGE_INTO) ? 1 : 0;
  a.part_lse = plan.n_parts ? reinterpret_cast<float *>(ws + lay.part_lse) : nullptr;
  a.part_o = plan.n_parts ? reinterpret_cast<float *>(ws + lay.part_o) : nullptr;
  SplitMergeArgs m{};
  m.tiles = inline_tables ? nullptr : reinterpret_cast<const int32_t *>(ws + lay.split_tiles);
  if (inline_tables) std::copy(plan.split_tiles.begin(), plan.split_tiles.end(), m.inline_tiles);
  m.n_tiles = n_split;
  m.hq = shape->hq;
  m.tokens = shape->tokens;
  m.part_lse = a.part_lse;
  m.part_o = a.part_o;
  m.o = o;
  m.lse = lse;
  m.merge = a.merge;
  if ((int64_t)a.n_units * a.hq > 0x7fffffffLL) return fail(SEGATTN_E_RANGE, "%s: grid too large", fn);
  if (hipError_t e = launch_fwd(a, m, shape->d, shape->in_dtype, o_dtype, s)) return device_error(e, fn);
  return SEGATTN_OK;
}

// ==================================================================== merge

extern "C" int segattn_merge(int64_t rows, int32_t h, int32_t d, int64_t lse_stride, const float *o_a,
                             const float *lse_a, const float *o_b, const float *lse_b, float *o_out, float *lse_out,
                             void *stream) {
  clear_error();
  static const char *fn = "segattn_merge";
  if (rows < 1 || h < 1 || d < 4 || d % 4) return fail(SEGATTN_E_INVALID, "%s: rows, h >= 1 and d a multiple of 4", fn);
  if (d > 1024) return fail(SEGATTN_E_UNSUPPORTED, "%s: d = %d > 1024", fn, d);
  if (lse_stride < rows) return fail(SEGATTN_E_INVALID, "%s: lse_stride < rows", fn);
  if (rows > (int64_t)1 << 40 || (int64_t)h * lse_stride > (int64_t)1 << 40)
    return fail(SEGATTN_E_RANGE, "%s: sizes too large", fn);
  for (auto pr : {std::make_pair((const void *)o_a, "o_a"), std::make_pair((const void *)o_b, "o_b"),
                  std::make_pair((const void *)o_out, "o_out")})
    if (int rc = check_ptr(pr.first, fn, pr.second)) return rc;
  if (!lse_a || !lse_b || !lse_out) return fail(SEGATTN_E_INVALID, "%s: lse pointer is NULL", fn);
  if (((uintptr_t)lse_a | (uintptr_t)lse_b | (uintptr_t)lse_out) & 3u)
    return fail(SEGATTN_E_INVALID, "%s: lse pointers must be 4-byte aligned", fn);
  MergeArgs a{rows, h, d, lse_stride, o_a, lse_a, o_b, lse_b, o_out, lse_out};
  if (hipError_t e = launch_merge(a, static_cast<hipStream_t>(stream))) return device_error(e, fn);
  return SEGATTN_OK;
}

// ================================================================= backward

extern "C" int segattn_bwd_workspace(const segattn_shape *shape, const segattn_item *items, int32_t n_items,
                                     size_t *bytes) {
  clear_error();
  static const char *fn = "segattn_bwd_workspace";
  if (!bytes) return fail(SEGATTN_E_INVALID, "%s: bytes is NULL", fn);
  if (int rc = check_shape(shape, fn)) return rc;
  if (int rc = check_items(shape, items, n_items, fn)) return rc;
  BwdPlan plan;
  if (int rc = build_bwd_plan(items, n_items, plan, fn)) return rc;
  *bytes = bwd_ws_bytes(shape, plan);
  return SEGATTN_OK;
}

extern "C" int segattn_bwd_preprocess(const segattn_shape *shape, const void *o, int32_t o_dtype, const void *d_o,
                                      const segattn_item *items, int32_t n_items, void *workspace, size_t ws_bytes,
                                      void *stream) {
  clear_error();
  static const char *fn = "segattn_bwd_preprocess";
  if (int rc = check_shape(shape, fn)) return rc;
  if (int rc = check_ptr(o, fn, "o")) return rc;
  if (int rc = check_ptr(d_o, fn, "d_o")) return rc;
  if (o_dtype != SEGATTN_BF16 && o_dtype != SEGATTN_F32) return fail(SEGATTN_E_INVALID, "%s: o_dtype %d unknown", fn, o_dtype);
  if (int rc = check_items(shape, items, n_items, fn)) return rc;
  BwdPlan plan;
  if (int rc = build_bwd_plan(items, n_items, plan, fn)) return rc;
  const size_t need = bwd_ws_bytes(shape, plan);
  if (!workspace || ws_bytes < need)
    return fail(SEGATTN_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? ws_bytes : 0);
  if (!aligned16(workspace)) return fail(SEGATTN_E_INVALID, "%s: workspace is not 16-byte aligned", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  BwdTables t;
  if (hipError_t e = upload_bwd_tables(shape, plan, workspace, s, t)) return device_error(e, fn);
  const PreArgs a = pre_args(shape, plan, o, d_o, static_cast<float *>(workspace), t);
  if (hipError_t e = launch_bwd_pre(a, shape->d, o_dtype, shape->in_dtype, s)) return device_error(e, fn);
  return SEGATTN_OK;
}

namespace {

// Everything segattn_bwd checks except the workspace; builds the plan.
int bwd_check(const char *fn, const segattn_shape *shape, const void *q, const void *k, const void *v,
              const void *o, int32_t o_dtype, const float *lse, const void *d_o, const segattn_item *items,
              int32_t n_items, void *dq, void *dk, void *dv, int32_t g_dtype, uint32_t flags, BwdPlan &plan) {
  if (int rc = check_shape(shape, fn)) return rc;
  const void *ptrs[] = {q, k, v, o, lse, d_o, dq, dk, dv};
  const char *names[] = {"q", "k", "v", "o", "lse", "d_o", "dq", "dk", "dv"};
  for (int i = 0; i < 9; ++i)
    if (int rc = check_ptr(ptrs[i], fn, names[i])) return rc;
  if (o_dtype != SEGATTN_BF16 && o_dtype != SEGATTN_F32) return fail(SEGATTN_E_INVALID, "%s: o_dtype %d unknown", fn, o_dtype);
  if (g_dtype != SEGATTN_BF16 && g_dtype != SEGATTN_F32) return fail(SEGATTN_E_INVALID, "%s: g_dtype %d unknown", fn, g_dtype);
  if (flags & ~(SEGATTN_ACCUMULATE | SEGATTN_D_READY)) return fail(SEGATTN_E_INVALID, "%s: unknown flags 0x%x", fn, flags);
  if ((flags & SEGATTN_ACCUMULATE) && g_dtype != SEGATTN_F32)
    return fail(SEGATTN_E_INVALID, "%s: SEGATTN_ACCUMULATE needs fp32 gradients", fn);
  if (int rc = check_items(shape, items, n_items, fn)) return rc;
  if (int rc = build_bwd_plan(items, n_items, plan, fn)) return rc;
  const int64_t kv_blocks = (int64_t)plan.n_kv_units * shape->hkv;
  const int64_t kv_pad = (kv_blocks + 7) / 8 * 8;
  const int64_t q_blocks = (int64_t)plan.n_q_units * shape->hq;
  if (kv_pad + q_blocks + 8 > 0x7fffffffLL) return fail(SEGATTN_E_RANGE, "%s: grid too large", fn);
  return SEGATTN_OK;
}

// Table upload, D (unless SEGATTN_D_READY) and the backward kernel, with D
// and the tables in `workspace` (at least bwd_ws_bytes(shape, plan) bytes).
int bwd_launch(const char *fn, const segattn_shape *shape, const void *q, const void *k, const void *v,
               const void *o, int32_t o_dtype, const float *lse, const void *d_o, int32_t n_items, void *dq,
               void *dk, void *dv, int32_t g_dtype, uint32_t flags, const BwdPlan &plan, void *workspace,
               hipStream_t s) {
  const int64_t kv_blocks = (int64_t)plan.n_kv_units * shape->hkv;
  const int64_t kv_pad = (kv_blocks + 7) / 8 * 8;
  const int64_t q_blocks = (int64_t)plan.n_q_units * shape->hq;
  const int64_t q_pad = (q_blocks + 7) / 8 * 8;
  float *delta = static_cast<float *>(workspace);
  BwdTables t;
  if (hipError_t e = upload_bwd_tables(shape, plan, workspace, s, t)) return device_error(e, fn);
  if (!(flags & SEGATTN_D_READY)) {
    const PreArgs pa = pre_args(shape, plan, o, d_o, delta, t);
    if (hipError_t e = launch_bwd_pre(pa, shape->d, o_dtype, shape->in_dtype, s)) return device_error(e, fn);
  }
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.d_o = d_o;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.items = t.items;
  a.kvg = t.kvg;
  a.qg = t.qg;
  a.n_items = n_items;
  a.n_kvg = (int32_t)(plan.kvg.size() / 4);
  a.n_qg = (int32_t)(plan.qg.size() / 4);
  a.n_kv_units = plan.n_kv_units;
  a.n_q_units = plan.n_q_units;
  a.kv_blocks = (int32_t)kv_blocks;
  a.kv_pad = (int32_t)kv_pad;
  a.q_blocks = (int32_t)q_blocks;
  a.q_pad = (int32_t)q_pad;
  a.dq_first = plan.q_walk > plan.kv_walk * (shape->hq / shape->hkv) ? 1 : 0;
  a.tokens = shape->tokens;
  a.hq = shape->hq;
  a.hkv = shape->hkv;
  a.scale = shape->scale;
  a.scale_log2 = shape->scale * 1.4426950408889634f;
  a.accumulate = (flags & SEGATTN_ACCUMULATE) ? 1 : 0;
  if (hipError_t e = launch_bwd(a, shape->d, shape->in_dtype, g_dtype, s)) return device_error(e, fn);
  return SEGATTN_OK;
}

}  // namespace

extern "C" int segattn_bwd(const segattn_shape *shape, const void *q, const void *k, const void *v, const void *o,
                           int32_t o_dtype, const float *lse, const void *d_o, const segattn_item *items,
                           int32_t n_items, void *dq, void *dk, void *dv, int32_t g_dtype, uint32_t flags,
                           void *workspace, size_t ws_bytes, void *stream) {
  clear_error();
  static const char *fn = "segattn_bwd";
  BwdPlan plan;
  if (int rc = bwd_check(fn, shape, q, k, v, o, o_dtype, lse, d_o, items, n_items, dq, dk, dv, g_dtype, flags, plan))
    return rc;
  const size_t need = bwd_ws_bytes(shape, plan);
  if (!workspace || ws_bytes < need)
    return fail(SEGATTN_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? ws_bytes : 0);
  if (!aligned16(workspace)) return fail(SEGATTN_E_INVALID, "%s: workspace is not 16-byte aligned", fn);
  return bwd_launch(fn, shape, q, k, v, o, o_dtype, lse, d_o, n_items, dq, dk, dv, g_dtype, flags, plan, workspace,
                    static_cast<hipStream_t>(stream));
}

// ------------------------------------------------- backward, no allocation
// The backward's scratch (D and the plan tables) in the library's own device
// array (noalloc_scratch, misc.hip) instead of a caller's workspace.
namespace {

int scratch_of_current_device(const char *fn, void **out) {
  if (hipError_t e = noalloc_scratch(out)) return device_error(e, fn);
  if (!*out) return fail(SEGATTN_E_DEVICE, "%s: no device address for the scratch array", fn);
  return SEGATTN_OK;
}

}  // namespace

extern "C" int segattn_bwd_noalloc(const segattn_shape *shape, const void *q, const void *k, const void *v,
                                   const void *o, int32_t o_dtype, const float *lse, const void *d_o,
                                   const segattn_item *items, int32_t n_items, void *dq, void *dk, void *dv,
                                   int32_t g_dtype, uint32_t flags, void *stream) {
  clear_error();
  static const char *fn = "segattn_bwd_noalloc";
  if (flags & SEGATTN_D_READY)
    return fail(SEGATTN_E_INVALID, "%s: SEGATTN_D_READY is not available (D lives in the library's scratch)", fn);
  BwdPlan plan;
  if (int rc = bwd_check(fn, shape, q, k, v, o, o_dtype, lse, d_o, items, n_items, dq, dk, dv, g_dtype, flags, plan))
    return rc;
  const size_t need = bwd_ws_bytes(shape, plan);
  if (need > (size_t)SEGATTN_NOALLOC_SCRATCH_BYTES)
    return fail(SEGATTN_E_WORKSPACE,
                "%s: this call needs %zu bytes of scratch; the no-allocation entry point holds %zu "
                "(use segattn_bwd with a workspace)",
                fn, need, (size_t)SEGATTN_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (int rc = scratch_of_current_device(fn, &ws)) return rc;
  return bwd_launch(fn, shape, q, k, v, o, o_dtype, lse, d_o, n_items, dq, dk, dv, g_dtype, flags, plan, ws,
                    static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ offload
// Row copies and stream ordering for moving backward-only activations to
// host memory beside the computation (SPPO sections 5.1-5.2).
extern "C" int segattn_copy_rows(void *dst, int64_t dst_pitch, const void *src, int64_t src_pitch,
                                 int64_t row_bytes, int64_t rows, int32_t kind, void *stream) {
  clear_error();
  static const char *fn = "segattn_copy_rows";
  if (kind != SEGATTN_D2H && kind != SEGATTN_H2D) return fail(SEGATTN_E_INVALID, "%s: bad kind %d", fn, kind);
  if (rows < 0 || row_bytes < 0) return fail(SEGATTN_E_INVALID, "%s: negative size", fn);
  if (rows == 0 || row_bytes == 0) return SEGATTN_OK;
  if (!dst || !src) return fail(SEGATTN_E_INVALID, "%s: NULL pointer", fn);
  if (dst_pitch < row_bytes || src_pitch < row_bytes)
    return fail(SEGATTN_E_INVALID, "%s: pitch smaller than the row", fn);
  const hipMemcpyKind k = kind == SEGATTN_D2H ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  hipError_t e;
  if (rows == 1 || (dst_pitch == row_bytes && src_pitch == row_bytes))
    e = hipMemcpyAsync(dst, src, (size_t)(row_bytes * rows), k, (hipStream_t)stream);
  else
    e = hipMemcpy2DAsync(dst, (size_t)dst_pitch, src, (size_t)src_pitch, (size_t)row_bytes, (size_t)rows, k,
                         (hipStream_t)stream);
  return e == hipSuccess ? SEGATTN_OK : device_error(e, fn);
}

extern "C" int segattn_stream_order(void *event, void *from_stream, void *to_stream) {
  clear_error();
  static const char *fn = "segattn_stream_order";
  if (!event) return fail(SEGATTN_E_INVALID, "%s: NULL event", fn);
  hipError_t e = hipEventRecord((hipEvent_t)event, (hipStream_t)from_stream);
  if (e == hipSuccess) e = hipStreamWaitEvent((hipStream_t)to_stream, (hipEvent_t)event, 0);
  return e == hipSuccess ? SEGATTN_OK : device_error(e, fn);
}

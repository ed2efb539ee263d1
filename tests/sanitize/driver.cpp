// Exercises every host-side entry point of the C ABI -- planners, offload
// plan, workspace queries, argument validation, plan-table construction and
// upload -- with random valid and invalid inputs, for the AddressSanitizer /
// UndefinedBehaviorSanitizer build (tests/test_sanitize_cpu.py).  Device
// pointers are fake (aligned, never dereferenced: the launchers are stubs);
// workspaces are real host memory of exactly the size the library asks for.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "segattn.h"

extern int g_launches;

namespace {

std::mt19937_64 rng(20261202);
int64_t uni(int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); }
void *const F = reinterpret_cast<void *>(0x100000);  // fake 16-byte aligned device pointer
float *const FF = reinterpret_cast<float *>(0x200000);

int fails = 0;
void expect(bool ok, const char *what, long long a = 0, long long b = 0) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s (%lld, %lld): %s\n", what, a, b, segattn_last_error());
    ++fails;
  }
}

struct Batch {
  std::vector<int64_t> cu;
};

Batch random_batch() {
  Batch b;
  b.cu.push_back(0);
  const int nseq = (int)uni(0, 12);
  for (int i = 0; i < nseq; ++i) {
    const int kind = (int)uni(0, 4);
    int64_t L = kind == 0 ? uni(0, 3) : kind == 1 ? uni(1, 300) : kind == 2 ? uni(200, 5000) : uni(4000, 70000);
    b.cu.push_back(b.cu.back() + L);
  }
  return b;
}

std::vector<segattn_item> varlen_items(const Batch &b, int64_t cap_slice, int *rc_out) {
  int32_t n = 0;
  const int nseq = (int)b.cu.size() - 1;
  int rc = segattn_partition_varlen(b.cu.data(), nseq, cap_slice, nullptr, 0, &n);
  std::vector<segattn_item> it;
  if (rc == SEGATTN_E_CAPACITY || (rc == SEGATTN_OK && n > 0)) {
    it.resize(n);
    rc = segattn_partition_varlen(b.cu.data(), nseq, cap_slice, it.data(), n, &n);
    expect(rc == SEGATTN_OK && n == (int32_t)it.size(), "varlen second call", rc, n);
  }
  *rc_out = rc;
  return it;
}

// forward / backward / preprocess / no-alloc / workspace queries on one table
void run_tables(const std::vector<segattn_item> &items, int64_t tokens) {
  if (items.empty() || tokens < 1) return;
  const int32_t hkv = (int32_t)std::vector<int>{1, 2, 4, 8}[uni(0, 3)];
  const int32_t hq = hkv * (int32_t)std::vector<int>{1, 2, 3, 4}[uni(0, 3)];
  segattn_shape s{tokens, hq, hkv, uni(0, 5) ? 128 : 64, (int32_t)uni(0, 1), 0.0883883f};
  const int32_t n = (int32_t)items.size();
  size_t fb = 0, bb = 0;
  const int rf = segattn_fwd_workspace(&s, items.data(), n, &fb);
  const int rb = segattn_bwd_workspace(&s, items.data(), n, &bb);
  if (rf != SEGATTN_OK) return;
  {
    std::vector<char> ws(fb + 256);
    char *w = ws.data() + (256 - (reinterpret_cast<uintptr_t>(ws.data()) & 255)) % 256;
    const int32_t odt = (int32_t)uni(0, 1);
    const uint32_t flags = (odt == 1 && uni(0, 1) ? SEGATTN_MERGE_INTO : 0) | (uni(0, 1) ? SEGATTN_SPLIT_KEYS : 0);
    const int rc = segattn_fwd(&s, F, F, F, items.data(), n, F, odt, FF, flags, w, fb, nullptr);
    expect(rc == SEGATTN_OK || rc == SEGATTN_E_INVALID, "fwd status", rc);
    // the item table alone needs 32 bytes per item
    expect(segattn_fwd(&s, F, F, F, items.data(), n, F, odt, FF, flags, w, 32 * (size_t)n - 4, nullptr) != SEGATTN_OK,
           "fwd short workspace");
  }
  std::vector<segattn_item> rev(items.rbegin(), items.rend());
  size_t rbb = 0;
  if (segattn_bwd_workspace(&s, rev.data(), n, &rbb) != SEGATTN_OK) return;
  (void)rb;
  std::vector<char> ws(rbb + 256);
  char *w = ws.data() + (256 - (reinterpret_cast<uintptr_t>(ws.data()) & 255)) % 256;
  const int32_t gdt = (int32_t)uni(0, 1);
  const uint32_t flags = gdt == 1 && uni(0, 1) ? SEGATTN_ACCUMULATE : 0;
  int rc = segattn_bwd_preprocess(&s, F, 0, F, rev.data(), n, w, rbb, nullptr);
  expect(rc == SEGATTN_OK, "bwd_preprocess", rc);
  rc = segattn_bwd(&s, F, F, F, F, 0, FF, F, rev.data(), n, F, F, F, gdt, flags | (uni(0, 1) ? SEGATTN_D_READY : 0),
                   w, rbb, nullptr);
  expect(rc == SEGATTN_OK, "bwd", rc);
  expect(segattn_bwd(&s, F, F, F, F, 0, FF, F, rev.data(), n, F, F, F, gdt, flags, w, rbb - 1, nullptr) ==
             SEGATTN_E_WORKSPACE,
         "bwd short workspace");
  rc = segattn_bwd_noalloc(&s, F, F, F, F, 0, FF, F, rev.data(), n, F, F, F, gdt, flags, nullptr);
  expect(rc == (rbb <= SEGATTN_NOALLOC_SCRATCH_BYTES ? SEGATTN_OK : SEGATTN_E_WORKSPACE), "bwd_noalloc", rc);
}

}  // namespace

int main() {
  // 1. partition
  for (int t = 0; t < 8000; ++t) {
    const int64_t S = uni(0, 3) ? uni(1, 1 << 21) : uni(-3, 200);
    const int32_t N = (int32_t)(uni(0, 3) ? uni(1, 128) : uni(-2, 400));
    std::vector<int64_t> b((size_t)std::max(N + 1, 1), -7);
    const int rc = segattn_partition(S, N, b.data());
    if (rc == SEGATTN_OK) {
      bool ok = b[0] == 0 && b[N] == S;
      for (int i = 0; i < N; ++i) ok = ok && b[i] < b[i + 1];
      expect(ok, "partition bounds", S, N);
      if (uni(0, 9) == 0) {
        int32_t ni = 0;
        const int64_t block = uni(-1, 5000);
        int r2 = segattn_ring_items(b.data(), N, block, nullptr, 0, &ni);
        if (r2 == SEGATTN_E_CAPACITY || (r2 == SEGATTN_OK && ni > 0)) {
          std::vector<segattn_item> it((size_t)ni);
          r2 = segattn_ring_items(b.data(), N, block, it.data(), ni, &ni);
          expect(r2 == SEGATTN_OK, "ring items", S, N);
          if (S <= 200000 && r2 == SEGATTN_OK) run_tables(it, S);
        }
        std::vector<segattn_item> seg;
        for (int i = 0; i < N; ++i) seg.push_back({0, b[i], b[i + 1], 0, b[i + 1]});
        if (S <= 200000) run_tables(seg, S);
      }
    } else {
      for (int64_t x : b) expect(x == -7, "partition wrote on error", S, N);
    }
  }
  // 2. varlen slicing, chunking, and the attention entry points on their items
  for (int t = 0; t < 1500; ++t) {
    Batch bt = random_batch();
    const int64_t cap = uni(0, 7) ? uni(256, 20000) : uni(-2, 300);
    int rc = 0;
    std::vector<segattn_item> it = varlen_items(bt, cap, &rc);
    if (rc == SEGATTN_OK && !it.empty()) run_tables(it, bt.cu.back());
    const int nseq = (int)bt.cu.size() - 1;
    const int32_t K = (int32_t)uni(-1, 6);
    const double a1 = uni(0, 5) ? std::ldexp((double)uni(1, 1000), -30) : -1.0, a2 = uni(0, 1) ? 1e-5 : 0.0;
    const int64_t tcap = uni(-1, 40000);
    int32_t ni = 0, nc = 0;
    double tt = 0;
    int r2 = segattn_chunk_varlen(bt.cu.data(), nseq, K, a1, a2, tcap, nullptr, nullptr, 0, &ni, &nc, &tt);
    if (r2 == SEGATTN_E_CAPACITY || (r2 == SEGATTN_OK && ni > 0)) {
      std::vector<segattn_item> ci((size_t)ni);
      std::vector<int32_t> owner((size_t)ni);
      r2 = segattn_chunk_varlen(bt.cu.data(), nseq, K, a1, a2, tcap, ci.data(), owner.data(), ni, &ni, &nc, &tt);
      expect(r2 == SEGATTN_OK, "chunk second call", r2);
      for (int c = 0; r2 == SEGATTN_OK && c < nc && c < 4; ++c) {
        std::vector<segattn_item> ch;
        for (int i = 0; i < ni; ++i)
          if (owner[i] == c) ch.push_back(ci[i]);
        run_tables(ch, bt.cu.back());
      }
    }
    // junk item tables: validation must reject them without reading past n
    std::vector<segattn_item> junk((size_t)uni(1, 6));
    for (auto &j : junk) j = {uni(-2, 50), uni(-2, 60), uni(-2, 80), uni(-2, 60), uni(-2, 80)};
    run_tables(junk, uni(1, 100));
  }
  // 3. offload plan
  for (int t = 0; t < 5000; ++t) {
    const int32_t n = (int32_t)uni(-1, 70);
    std::vector<int64_t> rows((size_t)std::max(n, 1)), rb((size_t)std::max(n, 1));
    for (auto &r : rows) r = uni(-1, 40000);
    for (auto &r : rb) r = uni(-1, 20000);
    std::vector<double> alpha(rows.size()), mem(rows.size());
    std::vector<int64_t> moved(rows.size());
    double peak = 0;
    segattn_offload_plan(rows.data(), rb.data(), n, uni(0, 3) ? (double)uni(0, 1 << 30) : -1.0, alpha.data(),
                         moved.data(), mem.data(), &peak);
  }
  // 4. merge, copies, stream ordering
  for (int t = 0; t < 2000; ++t) {
    segattn_merge(uni(-1, 1 << 20), (int32_t)uni(-1, 64), (int32_t)uni(-4, 1100), uni(-1, 1 << 20), FF, FF, FF, FF,
                  FF, FF, nullptr);
    segattn_copy_rows(F, uni(-1, 4096), F, uni(-1, 4096), uni(-1, 4096), uni(-1, 100), (int32_t)uni(-1, 2), nullptr);
  }
  segattn_stream_order(nullptr, nullptr, nullptr);
  for (int st = -1; st < 9; ++st) segattn_status_string(st);
  std::printf("sanitized driver: %d stub launches, %d failures\n", g_launches, fails);
  return fails ? 1 : 0;
}

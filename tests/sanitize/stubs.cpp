// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// of the host layer (api.cpp), for the sanitizer build of the planners and
// the C ABI.  Nothing here touches a device.  The table upload copies its
// words into the destination, which the driver points at real host memory
// of exactly the workspace size the library asked for, so AddressSanitizer
// checks the workspace layout; the launchers check their arguments against
// the tables the same way the kernels index them.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.h"
#include "segattn.h"

namespace {
void require(bool ok, const char *what) {
  if (!ok) {
    std::fprintf(stderr, "stub check failed: %s\n", what);
    std::abort();
  }
}
char g_scratch_host[SEGATTN_NOALLOC_SCRATCH_BYTES] __attribute__((aligned(256)));
}  // namespace

int g_launches = 0;

extern "C" {
const char *hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t) { return hipSuccess; }
hipError_t hipMemcpy2DAsync(void *, size_t, const void *, size_t, size_t, size_t, hipMemcpyKind, hipStream_t) {
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
}

namespace segattn {

hipError_t launch_upload(int32_t *dst, const int32_t *words, int64_t n, hipStream_t) {
  require(n > 0 && dst && words, "upload arguments");
  std::memcpy(dst, words, (size_t)n * sizeof(int32_t));  // ASan: both ranges must be whole
  return hipSuccess;
}

hipError_t launch_fwd(const FwdArgs &a, const SplitMergeArgs &m, int d, int in_dtype, int o_dtype, hipStream_t) {
  require(d == 64 || d == 128, "fwd d");
  require(in_dtype == 0 || in_dtype == 1, "fwd in_dtype");
  require(o_dtype == 0 || o_dtype == 1, "fwd o_dtype");
  require(a.n_items >= 1 && a.n_units >= 1, "fwd sizes");
  const int32_t *items = a.items ? a.items : a.inline_items;
  require(a.items || a.n_items <= kInlineItems, "inline item table size");
  // units: item i owns [unit_begin_i, unit_begin_{i+1}), ascending from 0
  int32_t prev = -1;
  int64_t split_tiles = 0;
  for (int i = 0; i < a.n_items; ++i) {
    const int32_t *w = items + i * kItemWords;
    require(w[5] > prev && w[5] < a.n_units, "fwd unit order");
    require(w[2] > w[1] && w[4] > w[3] && w[4] <= w[2], "fwd item ranges");
    require(w[6] >= 1 && w[6] <= 8, "fwd pieces");
    prev = w[5];
    if (w[6] > 1) {
      // touch every partial the pieces write, so that AddressSanitizer
      // checks them against the (host) workspace
      require(a.part_lse && a.part_o, "fwd split buffers");
      const int tiles = (w[2] - w[1] + kFwdBM - 1) / kFwdBM;
      for (int t = 0; t < tiles; ++t)
        for (int c = 0; c < w[6]; ++c)
          for (int h = 0; h < a.hq; ++h) {
            const int64_t pr = ((int64_t)(w[7] + t * w[6] + c) * a.hq + h) * kFwdBM;
            a.part_lse[pr] = a.part_lse[pr + kFwdBM - 1] = 0.f;
            a.part_o[pr * d] = a.part_o[(pr + kFwdBM) * d - 1] = 0.f;
          }
      split_tiles += tiles;
    }
  }
  require(items[5] == 0, "fwd first unit");
  // the merge's tile table: rows within their item, partials within range
  require(m.n_tiles == split_tiles, "split tile count");
  for (int t = 0; t < m.n_tiles; ++t) {
    const int32_t *st = (m.tiles ? m.tiles : m.inline_tiles) + t * kSplitTileWords;
    require(st[2] > st[1] && st[2] - st[1] <= kFwdBM && st[3] > 1, "split tile rows");
    const int64_t last = ((int64_t)(st[4] + st[3] - 1) * m.hq + m.hq - 1) * kFwdBM + (st[2] - st[1]) - 1;
    volatile float x = m.part_lse[last];
    (void)x;
  }
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_bwd_pre(const PreArgs &a, int d, int, int, hipStream_t) {
  require(d == 64 || d == 128, "pre d");
  for (int g = 0; g < a.n_qg; ++g) require(a.qg[4 * g + 2] < a.n_q_units, "pre q units");
  volatile float sink = a.delta[0];  // D lives at the start of the workspace
  (void)sink;
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs &a, int d, int, int, hipStream_t) {
  require(d == 64 || d == 128, "bwd d");
  require(a.kv_pad >= a.kv_blocks && a.kv_pad % 8 == 0 && a.kv_pad - a.kv_blocks < 8, "bwd kv_pad");
  require(a.q_pad >= a.q_blocks && a.q_pad % 8 == 0 && a.q_pad - a.q_blocks < 8, "bwd q_pad");
  require(a.q_blocks == a.n_q_units * a.hq && (a.dq_first == 0 || a.dq_first == 1), "bwd q blocks");
  require(a.kv_blocks == a.n_kv_units * a.hkv, "bwd kv blocks");
  int32_t prev = -1;
  for (int g = 0; g < a.n_kvg; ++g) {
    const int32_t *r = a.kvg + 4 * g;
    require(r[3] > prev && r[3] < a.n_kv_units && r[2] > r[1], "bwd kv groups");
    prev = r[3];
  }
  prev = -1;
  for (int g = 0; g < a.n_qg; ++g) {
    const int32_t *r = a.qg + 4 * g;
    require(r[2] > prev && r[2] < a.n_q_units && r[0] >= 0 && r[1] >= 1 && r[0] + r[1] <= a.n_items, "bwd q groups");
    prev = r[2];
  }
  for (int i = 0; i < a.n_items; ++i) {
    const int32_t *w = a.items + i * kItemWords;
    require(w[0] >= 0 && (int64_t)w[0] + w[2] <= a.tokens, "bwd item reach");
  }
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t) {
  require(a.rows >= 1 && a.h >= 1 && a.d % 4 == 0 && a.lse_stride >= a.rows, "merge sizes");
  ++g_launches;
  return hipSuccess;
}

hipError_t noalloc_scratch(void **out) {
  *out = g_scratch_host;
  return hipSuccess;
}

}  // namespace segattn

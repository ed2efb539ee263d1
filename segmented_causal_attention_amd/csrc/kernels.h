// Internal interface between the C-ABI host layer (api.cpp) and the HIP
// kernels.  Not installed; no torch or HIP types appear in segattn.h.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace segattn {

// Device item table: one row of kItemWords int32 per work item.
//   [0] seq_off  [1] q_lo  [2] q_hi  [3] k_lo  [4] k_hi   (sequence-local)
//   [5] unit_begin: first work unit of this item in the launch's unit order
//   [6] aux0  [7] aux1  (per-kernel meaning: forward -- key pieces per query
//   tile and the item's first partial result; see FwdArgs)
constexpr int kItemWords = 8;

// Forward tile shape: kFwdWaves wavefronts x kFwdWaveRows query rows per
// workgroup, 64 keys per K/V tile staged through LDS in a ring of
// kFwdStages tiles.
constexpr int kFwdWaves = 8;
constexpr int kFwdWaveRows = 32;
constexpr int kFwdBM = kFwdWaveRows * kFwdWaves;
constexpr int kFwdBN = 64;
constexpr int kFwdStages = 4;

// Backward tile shapes.
//   dK/dV kernel: 128 keys per workgroup (4 key groups x 32 keys, each with
//                 a dV wavefront and a dK wavefront), 64 query rows per
//                 staged Q/dO tile pair.
//   dQ kernel:    256 query rows per workgroup (8 waves x 32 rows), 64 keys
//                 per staged K/V tile.
constexpr int kBwdKvWaves = 8;
constexpr int kBwdKvBN = 32 * (kBwdKvWaves / 2);
constexpr int kBwdKvBM = 64;
constexpr int kBwdQWaves = 8;
constexpr int kBwdQBM = 32 * kBwdQWaves;
constexpr int kBwdQBN = 64;
// Depth of the LDS rings.  dK/dV role: the tile the dV wavefronts use, the
// one the dK wavefronts (one step behind) use, and one in flight.  dQ role:
// the tile in use and three in flight.
constexpr int kBwdKvStages = 3;
constexpr int kBwdQStages = 4;

// Small launches carry their tables in the kernel arguments (no upload
// launch): up to kInlineItems item rows, kInlineSplitTiles split tiles.
constexpr int kInlineItems = 64;
constexpr int kInlineSplitTiles = 64;

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *items;  // device table, n_items rows; NULL: inline_items
  int32_t n_items;
  int32_t n_units;       // query tiles over all items
  int64_t tokens;
  int32_t hq, hkv;
  float scale_log2;      // scale * log2(e)
  int32_t merge;         // 1: merge into the fp32 (O, LSE) already in o/lse
  // Split query tiles (item word [6] = P > 1 key pieces): piece c of query
  // tile t of an item whose first partial is f = word [7] writes partial
  // (f + t P + c) of head h, index (f + t P + c) * hq + h, into part_lse
  // [.][kFwdBM] and part_o [.][kFwdBM][d] (rows local to the tile).
  float *part_lse, *part_o;
  int32_t inline_items[kInlineItems * kItemWords];
};

// The pieces' combination, launched after the forward: one row of
// kSplitTileWords int32 per split query tile:
//   [0] seq_off  [1] r0  [2] r1 (its rows, sequence-local)  [3] P  [4] first partial
constexpr int kSplitTileWords = 5;
constexpr int kFwdMaxPieces = 8;  // key pieces per split query tile, at most
struct SplitMergeArgs {
  const int32_t *tiles;  // device table, n_tiles rows; NULL: inline_tiles
  int32_t n_tiles;       // 0: nothing was split
  int32_t hq;
  int64_t tokens;
  const float *part_lse, *part_o;
  void *o;
  float *lse;
  int32_t merge;         // as FwdArgs::merge
  int32_t inline_tiles[kInlineSplitTiles * kSplitTileWords];
};

// delta[h][t] = -D = -<dO[t,h,:], O[t,h,:]> for the query rows of the items
// (negated: the backward's products dP = dO V^T start from it and yield
// dP - D directly).  One workgroup per (q unit, query head), the q units of
// the backward's q groups (BwdArgs below).
struct PreArgs {
  const void *o, *d_o;
  float *delta;
  const int32_t *items, *qg;
  int32_t n_qg, n_q_units;
  int64_t tokens;
  int32_t hq;
};

// Backward tables.  Items keep the caller's order (the kernels walk them in
// reverse).  kv units: one per (kv group, 128-key tile); kv group g covers
// keys [kb, ke) of one sequence, stored as rows of kvg (4 int32):
//   [0] seq_off [1] kb [2] ke [3] unit_begin
// q units: one per (q group, 256-row tile); q group = a run of adjacent items
// with identical query ranges, stored as rows of qg (4 int32):
//   [0] first item  [1] item count  [2] unit_begin  [3] unused
struct BwdArgs {
  const void *q, *k, *v, *d_o;
  const float *lse, *delta;
  void *dq, *dk, *dv;
  const int32_t *items, *kvg, *qg;
  int32_t n_items, n_kvg, n_qg;
  int32_t n_kv_units, n_q_units;
  int32_t kv_blocks;     // n_kv_units * hkv: dK/dV workgroups
  int32_t kv_pad;        // kv_blocks rounded up to a multiple of 8
  int32_t q_blocks;      // n_q_units * hq: dQ workgroups
  int32_t q_pad;         // q_blocks rounded up to a multiple of 8
  int32_t dq_first;      // 1: workgroups [0, q_blocks) are dQ, then from q_pad dK/dV;
                         // 0: [0, kv_blocks) dK/dV, then from kv_pad dQ
  int64_t tokens;
  int32_t hq, hkv;
  float scale, scale_log2;
  int32_t accumulate;    // 1: fp32 outputs, add to them
};

struct MergeArgs {
  int64_t rows;
  int32_t h, d;
  int64_t lse_stride;
  const float *o_a, *lse_a, *o_b, *lse_b;
  float *o_out, *lse_out;
};

// Launchers (return the hipError_t of the launch).  Template arguments are
// resolved inside the .hip files from the runtime dtype codes.
hipError_t launch_fwd(const FwdArgs &a, const SplitMergeArgs &m, int d, int in_dtype, int o_dtype, hipStream_t s);
hipError_t launch_bwd_pre(const PreArgs &a, int d, int o_dtype, int in_dtype, hipStream_t s);
hipError_t launch_bwd(const BwdArgs &a, int d, int in_dtype, int g_dtype, hipStream_t s);
// launch_bwd's kernel for a.dq_first (bwd_dqfirst.hip)
hipError_t launch_bwd_dq_first(const BwdArgs &a, int d, int in_dtype, int g_dtype, hipStream_t s);
hipError_t launch_merge(const MergeArgs &a, hipStream_t s);
// Copies n int32 words from host memory into dst (device) through kernel
// arguments: stream-ordered, graph-capturable, no pageable-memory copy.
hipError_t launch_upload(int32_t *dst, const int32_t *words, int64_t n, hipStream_t s);
// Device address of the no-allocation scratch array (SEGATTN_NOALLOC_SCRATCH_BYTES)
// on the current device, looked up once per device.
hipError_t noalloc_scratch(void **out);

}  // namespace segattn

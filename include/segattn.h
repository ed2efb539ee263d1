/*
 * segattn.h -- C ABI of the segmented causal attention library (libsegattn.so)
 *
 * One causal softmax attention layer over token-major packed sequences, cut
 * into work items, on one AMD Instinct MI355X (gfx950).  Forward returns the
 * output O and the per-row log-sum-exp LSE; partial results over disjoint key
 * ranges are combined with a log-sum-exp merge; backward returns dQ, dK, dV.
 *
 * Sources (the web pages this implements):
 *   - SPPO: Efficient Long-sequence LLM Training via Adaptive Sequence
 *     Pipeline Parallel Offloading -- section 3.2 (FLOPs-based partition,
 *     earlier subsequences longer), section 5.1 / Figure 9 (segment i's
 *     queries attend to the resident K/V of segments 0..i), section 5.2
 *     (FLOPs-optimized partition s0..sN), section 6.1 (2K-16K tokens per
 *     layer per device).
 *   - InfiniPipe: Elastic Pipeline Parallelism for Efficient Variable-Length
 *     Long-Context LLM Training -- section II-A (ring-style multi-step online
 *     self-attention; forward after preceding slices, backward after
 *     subsequent slices), section II-B (packed [sum(S), D] layout),
 *     section III-A1 (chunk {C, S}), eq. (1) (quadratic causal work).
 *   - Sequence Parallelism: Long Sequence Training from System Perspective
 *     (blog) -- Ring Self-Attention: a device uses its own K block first,
 *     then receives the earlier ones around the ring.
 *
 * Conventions shared by every call
 * --------------------------------
 *   - Status: every entry point returns 0 (SEGATTN_OK) or one of the
 *     SEGATTN_E_* codes.  All arguments are validated on the host before
 *     anything is launched; on error nothing is written and nothing is
 *     launched.  segattn_last_error() gives a thread-local detail string.
 *     No C++ exception crosses this interface.
 *   - Launches are asynchronous on the caller's HIP stream (hipStream_t
 *     passed as void*, NULL = the default stream).  The library never
 *     synchronises, never allocates or frees memory, keeps no pointer after
 *     a call returns and has no global mutable state except the thread-local
 *     error string and the per-device scratch of segattn_bwd_noalloc (its
 *     comment says how calls share it).  Device faults surface at the
 *     caller's next sync.
 *   - Ownership: the caller owns every buffer.  "device" pointers are HIP
 *     device memory, "host" pointers ordinary host memory.
 *   - Layouts (contiguous, strides implied, 16-byte aligned device pointers):
 *       Q, O, dO, dQ : [tokens][hq][d]        K, V, dK, dV : [tokens][hkv][d]
 *       LSE, D       : float [hq][tokens] (natural logarithm)
 *     Query head h reads KV head floor(h * hkv / hq) (contiguous groups).
 *   - Work item (sequence-local, half-open): query rows [q_lo, q_hi) and key
 *     rows [k_lo, k_hi) of the packed sequence starting at token seq_off.
 *     A query row q sees key k iff k_lo <= k < k_hi and k <= q.
 */
#ifndef SEGATTN_H
#define SEGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SEGATTN_OK             0
#define SEGATTN_E_INVALID      1 /* null / misaligned pointer, bad dtype, bad flag, bad item table */
#define SEGATTN_E_UNSUPPORTED  2 /* d not in {64,128}, hq % hkv != 0 */
#define SEGATTN_E_RANGE        3 /* S < N, empty segment or item, index beyond tokens, k_hi > q_hi, int32 overflow */
#define SEGATTN_E_CAPACITY     4 /* output array too small; *n_items receives the size needed */
#define SEGATTN_E_WORKSPACE    5 /* workspace missing or smaller than *_workspace() reported */
#define SEGATTN_E_DEVICE       6 /* a HIP launch or runtime call failed */

/* element types */
#define SEGATTN_BF16 0
#define SEGATTN_F32  1

/* flags */
#define SEGATTN_MERGE_INTO  1u /* fwd: merge the new partial into the fp32 (O, LSE) already in o/lse */
#define SEGATTN_ACCUMULATE  2u /* bwd: dq/dk/dv are fp32 accumulators; results are added to them */
#define SEGATTN_D_READY     4u /* bwd: D was already computed into the workspace by segattn_bwd_preprocess */
#define SEGATTN_SPLIT_KEYS  8u /* fwd: on a launch too small to fill the GPU, cut long key walks across workgroups */

typedef struct {
  int64_t seq_off, q_lo, q_hi, k_lo, k_hi;
} segattn_item;

typedef struct {
  int64_t tokens;   /* packed token count T (<= 2^31 - 1) */
  int32_t hq, hkv;  /* query heads, KV heads (hq % hkv == 0) */
  int32_t d;        /* head dimension: 64 or 128 */
  int32_t in_dtype; /* SEGATTN_BF16, or SEGATTN_F32 (rounded to bf16, nearest-even, while staging) */
  float scale;      /* softmax scale applied to <q, k>, usually 1/sqrt(d); finite and > 0 */
} segattn_shape;

/* ---------------------------------------------------------------- planner
 * Host functions: integer arithmetic only, no device work. */

/* FLOPs-balanced partition of one causal sequence of S tokens into N segments
 * (SPPO section 3.2 FLOPs-based policy, section 5.2; InfiniPipe eq. (1)
 * quadratic term).  bounds (host, N+1 entries) receives b_0 = 0 < b_1 < ... <
 * b_N = S where every inner b_i minimises |N*T(b) - i*T(S)|, T(x) = x(x+1)/2,
 * ties to the smaller b.  Segment lengths come out non-increasing (earlier
 * segments longer) whenever S >= 8*N*N.
 * Errors: E_INVALID (bounds NULL, N < 1), E_RANGE (S < N, S > 2^31-1, or an
 * empty segment). */
int segattn_partition(int64_t S, int32_t N, int64_t *bounds);

/* Work items of a packed variable-length batch (InfiniPipe section II-B
 * packing, section III-A1 split chunks; SPPO section 6.1 slice cap).
 * cu_seqlens (host, nseq+1 entries, non-decreasing from 0).  A sequence of
 * length L <= max_slice is one item {cu[s], 0, L, 0, L}; a longer one is cut
 * by segattn_partition(L, n) for the least n >= 2 whose first (longest) slice
 * is <= max_slice, each slice [lo, hi) giving {cu[s], lo, hi, 0, hi}.  Empty
 * sequences give no item.  items (host, cap entries) receives the items in
 * sequence order; *n_items the count.
 * Errors: E_INVALID (NULL pointer, nseq < 0, max_slice < 1, cu not starting
 * at 0 or decreasing), E_RANGE (total > 2^31-1, a slice would be empty),
 * E_CAPACITY (cap too small: *n_items = needed, items untouched). */
int segattn_partition_varlen(const int64_t *cu_seqlens, int32_t nseq, int64_t max_slice,
                             segattn_item *items, int32_t cap, int32_t *n_items);

/* Ring-order items of one sequence (InfiniPipe section II-A ring-style SP;
 * Ring Self-Attention in the sequence-parallelism blog): for each segment
 * i of bounds (host, N+1 entries) and blocks of `block` keys, the blocks
 * j = ceil(b_{i+1}/block)-1 down to 0 each give the item
 * {0, b_i, b_{i+1}, j*block, min((j+1)*block, b_{i+1})}: the segment's own
 * (diagonal) block first, then the earlier blocks in the order they arrive.
 * Errors: E_INVALID (NULL, N < 1, block < 1, bounds not strictly increasing
 * from 0), E_RANGE (> 2^31-1), E_CAPACITY (as above). */
int segattn_ring_items(const int64_t *bounds, int32_t N, int64_t block,
                       segattn_item *items, int32_t cap, int32_t *n_items);

/* Workload-balanced chunks of a packed variable-length batch (InfiniPipe
 * section III-B, Algorithm 1; slice cost of section III-A2, eq. (1)).  A
 * slice of s tokens after a context of C tokens costs
 * alpha1 ((C + s)^2 - C^2) + alpha2 s.
 *  1. The longest sequence L is cut into min(K, L) slices of equal cost (the
 *     mesh): inner boundary i is the integer b minimising |K f(b) - i f(L)|,
 *     f(b) = alpha1 b^2 + alpha2 b, ties to the smaller b.
 *  2. Every sequence is cut at the inner mesh boundaries inside it; the
 *     pieces before its last cut are split chunks, the last piece its tail
 *     slice.  A sequence without a cut is short; empty ones are dropped.
 *  3. Best-fit-decreasing: one bucket per tail slice, ordered by
 *     time / tokens ascending (ties: older bucket first); short sequences
 *     by decreasing cost (ties: earlier sequence first).  A sequence opens a
 *     new bucket when even the bucket with the fewest tokens would exceed
 *     token_cap (T_m); otherwise it joins the first bucket within both the
 *     time threshold T_t (initially f(L) / min(K, L)) and T_m; if none,
 *     T_t becomes the least bucket time plus the sequence's cost over the
 *     buckets within T_m, and the placement is retried.
 * Output: the split chunks (by sequence, then position), then the buckets in
 * the order they were opened, as work items {seq_off = cu[j], q = [lo, hi),
 * k = [0, hi)} grouped by chunk; chunk_of[i] (optional, may be NULL) is the
 * chunk of item i.  *n_chunks receives the chunk count and *time_threshold
 * (optional) the final T_t.  All float64 arithmetic in a fixed order.
 * cu_seqlens: HOST int64[nseq + 1] from 0, non-decreasing, <= 2^31-1 tokens.
 * Errors: E_INVALID (NULL, nseq < 1, K < 1, alpha1 <= 0, alpha2 < 0 or not
 * finite, token_cap < 1, cu_seqlens invalid, every sequence empty),
 * E_RANGE (> 2^31-1 tokens), E_CAPACITY (*n_items receives the size needed;
 * nothing else is written). */
int segattn_chunk_varlen(const int64_t *cu_seqlens, int32_t nseq, int32_t K, double alpha1, double alpha2,
                         int64_t token_cap, segattn_item *items, int32_t *chunk_of, int32_t cap,
                         int32_t *n_items, int32_t *n_chunks, double *time_threshold);

/* ---------------------------------------------------------------- forward */

/* Workspace bytes segattn_fwd needs for this shape and item table. */
int segattn_fwd_workspace(const segattn_shape *shape, const segattn_item *items, int32_t n_items,
                          size_t *bytes);

/* Partial causal attention of the items (SPPO section 5.1: the queries of a
 * segment against the resident K/V prefix; InfiniPipe section II-A: one step
 * of the multi-step online self-attention).  For every item and query head h:
 *   z_j = scale * <Q_q, K_j> over the item's visible keys j,
 *   LSE_q = log sum_j exp(z_j),  O_q = sum_j exp(z_j - LSE_q) V_j.
 * A row with no visible key gives (O, LSE) = (0, -inf).
 * q, k, v: device, in_dtype.  items: HOST array, n_items >= 1; the items'
 * global query ranges [seq_off+q_lo, seq_off+q_hi) must be pairwise
 * disjoint.  o: device [tokens][hq][d] of o_dtype (SEGATTN_BF16 or
 * SEGATTN_F32); lse: device float [hq][tokens].  Only the items' rows are
 * written.  flags: 0, or SEGATTN_MERGE_INTO (o must be F32): the new partial
 * is merged into the (O, LSE) already held in o/lse with the log-sum-exp
 * rule of segattn_merge.  SEGATTN_SPLIT_KEYS (for launches too small to
 * fill the GPU: fewer than 1024 (query tile, head) work units): the keys of
 * each query tile may be cut into up to 8 pieces of at least 2 64-key
 * tiles, computed by separate workgroups, and a second kernel on the
 * stream combines them with the same log-sum-exp merge, in piece order (the
 * segmented-plus-merged evaluation of InfiniPipe section II-A within one
 * call).  The piece count is the one whose longest-first schedule on the
 * GPU finishes first (at most 512 MiB of partials).  Results are deterministic but rounded differently from the
 * unsplit walk; without the flag a row's result does not depend on which
 * other items share the call.  workspace: device, >= segattn_fwd_workspace
 * bytes, which covers the call with or without the flag.  stream:
 * hipStream_t.
 * Errors: E_INVALID, E_UNSUPPORTED, E_RANGE, E_WORKSPACE, E_DEVICE. */
int segattn_fwd(const segattn_shape *shape, const void *q, const void *k, const void *v,
                const segattn_item *items, int32_t n_items, void *o, int32_t o_dtype, float *lse,
                uint32_t flags, void *workspace, size_t ws_bytes, void *stream);

/* Log-sum-exp merge of two partial results over disjoint key sets
 * (InfiniPipe section II-A online self-attention; the combination follows
 * from softmax over a disjoint union): for every row r < rows and head
 * hh < h, with m = max(l_a, l_b):
 *   m = -inf            ->  (O, LSE) = (0, -inf)
 *   otherwise w = e^(l - m),  LSE = m + log(w_a + w_b),
 *                             O = (w_a O_a + w_b O_b) / (w_a + w_b).
 * o_*: device float [rows][h][d]; lse_*: device float, element (hh, r) at
 * lse[hh * lse_stride + r] (lse_stride >= rows, e.g. the full token count
 * when merging a row range of a larger tensor).  o_out/lse_out may alias
 * the a or b operands exactly (in place).  d: a multiple of 4, at most 1024.
 * Errors: E_INVALID, E_UNSUPPORTED (d > 1024), E_RANGE, E_DEVICE. */
int segattn_merge(int64_t rows, int32_t h, int32_t d, int64_t lse_stride,
                  const float *o_a, const float *lse_a, const float *o_b, const float *lse_b,
                  float *o_out, float *lse_out, void *stream);

/* --------------------------------------------------------------- backward */

/* Workspace bytes segattn_bwd / segattn_bwd_preprocess need. */
int segattn_bwd_workspace(const segattn_shape *shape, const segattn_item *items, int32_t n_items,
                          size_t *bytes);

/* D_q = <dO_q, O_q> for every query row of the items, stored NEGATED (-D_q)
 * into the workspace (float [hq][tokens] at its start; entries of rows
 * outside the items' query ranges are not written), followed by the plan
 * tables.  Lets the caller time or schedule the reduction apart from the
 * main backward kernel; segattn_bwd then takes SEGATTN_D_READY with items
 * whose query rows are among these.  Arguments as in segattn_bwd. */
int segattn_bwd_preprocess(const segattn_shape *shape, const void *o, int32_t o_dtype, const void *d_o,
                           const segattn_item *items, int32_t n_items, void *workspace, size_t ws_bytes,
                           void *stream);

/* Gradients of f = sum(dO * O) for the items' attention, given the final
 * (merged) O and LSE of the forward (dLSE = 0).  With P = e^(z - LSE):
 *   dV_j += sum_q P_qj dO_q,  dS_qj = P_qj (<dO_q, V_j> - D_q),
 *   dQ_q += scale sum_j dS_qj K_j,  dK_j += scale sum_q dS_qj Q_q,
 * summed over the items in REVERSE item order (InfiniPipe section II-A:
 * a slice's backward follows those of the slices after it), and for dK/dV
 * over the query heads of each KV head's group.
 * q, k, v, d_o: device, in_dtype; o: device, o_dtype; lse: device float.
 * items: HOST array; items whose global query ranges overlap must have
 * identical query ranges and be adjacent in the array (e.g. the blocks of one
 * segment in ring order).  dq [tokens][hq][d], dk/dv [tokens][hkv][d]:
 * device, g_dtype (BF16 or F32).  Without SEGATTN_ACCUMULATE the rows of dq
 * covered by some item's query range and the rows of dk/dv covered by some
 * item's key range are overwritten (other rows untouched); with it g_dtype
 * must be F32 and the gradients are added.  workspace: device, >=
 * segattn_bwd_workspace bytes.
 * dQ is evaluated as dQ_q = scale sum_j dS_qj (K_j - K_q), keys measured
 * from the query row's own key K_q.  That is the same value (sum_j dS_qj = 0
 * over a row's visible keys), and it keeps a component that all keys share
 * out of dQ's rounding error.  So a call's dQ is the full gradient only for
 * rows whose visible keys the call's items cover completely (as one call
 * over all items, or the per-segment calls of a reverse-order schedule,
 * do); calls that split one row's keys between them sum to it exactly, but
 * each one alone is not the gradient through its own keys.
 * Errors: E_INVALID, E_UNSUPPORTED, E_RANGE, E_WORKSPACE, E_DEVICE. */
int segattn_bwd(const segattn_shape *shape, const void *q, const void *k, const void *v,
                const void *o, int32_t o_dtype, const float *lse, const void *d_o,
                const segattn_item *items, int32_t n_items, void *dq, void *dk, void *dv,
                int32_t g_dtype, uint32_t flags, void *workspace, size_t ws_bytes, void *stream);

/* Maximum scratch of segattn_bwd_noalloc: 64 MiB per device. */
#define SEGATTN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* segattn_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, meaning and results as segattn_bwd, without the
 * workspace: D and the plan tables go into a 64 MiB array of the library's
 * own device memory (SEGATTN_NOALLOC_SCRATCH_BYTES), which every GPU the
 * library runs on holds until the process ends.  The call allocates
 * nothing.  It uses the scratch of the CALLER'S CURRENT DEVICE (the stream
 * must belong to it).  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give wrong results.  Nothing in the scratch has to start at zero (D and
 * the tables are written before they are read).  SEGATTN_D_READY is not
 * accepted (D is always computed).  A call whose scratch need --
 * segattn_bwd_workspace bytes, about 4 * hq * tokens for D -- exceeds the
 * maximum returns E_WORKSPACE before launching anything.
 * Errors: as segattn_bwd, plus E_WORKSPACE for a too-large call. */
int segattn_bwd_noalloc(const segattn_shape *shape, const void *q, const void *k, const void *v, const void *o,
                        int32_t o_dtype, const float *lse, const void *d_o, const segattn_item *items,
                        int32_t n_items, void *dq, void *dk, void *dv, int32_t g_dtype, uint32_t flags,
                        void *stream);

/* ---------------------------------------------------------------- offload
 * Moving a subsequence's backward-only activations to host memory while the
 * next subsequence computes (SPPO section 5.1, two-level activation
 * management: keys and values stay resident because later subsequences
 * attend to them; section 5.2, sequence-aware offloading).  For attention
 * the backward-only tensors of a segment are its Q and O rows and its LSE
 * entries.  The library plans and copies; the caller owns every buffer and
 * decides when device rows may be released or overwritten. */

/* Copy directions of segattn_copy_rows. */
#define SEGATTN_D2H 0 /* device -> host */
#define SEGATTN_H2D 1 /* host -> device */

/* Offload plan of n subsequences, subsequence i holding rows[i] rows of
 * row_bytes[i] bytes (A_i = rows[i] * row_bytes[i], exact in int64 then
 * converted to double).  SPPO section 5.2: each stage moves the same volume,
 * alpha_i A_i = threshold_bytes, so alpha_i = min(1, threshold / A_i)
 * (0 when A_i = 0); rows_moved[i] = floor(alpha_i * rows[i]) whole rows; the
 * GPU memory after stage i is M_0 = A_0, M_i = M_{i-1} + A_i - alpha_{i-1}
 * A_{i-1}, and *peak_bytes = max_i M_i.  Double arithmetic, in that order.
 * alpha, rows_moved, mem_bytes: HOST arrays of n entries; peak_bytes may be
 * NULL.  Errors: E_INVALID (NULL arrays, n < 1, threshold not finite and
 * > 0, a negative rows or row_bytes, or an int64 overflow in A_i). */
int segattn_offload_plan(const int64_t *rows, const int64_t *row_bytes, int32_t n, double threshold_bytes,
                         double *alpha, int64_t *rows_moved, double *mem_bytes, double *peak_bytes);

/* Copies `rows` rows of `row_bytes` bytes, row r from src + r*src_pitch to
 * dst + r*dst_pitch, asynchronously on `stream` (a hipStream_t, NULL = the
 * null stream).  kind SEGATTN_D2H: src device, dst host; SEGATTN_H2D: src
 * host, dst device.  The host side should be pinned memory (from
 * hipHostMalloc) for the copy to run beside kernels.  Pitches >= row_bytes.
 * rows == 0 or row_bytes == 0 is a no-op.  Errors: E_INVALID (NULL pointer
 * with a non-empty copy, bad kind, negative sizes, pitch < row_bytes),
 * E_DEVICE. */
int segattn_copy_rows(void *dst, int64_t dst_pitch, const void *src, int64_t src_pitch, int64_t row_bytes,
                      int64_t rows, int32_t kind, void *stream);

/* Makes to_stream wait, without blocking the host, for all work enqueued on
 * from_stream so far: records `event` (a hipEvent_t owned by the caller) on
 * from_stream and makes to_stream wait for it.  Errors: E_INVALID (NULL
 * event), E_DEVICE. */
int segattn_stream_order(void *event, void *from_stream, void *to_stream);

/* ------------------------------------------------------------- diagnostics */

/* Static name of a status code ("SEGATTN_OK", ...). */
const char *segattn_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
const char *segattn_last_error(void);
/* Library version string. */
const char *segattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEGATTN_H */

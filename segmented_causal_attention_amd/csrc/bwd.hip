// Backward kernels for gfx950 (CDNA4), bf16 MFMA, fp32 accumulation.
//
// Gradients of f = sum(dO * O) for the items' attention, given the forward's
// final LSE and D = <dO, O> (computed beforehand and stored negated: the dP
// products start their accumulators from -D and so yield dP - D directly):
//   P = exp(scale <Q, K> - LSE),  dV += P^T dO,  dP = dO V^T,
//   dS = P (dP - D),  dQ += scale dS K,  dK += scale dS^T Q.
// InfiniPipe section II-A: a slice's backward runs after those of the slices
// that follow it (a key's gradient needs every later query); section III-A3:
// dK/dV of earlier slices are completed by the later slices' backward.  Here
// one launch covers all items; each key tile's dK/dV accumulate in registers
// over the items in REVERSE item order, so no atomics are needed and the
// result is deterministic.
//
// One kernel, two kinds of workgroup (bwd_kernel at the end of this file):
// dK/dV role: key-stationary.  A workgroup owns 128 keys of one KV head in
//   4 groups of 32; each group is handled by two wavefronts on one SIMD.  It
//   walks every (item, query head of the group, 64-row query tile) that can
//   see its keys, one tile per barrier.  In iteration i the dV wavefront
//   computes S = Q K^T and P of tile i, leaves P (bf16) in an LDS buffer and
//   accumulates dV += P^T dO.  The dK wavefront first finishes tile i-1:
//   dS = P (dP - D) with the P left in iteration i-1 and the dP - D it
//   computed then, and dK += dS^T Q; then it computes dP = dO V^T of tile i
//   (its accumulators start from -D, so they hold dP - D).  The two
//   wavefronts on a SIMD thus run their matrix products and their
//   elementwise work at different times.  Each wavefront keeps only its own key-side operand (K or V) and
//   accumulator in registers, so two fit on every SIMD, and the two do equal
//   MFMA work (2 products each per tile).  Q and dO tiles are staged once, in
//   the column layout: row reads for the products over the head dim,
//   transposing reads for those over query rows.
// dQ role: query-stationary, like the forward.  A workgroup owns 256 query
//   rows of one head (8 wavefronts x 32 rows, two per SIMD; Q and dO in
//   registers) and walks the 64-key tiles of every item of its query group;
//   per tile it recomputes S^T, P, dP^T - D, dS^T and accumulates dQ^T
//   (3 products).
//   Keys are measured from the query row's own key: dQ_i = scale sum_j dS_ij
//   (K_j - K_i).  The two forms agree exactly because a row's dS sums to zero
//   over its visible keys (softmax is shift invariant).  In floating point
//   they do not: dS is rounded to bf16 for the product, and D comes from the
//   forward's O (built from bf16 P) while P here is fp32, so the computed dS
//   of a row misses zero by about 2^-9 of its size.  Multiplied by K_j, that
//   miss carries every component the keys share; multiplied by K_j - K_i, only
//   how the keys vary near the row.  The row sum R_i of the bf16 dS values
//   that enter the product is accumulated beside it (v_dot2 against ones),
//   and the epilogue subtracts R_i K_i from sum_j dS_ij K_j.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile.h"

namespace segattn {
namespace dev {

template <int D>
struct BwdCfg {
  static constexpr int KS = D / 32;   // depth steps over the head dim
  static constexpr int NT = D / 16;   // 16-wide head-dim tiles
  static constexpr int TSZ = kTileRows * D;  // one swizzled 64-row tile (bf16 elements)
};
static_assert(kBwdKvBM == kTileRows && kBwdQBN == kTileRows, "backward tiles are 64-row LDS tiles");

template <typename GT>
__device__ __forceinline__ void put1(GT *p, float v, int accumulate);
template <>
__device__ __forceinline__ void put1<float>(float *p, float v, int accumulate) {
  *p = accumulate ? *p + v : v;
}
template <>
__device__ __forceinline__ void put1<__bf16>(__bf16 *p, float v, int) {
  *p = __builtin_bit_cast(__bf16, (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu));
}

template <typename GT>
__device__ __forceinline__ void put4(GT *p, const f32x4 &v, int accumulate);
template <>
__device__ __forceinline__ void put4<float>(float *p, const f32x4 &v, int accumulate) {
  f32x4 x = v;
  if (accumulate) x += *reinterpret_cast<const f32x4 *>(p);
  *reinterpret_cast<f32x4 *>(p) = x;
}
template <>
__device__ __forceinline__ void put4<__bf16>(__bf16 *p, const f32x4 &v, int) {
  *reinterpret_cast<u32x2 *>(p) = (u32x2){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// The plan tables (items, key groups, query groups) are read through the
// constant address space: they are not written while the kernel runs, and
// wave-uniform reads of them become scalar loads.  Vector loads would be
// waited for with vmcnt(0), which also waits for every tile copy in flight.
typedef const __attribute__((address_space(4))) int32_t *ctab;
__device__ __forceinline__ ctab as_ctab(const int32_t *p) { return (ctab)p; }

// One row of the item table (kItemWords words) in a single scalar load.  The
// walkers below keep the ranges of their current item in registers and read
// the table only when they move to another item, so a step does not wait
// for table loads.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
static_assert(kItemWords == 8, "item rows are loaded as 8 words");
__device__ __forceinline__ i32x8 item_row(ctab items, int i) {
  return *(const __attribute__((address_space(4))) i32x8 *)(items + i * kItemWords);
}

__device__ __forceinline__ int find_unit(ctab tab, int words, int field, int n, int rank) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab[mid * words + field] <= rank)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// =================================================================== dK/dV

struct KvStep {
  int item;  // < 0: done
  int hh;    // query head within the group
  int qt0;   // first query row of the tile (sequence-local)
  int q_lo, q_hi, k_lo, k_hi;  // the item's query and key ranges
  int64_t qoff;  // element offset of the tile's first Q / dO row: ((seq_off + qt0) hq + h) d
  int64_t soff;  // offset of its first LSE / D entry: h T + seq_off + qt0
};

// What the dK/dV walker needs to know about its workgroup.
struct KvWalk {
  ctab items;
  int G, seq_off, kt0, kt1, g, hq, d;
  int64_t T;
  __device__ __forceinline__ void offsets(KvStep &s) const {
    const int64_t h = (int64_t)g * G + s.hh, row = (int64_t)seq_off + s.qt0;
    s.qoff = (row * hq + h) * d;
    s.soff = h * T + row;
  }
  // Next step at or below item i: the first item (walking down) of sequence
  // seq_off whose keys meet [kt0, kt1) and whose queries reach past kt0.
  __device__ __forceinline__ KvStep first_from(int i) const {
    for (; i >= 0; --i) {
      const i32x8 r = item_row(items, i);
      if (r[0] == seq_off && r[3] < kt1 && r[4] > kt0 && r[2] > kt0) {
        KvStep s{i, 0, max(r[1], kt0), r[1], r[2], r[3], r[4], 0, 0};
        offsets(s);
        return s;
      }
    }
    return KvStep{-1, 0, 0, 0, 0, 0, 0, 0, 0};
  }
  // The next 64-row tile: within a run of tiles the offsets just move on.
  __device__ __forceinline__ KvStep advance(KvStep s) const {
    s.qt0 += kBwdKvBM;
    if (s.qt0 < s.q_hi) {
      s.qoff += (int64_t)kBwdKvBM * hq * d;
      s.soff += kBwdKvBM;
      return s;
    }
    if (++s.hh < G) {
      s.qt0 = max(s.q_lo, kt0);
      offsets(s);
      return s;
    }
    return first_from(s.item - 1);
  }
};

// LDS of the backward kernel.  Each role carves the same block its own way:
//   dK/dV role: a ring of kBwdKvStages (Q, dO) 64-row tile pairs, their row
//     statistics, and the P hand-over buffers (kKvPBufs);
//   dQ role:    a ring of kBwdQStages (K, V) 64-key tile pairs.
template <int D>
struct BwdLds {
  static constexpr int kTile = kTileRows * D;                     // bf16 elements of one tile
  static constexpr int kKvRing = kBwdKvStages * 2 * kTile * 2;    // bytes
  static constexpr int kKvStat = kBwdKvStages * 2 * kBwdKvBM * 4;
  // P of step i is written in step i and read in step i+1: two buffers (by
  // step parity) suffice when the ring length is even.
  static constexpr int kKvPBufs = kBwdKvStages % 2 == 0 ? 2 : kBwdKvStages;
  static constexpr int kKvP = kKvPBufs * 4 * 2 * 2 * 64 * 16;  // [buffer][group][half][key block][lane] x 16 B
  static constexpr int kKv = kKvRing + kKvStat + kKvP;
  static constexpr int kQ = kBwdQStages * 2 * kTile * 2;
  static constexpr int kBytes = kKv > kQ ? kKv : kQ;
};

template <int D, typename InT, typename GT>
__device__ __forceinline__ void dkdv_body(const BwdArgs &a, int x, char *smem) {
  using C = BwdCfg<D>;
  using L = BwdLds<D>;
  constexpr int W = kBwdKvWaves;
  constexpr int NG = W / 2;        // key groups of 32 keys
  constexpr int BQ = kBwdKvBM;     // 64 query rows per tile
  constexpr int NS = kBwdKvStages;
  constexpr int BUF = 2 * C::TSZ;  // Q, dO (column layout, read both ways)
  static_assert(NG == 4 && BUF == 2 * L::kTile, "backward LDS layout");
  __bf16 *lds = reinterpret_cast<__bf16 *>(smem);
  const uint32_t lds0 = lds_addr(smem);  // LDS byte address of the block
  float(*stat)[2][BQ] = reinterpret_cast<float(*)[2][BQ]>(smem + L::kKvRing);
  // P of a tile, handed from each group's dV wavefront to its dK wavefront:
  // [buffer][group][32-row half][16-key block][lane] x 8 bf16 values (the very
  // operand of dV += P^T dO; bf16 keeps fp32's exponent range, which matters
  // at a million keys where P ~ 1e-6 would be subnormal in fp16).
  uint32_t(*pshare)[NG][2][2][64][4] = reinterpret_cast<uint32_t(*)[NG][2][2][64][4]>(smem + L::kKvRing + L::kKvStat);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  // Wavefronts w and w + NG share key group w % NG (and a SIMD): the first
  // computes P and accumulates dV, the second computes dP, takes P from the
  // first through LDS, and accumulates dK -- one query tile behind, so that
  // the two never wait for each other inside a tile.
  const int kgrp = wave % NG;
  const bool dk_role = wave >= NG;

  int rank, g;
  map_xcd(x, a.hkv, a.n_kv_units, rank, g);
  const ctab kv = as_ctab(a.kvg) + find_unit(as_ctab(a.kvg), 4, 3, a.n_kvg, rank) * 4;
  const int seq_off = kv[0], kb = kv[1], ke = kv[2];
  const int kt0 = kb + (rank - kv[3]) * kBwdKvBN;
  const int kt1 = min(ke, kt0 + kBwdKvBN);
  const int G = a.hq / a.hkv;
  const int64_t T = a.tokens;
  const ctab items = as_ctab(a.items);
  const float *__restrict__ lse = a.lse;
  const float *__restrict__ delta = a.delta;
  const int hq = a.hq, hkv = a.hkv;
  const InT *qg = static_cast<const InT *>(a.q);
  const InT *dg = static_cast<const InT *>(a.d_o);

  // This wavefront's keys [kw0, kw0 + 32).
  const int kw0 = kt0 + 32 * kgrp;
  const bool has_keys = kw0 < kt1;

  // Key-side fragments, B operand of the contraction over the head dim:
  // K (dV role: S = Q K^T) or V (dK role: dP = dO V^T);
  // lane holds X[key = kw0 + 16nk + l16][32ks + 8lg ..].
  bf16x8 xf[2][C::KS];
  {
    const InT *xg = static_cast<const InT *>(dk_role ? a.v : a.k);
#pragma unroll
    for (int nk = 0; nk < 2; ++nk) {
      const int key = kw0 + 16 * nk + l16;
      const bool ok = key < kt1;
      const int64_t base = ((int64_t)(seq_off + (ok ? key : kt0)) * hkv + g) * D + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        xf[nk][ks] = __builtin_bit_cast(bf16x8, ok ? load8<InT>(xg + base + 32 * ks) : (u32x4){0, 0, 0, 0});
    }
  }

  // dV (first role) or dK (second role) accumulator.
  f32x4 acc[2][C::NT];
#pragma unroll
  for (int nk = 0; nk < 2; ++nk)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[nk][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Loop-invariant LDS byte offsets of this lane's reads.
  int roff[C::KS], coff[C::NT];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) roff[ks] = row_read_off<D, kColTile>(ks, l16, lg);
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) coff[nt] = col_read_off<D>(nt, l16, lg);

  const int64_t qstride = (int64_t)hq * D;
  // The fragment loads above complete here, before the first tile copy: the
  // compiler then knows they are done, instead of waiting for vmcnt(0) (the
  // tile copies in flight included) before their first use in every step.
  wait_vm<0>();
  using Loader = TileLoader<D, InT, W>;
  Loader lqd;  // Q and dO tiles: same rows and stride
  lqd.init(wave, lane, qstride);
  // Stage s of the ring: the Q and dO tiles of step `st`, and (wavefront 0)
  // the tile's natural-log LSE and D rows.
  auto stage = [&](const KvStep &st, int s) __attribute__((always_inline)) {
    const int nvalid = min(BQ, st.q_hi - st.qt0);
    __bf16 *b = lds + s * BUF;
    const uint32_t ba = lds0 + s * BUF * 2;
    lqd.template stage<kColTile>(b, ba, qg + st.qoff, nvalid);
    lqd.template stage<kColTile>(b + C::TSZ, ba + C::TSZ * 2, dg + st.qoff, nvalid);
    if (wave == 0) {
      const uint32_t sa = lds0 + L::kKvRing + s * 2 * BQ * 4;  // stat[s][0], stat[s][1]
      stage_row_floats(sa, lse + st.soff, nvalid, lane);
      stage_row_floats(sa + BQ * 4, delta + st.soff, nvalid, lane);
    }
  };

  const float c2 = a.scale_log2;
  // Three walkers over the same step sequence: `ld` (staged), `cp` (the dV
  // wavefronts' step) and `pk` (the dK wavefronts' step, one behind).
  // Iteration i: stage i is published; stage i+AHEAD is copied into the slot
  // that step i-2 used (finished by both roles); the dV wavefronts work on
  // step i in slot i % NS and hand P over in buffer i % NP; the dK
  // wavefronts finish step i-1 in slot (i-1) % NS with its P, then compute
  // dP - D of step i in slot i % NS.
  constexpr int AHEAD = NS - 2;         // stages copied ahead of the dV step
  constexpr int NP = L::kKvPBufs;       // P hand-over buffers
  constexpr int LW = 2 * Loader::kInstr;  // copies per stage (wavefront 0: + 2 rows of statistics)
  static_assert(AHEAD >= 1 && (NP == 2 || NP == NS), "dK/dV ring");
  const KvWalk walk{items, G, seq_off, kt0, kt1, g, hq, D, T};
  KvStep cp = walk.first_from(a.n_items - 1);
  KvStep pk{-1, 0, 0, 0, 0, 0, 0, 0, 0};
  KvStep ld = cp;
  int issued = 0, done = 0;  // stages copied / steps of the dV wavefronts started
  // The copies of the next stage are issued after each wavefront's first
  // products of the step (or at its end when it has none) rather than right
  // after the barrier, where all eight wavefronts would queue theirs at once.
  bool pend = false;
  auto stage_if = [&](auto sc) __attribute__((always_inline)) {
    if (pend) {
      stage(ld, decltype(sc)::value);
      ld = walk.advance(ld);
      ++issued;
      pend = false;
    }
  };
#pragma unroll
  for (int s = 0; s < AHEAD; ++s)
    if (ld.item >= 0) {
      stage(ld, s);
      ld = walk.advance(ld);
      ++issued;
    }
  // Rows: half qp, sub-block ab of a 32-row half reads query rows
  // 32qp + 8*(m/4) + 4*ab + m%4, so a lane's 8 values of a half are the rows
  // 32qp + 8*lg + 0..7 for its key 16nk + l16 -- the A operand layout of the
  // contraction over query rows.  Slots are compile-time constants so every
  // LDS read is a precomputed lane offset plus an immediate.
  //
  // Does step st have work for this wavefront's keys?
  auto active = [&](const KvStep &st) __attribute__((always_inline)) {
    return st.item >= 0 && has_keys && kw0 < min(st.qt0 + BQ, st.q_hi);
  };
  // X = (rows of Xs) x (this wavefront's keys)^T over the head dim: S = Q K^T
  // from zero (dV role), or dP = dO V^T from -D of the rows of ring slot SL,
  // which leaves dP - D (dK role).
  auto rows_x = [&](const __bf16 *Xs, f32x4 (&xs)[2][2][2], auto dkc, auto slc) __attribute__((always_inline)) {
    constexpr int SL = decltype(slc)::value;
#pragma unroll
    for (int qp = 0; qp < 2; ++qp)
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) {
        f32x4 x0 = (f32x4){0.f, 0.f, 0.f, 0.f};
        if constexpr (decltype(dkc)::value) x0 = *reinterpret_cast<const f32x4 *>(&stat[SL][1][32 * qp + 8 * lg + 4 * ab]);
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) xs[qp][ab][nk] = x0;
      }
    pipelined<2 * C::KS>(
        [&](auto ic) __attribute__((always_inline)) {
          constexpr int qp = decltype(ic)::value / C::KS, ks = decltype(ic)::value % C::KS;
          struct {
            bf16x8 f[2];
          } xa;
#pragma unroll
          for (int ab = 0; ab < 2; ++ab) xa.f[ab] = lds_row8(Xs, roff[ks] + (32 * qp + 4 * ab) * 2 * D);
          return xa;
        },
        [&](auto ic, const auto &xa) __attribute__((always_inline)) {
          constexpr int qp = decltype(ic)::value / C::KS, ks = decltype(ic)::value % C::KS;
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int nk = 0; nk < 2; ++nk) xs[qp][ab][nk] = mfma16(xa.f[ab], xf[nk][ks], xs[qp][ab][nk]);
        });
  };
  // acc += opa^T Bt: dV += P^T dO or dK += dS^T Q; sub-step nt: the
  // transposed fragments of head-dim block nt, both halves
  auto accumulate = [&](const __bf16 *Bt, const bf16x8 (&opa)[2][2]) __attribute__((always_inline)) {
    pipelined<C::NT>(
        [&](auto ntc) __attribute__((always_inline)) {
          constexpr int nt = decltype(ntc)::value;
          struct {
            bf16x8 f[2];
          } bt;
#pragma unroll
          for (int qp = 0; qp < 2; ++qp) bt.f[qp] = lds_col8<D>(Bt, coff[nt] + 32 * qp * 2 * D);
          return bt;
        },
        [&](auto ntc, const auto &bt) __attribute__((always_inline)) {
          constexpr int nt = decltype(ntc)::value;
#pragma unroll
          for (int qp = 0; qp < 2; ++qp)
#pragma unroll
            for (int nk = 0; nk < 2; ++nk) acc[nk][nt] = mfma16(opa[qp][nk], bt.f[qp], acc[nk][nt]);
        });
  };
  // dV wavefronts, iteration i: S = Q K^T, P = exp(S - LSE) (masked on
  // boundary tiles; rows past q_hi of a partial tile repeat the last row in
  // LDS and drop out too), P handed to the dK wavefront through LDS, then
  // dV += P^T dO -- all of step i.
  auto dv_work = [&](auto slot) __attribute__((always_inline)) {
    constexpr int bslot = decltype(slot)::value;
    if (!active(cp)) return;
    const __bf16 *Qs = lds + bslot * BUF, *dOs = Qs + C::TSZ;
    const int k_lo = cp.k_lo, k_hi = cp.k_hi, q_hi = cp.q_hi, qt0 = cp.qt0;
    f32x4 xs[2][2][2];
    rows_x(Qs, xs, std::false_type{}, slot);
    stage_if(std::integral_constant<int, (bslot + AHEAD) % NS>{});

    bf16x8 opa[2][2];
    const bool need_mask = !(kw0 + 31 <= qt0 && kw0 >= k_lo && kw0 + 32 <= k_hi && qt0 + BQ <= q_hi);
    // The masked variant is a separate code path so that interior tiles
    // carry no mask arithmetic.
    auto make_p = [&](auto maskc) __attribute__((always_inline)) {
#pragma unroll
      for (int qp = 0; qp < 2; ++qp) {
        const f32x4 l0 = *reinterpret_cast<const f32x4 *>(&stat[bslot][0][32 * qp + 8 * lg]) * -kLog2e;
        const f32x4 l1 = *reinterpret_cast<const f32x4 *>(&stat[bslot][0][32 * qp + 8 * lg + 4]) * -kLog2e;
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) {
          // Row q = qt0 + 8lg + c (c = 32qp + 4ab + i) sees key `key` iff
          // key - qt0 - 8lg <= c <= q_hi - 1 - qt0 - 8lg and k_lo <= key < k_hi:
          // all of (c - c_lo), (c_hi - c) and kin are >= 0.  Their sign bit
          // picks a +inf / -inf bound for the exponent's argument (no
          // per-element compares, which would hold scalar register pairs).
          const int key = kw0 + 16 * nk + l16;
          const int c_lo = key - qt0 - 8 * lg, c_hi = q_hi - 1 - qt0 - 8 * lg;
          const int kin = (key - k_lo) | (k_hi - 1 - key);
          f32x4 pv[2];
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float arg = fmaf(xs[qp][ab][nk][i], c2, ab ? l1[i] : l0[i]);
              if constexpr (decltype(maskc)::value) {
                const int c = 32 * qp + 4 * ab + i;
                const uint32_t sign = (uint32_t)((c - c_lo) | (c_hi - c) | kin) & 0x80000000u;
                arg = fminf(arg, __builtin_bit_cast(float, sign | 0x7f800000u));
              }
              pv[ab][i] = fast_exp2(arg);
            }
          opa[qp][nk] = pack_bf16x8(pv[0], pv[1]);
          *reinterpret_cast<bf16x8 *>(pshare[bslot % NP][kgrp][qp][nk][lane]) = opa[qp][nk];
        }
      }
    };
    if (need_mask)
      make_p(std::true_type{});
    else
      make_p(std::false_type{});

    accumulate(dOs, opa);

  };
  // dK wavefronts, iteration i: dS = P (dP - D) and dK += dS^T Q of step
  // i-1 (P from the dV wavefront, dP - D kept from the previous iteration),
  // then dP - D of step i.  In this order the dS arithmetic runs beside the
  // dV wavefront's S products and the dK products beside its exponentials,
  // so the two wavefronts sharing a SIMD tend to keep its matrix unit busy
  // in turn.
  f32x4 dp[2][2][2];  // dP - D of the step the dV wavefronts just did
  auto dk_work = [&](auto slot) __attribute__((always_inline)) {
    constexpr int bv = decltype(slot)::value;
    constexpr int bk = (bv + NS - 1) % NS;
    if (active(pk)) {
      bf16x8 opa[2][2];
#pragma unroll
      for (int qp = 0; qp < 2; ++qp)
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) {
          const u32x4 ph = *reinterpret_cast<const u32x4 *>(pshare[bk % NP][kgrp][qp][nk][lane]);
          f32x4 ds[2];
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t w = ph[2 * ab + (i >> 1)];
              const float pp = (i & 1) ? bf16_hi(w) : bf16_lo(w);
              ds[ab][i] = pp * dp[qp][ab][nk][i];
            }
          opa[qp][nk] = pack_bf16x8(ds[0], ds[1]);
        }

      accumulate(lds + bk * BUF, opa);
      stage_if(std::integral_constant<int, (bv + AHEAD) % NS>{});

    }
    if (active(cp)) {
      rows_x(lds + bv * BUF + C::TSZ, dp, std::true_type{}, slot);

    }
  };
  // The ring, one copy per role (same walkers, so the same barriers).
  auto ring = [&](auto &work) __attribute__((always_inline)) {
    auto step = [&](auto slot) __attribute__((always_inline)) -> bool {
      constexpr int bv = decltype(slot)::value;  // step i (dV role)
      // stage i landed; the stages copied after it may stay in flight
      if constexpr (AHEAD == 1)
        wait_vm<0>();  // only stage i was in flight
      else if (wave == 0)
        wait_stages<LW + 2, 3>(issued - done - 1);
      else
        wait_stages<LW, 3>(issued - done - 1);
      ring_barrier();

      pend = ld.item >= 0;
      work(slot);
      stage_if(std::integral_constant<int, (bv + AHEAD) % NS>{});
      pk = cp;
      if (cp.item >= 0) {
        cp = walk.advance(cp);
        ++done;
      }


      return pk.item >= 0;
    };
    if (cp.item >= 0)
      while (ring_pass<0, NS>(step)) {
      }
  };
  if (dk_role)
    ring(dk_work);
  else
    ring(dv_work);

  // ---- epilogue: lane holds rows key = kw0 + 16nk + 4lg + i, column 16nt + l16
  GT *outg = static_cast<GT *>(dk_role ? a.dk : a.dv);
  const float osc = dk_role ? a.scale : 1.f;
#pragma unroll
  for (int nk = 0; nk < 2; ++nk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kw0 + 16 * nk + 4 * lg + i;
      if (has_keys && key < kt1) {
        const int64_t base = ((int64_t)(seq_off + key) * hkv + g) * D + l16;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) put1<GT>(outg + base + 16 * nt, acc[nk][nt][i] * osc, a.accumulate);
      }
    }
}

// ====================================================================== dQ

struct QStep {
  int item;   // < 0: done
  int kv0;    // first key of the tile
  int k_end;  // min(k_hi, r1): end of the item's keys that this tile's rows can see
  int k_hi;   // the item's key range end
  int64_t kvoff;  // element offset of the tile's first K / V row: ((seq_off + kv0) hkv + g) d
};

// What the dQ walker needs to know about its workgroup.
struct QWalk {
  ctab items;
  int first, r1, seq_off, hkv, g, d;
  // Next step at or below item i of the query group (items first..): the
  // first item (walking down) with a key inside [k_lo, min(k_hi, r1)).
  __device__ __forceinline__ QStep first_from(int i) const {
    for (; i >= first; --i) {
      const i32x8 r = item_row(items, i);
      const int e = min(r[4], r1);
      if (e > r[3]) return QStep{i, r[3], e, r[4], (((int64_t)seq_off + r[3]) * hkv + g) * d};
    }
    return QStep{-1, 0, 0, 0, 0};
  }
  __device__ __forceinline__ QStep advance(QStep s) const {
    s.kv0 += kBwdQBN;
    s.kvoff += (int64_t)kBwdQBN * hkv * d;
    if (s.kv0 < s.k_end) return s;
    return first_from(s.item - 1);
  }
};

template <int D, typename InT, typename GT>
__device__ __forceinline__ void dq_body(const BwdArgs &a, int x, char *smem) {
  using C = BwdCfg<D>;
  constexpr int BN = kBwdQBN;  // 64 keys per tile
  constexpr int NS = kBwdQStages;
  constexpr int BUF = 2 * C::TSZ;  // K (column layout, read both ways), V (row layout)
  static_assert(NS * BUF * 2 == BwdLds<D>::kQ, "backward LDS layout");
  __bf16 *lds = reinterpret_cast<__bf16 *>(smem);
  const uint32_t lds0 = lds_addr(smem);  // LDS byte address of the block

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;

  int rank, h;
  map_xcd(x, a.hq, a.n_q_units, rank, h);
  const ctab items = as_ctab(a.items);
  const float *__restrict__ lse = a.lse;
  const float *__restrict__ delta = a.delta;
  const int hq = a.hq, hkv = a.hkv;
  const ctab grp = as_ctab(a.qg) + find_unit(as_ctab(a.qg), 4, 2, a.n_qg, rank) * 4;
  const int first = grp[0], count = grp[1];
  const ctab it0 = items + first * kItemWords;
  const int seq_off = it0[0], q_lo = it0[1], q_hi = it0[2];
  const int r1 = q_hi - (rank - grp[2]) * kBwdQBM;
  const int r0 = max(q_lo, r1 - kBwdQBM);
  const int g = h / (hq / hkv);
  const int64_t T = a.tokens;
  const InT *qg = static_cast<const InT *>(a.q);
  const InT *kg = static_cast<const InT *>(a.k);
  const InT *vg = static_cast<const InT *>(a.v);
  const InT *dg = static_cast<const InT *>(a.d_o);

  const int rw0 = r0 + 32 * wave;
  const int rw_end = min(rw0 + 32, r1);
  const bool has_rows = rw0 < rw_end;
  const int mkey = -8 * lg, mrow = l16 + mkey;  // lane constants of the mask

  bf16x8 qf[2][C::KS], dof[2][C::KS];
  float lse2[2], ndrow[2];  // LSE (base 2) and -D of the lane's two rows
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int row = rw0 + 16 * nq + l16;
    const bool ok = has_rows && row < r1;
    const int64_t grow = (int64_t)seq_off + (ok ? row : r0);
    const int64_t base = (grow * hq + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[nq][ks] = __builtin_bit_cast(bf16x8, ok ? load8<InT>(qg + base + 32 * ks) : (u32x4){0, 0, 0, 0});
      dof[nq][ks] = __builtin_bit_cast(bf16x8, ok ? load8<InT>(dg + base + 32 * ks) : (u32x4){0, 0, 0, 0});
    }
    const float l = ok ? lse[(int64_t)h * T + grow] : kNegInf;
    lse2[nq] = l == kNegInf ? __builtin_inff() : l * kLog2e;
    ndrow[nq] = ok ? delta[(int64_t)h * T + grow] : 0.f;  // stored as -D
  }

  f32x4 dq[2][C::NT];
  // Per-lane share of R = sum over keys of the bf16 dS of a row: lane
  // (l16, lg) holds keys 8lg .. 8lg+7 of each 32-key pair of rows 16nq + l16.
  float rsum[2] = {0.f, 0.f};
#pragma unroll
  for (int nq = 0; nq < 2; ++nq)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) dq[nq][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};


  // Loop-invariant LDS byte offsets of this lane's reads: step 0 only, the
  // other steps by XOR (row_step / col_step), which keeps this role's
  // register count within two wavefronts per SIMD.
  const int rkoff = row_read_off<D, kColTile>(0, l16, lg);
  const int rvoff = row_read_off<D, kRowTile>(0, l16, lg);
  const int coff = col_read_off<D>(0, l16, lg);

  const int64_t kstride = (int64_t)hkv * D;
  // The fragment loads above complete here, before the first tile copy: the
  // compiler then knows they are done, instead of waiting for vmcnt(0) (the
  // tile copies in flight included) before their first use in every step.
  wait_vm<0>();
  using Loader = TileLoader<D, InT, kBwdQWaves>;
  Loader lkv;  // K and V tiles: same rows and stride
  lkv.init(wave, lane, kstride);
  auto stage = [&](const QStep &st, int s) __attribute__((always_inline)) {
    const int nvalid = min(BN, st.k_end - st.kv0);
    __bf16 *b = lds + s * BUF;
    const uint32_t ba = lds0 + s * BUF * 2;
    lkv.template stage<kColTile>(b, ba, kg + st.kvoff, nvalid);
    lkv.template stage<kRowTile>(b + C::TSZ, ba + C::TSZ * 2, vg + st.kvoff, nvalid);
  };

  const float c2 = a.scale_log2;
  // `ld` stages NS-1 steps ahead of `cp`, which is computed.
  const QWalk walk{items, first, r1, seq_off, hkv, g, D};
  QStep cp = walk.first_from(first + count - 1);
  QStep ld = cp;
  int issued = 0, done = 0;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (ld.item >= 0) {
      stage(ld, s);
      ld = walk.advance(ld);
      ++issued;
    }
  auto step = [&](auto slot) __attribute__((always_inline)) -> bool {
    constexpr int buf = decltype(slot)::value;
    wait_stages<2 * Loader::kInstr, NS>(issued - done - 1);
    ring_barrier();  // stage `buf` visible; the slot staged next is free
    // copies of the next stage: after the first key pair's products (or at
    // the end of a step without rows), not all at once after the barrier
    bool pend = ld.item >= 0;
    auto stage_if = [&]() __attribute__((always_inline)) {
      if (pend) {
        stage(ld, (buf + NS - 1) % NS);
        ld = walk.advance(ld);
        ++issued;
        pend = false;
      }
    };
    const int kv0 = cp.kv0;
    const int k_hi = cp.k_hi;
    if (has_rows && kv0 <= rw_end - 1) {
      const __bf16 *Ks = lds + buf * BUF, *Vs = Ks + C::TSZ;
      const bool need_mask = (kv0 + BN - 1 > rw0) || (kv0 + BN > k_hi);
      bf16x8 dsb[2][2];
      // Each 32-key pair kp is finished (scores -> dS) before the next one
      // starts, which bounds the live score registers.
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        // ---- S^T = K Q^T, dP^T = V dO^T (half ab as in the forward)
        f32x4 s[2][2], dp[2][2];
#pragma unroll
        for (int nq = 0; nq < 2; ++nq)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab) {
            s[nq][ab] = (f32x4){0.f, 0.f, 0.f, 0.f};
            // dP^T starts from -D of the lane's query row: it yields dP - D
            dp[nq][ab] = (f32x4){ndrow[nq], ndrow[nq], ndrow[nq], ndrow[nq]};
          }
        // sub-steps 0 .. KS-1: the K row fragments of depth step ks (S^T);
        // KS .. 2KS-1: the V row fragments (dP^T).  One operand kind per
        // sub-step keeps half as many fragments in flight as loading both.
        pipelined<2 * C::KS>(
            [&](auto ic) __attribute__((always_inline)) {
              constexpr int ks = decltype(ic)::value % C::KS;
              constexpr bool is_v = decltype(ic)::value >= C::KS;
              struct {
                bf16x8 f[2];
              } f;
#pragma unroll
              for (int ab = 0; ab < 2; ++ab)
                f.f[ab] = is_v ? lds_row8(Vs, (rvoff ^ row_step(ks)) + (32 * kp + 4 * ab) * 2 * D)
                               : lds_row8(Ks, (rkoff ^ row_step(ks)) + (32 * kp + 4 * ab) * 2 * D);
              return f;
            },
            [&](auto ic, const auto &f) __attribute__((always_inline)) {
              constexpr int ks = decltype(ic)::value % C::KS;
              constexpr bool is_v = decltype(ic)::value >= C::KS;
#pragma unroll
              for (int ab = 0; ab < 2; ++ab)
#pragma unroll
                for (int nq = 0; nq < 2; ++nq) {
                  if constexpr (is_v)
                    dp[nq][ab] = mfma16(f.f[ab], dof[nq][ks], dp[nq][ab]);
                  else
                    s[nq][ab] = mfma16(f.f[ab], qf[nq][ks], s[nq][ab]);
                }
            });
        if (kp == 0) stage_if();
        // dS = P (dP - D); the masked variant is a separate code path so
        // that interior tiles carry no per-element compares.
        auto make_ds = [&](auto maskc) __attribute__((always_inline)) {
#pragma unroll
          for (int nq = 0; nq < 2; ++nq) {
            f32x4 ds[2];
#pragma unroll
            for (int ab = 0; ab < 2; ++ab)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float arg = fmaf(s[nq][ab][i], c2, -lse2[nq]);
                if constexpr (decltype(maskc)::value) {
                  // key kv0 + 32kp + 8lg + c (c = 4ab + i) is visible to row
                  // qrow = rw0 + 16nq + l16 iff c <= min(qrow, k_hi - 1) - kv0
                  // - 32kp - 8lg, written with the two per-lane constants
                  // mrow = l16 - 8lg and mkey = -8lg: the sign of the
                  // difference picks a +inf / -inf bound (no compares)
                  const int lim = min(rw0 + 16 * nq + mrow, k_hi - 1 + mkey) - kv0 - 32 * kp;
                  const uint32_t sign = (uint32_t)(lim - (4 * ab + i)) & 0x80000000u;
                  arg = fminf(arg, __builtin_bit_cast(float, sign | 0x7f800000u));
                }
                const float pv = fast_exp2(arg);
                ds[ab][i] = pv * dp[nq][ab][i];
              }
            dsb[nq][kp] = pack_bf16x8(ds[0], ds[1]);
          }
        };
        if (need_mask)
          make_ds(std::true_type{});
        else
          make_ds(std::false_type{});
      }
      // ---- dQ^T += K^T dS^T
      // sub-step nt: the transposed K fragments of head-dim block nt
      pipelined<C::NT>(
          [&](auto ntc) __attribute__((always_inline)) {
            constexpr int nt = decltype(ntc)::value;
            struct {
              bf16x8 f[2];
            } ka;
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) ka.f[kp] = lds_col8<D>(Ks, (coff ^ col_step(nt)) + 32 * kp * 2 * D);
            return ka;
          },
          [&](auto ntc, const auto &ka) __attribute__((always_inline)) {
            constexpr int nt = decltype(ntc)::value;
#pragma unroll
            for (int kp = 0; kp < 2; ++kp)
#pragma unroll
              for (int nq = 0; nq < 2; ++nq) dq[nq][nt] = mfma16(ka.f[kp], dsb[nq][kp], dq[nq][nt]);
          });
      // ---- this tile's share of R (the bf16 dS values of the product
      // above), after the product is issued so that it runs beside it; two
      // independent chains per row halve the dependent latency.  (Adding it
      // into per-lane LDS slots with ds_add_f32 instead, to save the two
      // registers, made the backward 14% slower.)
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        float t[2] = {0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const u32x4 w = __builtin_bit_cast(u32x4, dsb[nq][kp]);
#pragma unroll
          for (int e = 0; e < 4; ++e) t[kp] = sum_bf16x2(w[e], t[kp]);
        }
        rsum[nq] += t[0] + t[1];
      }
    }
    stage_if();
    cp = walk.advance(cp);
    ++done;
    return cp.item >= 0;
  };
  if (cp.item >= 0)
    while (ring_pass<0, NS>(step)) {
    }

  // ---- epilogue: lane holds dQ[row = rw0 + 16nq + l16][16nt + 4lg + i];
  // subtract R_row K_row (the bf16 values the products used), then scale.
  GT *dqg = static_cast<GT *>(a.dq);
  const XorLanes xl(lane);
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int row = rw0 + 16 * nq + l16;
    // the row's four lane shares (lanes l16 + 16 lg), in a fixed order
    const float r = wave_sum_xor16_32(rsum[nq], xl);
    if (has_rows && row < r1) {
      const int64_t grow = (int64_t)seq_off + row;
      const InT *kp = kg + (grow * hkv + g) * D + 4 * lg;
      GT *p = dqg + (grow * hq + h) * D + 4 * lg;
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        const f32x4 kr = load4_bf16<InT>(kp + 16 * nt);
        put4<GT>(p + 16 * nt, (dq[nq][nt] - r * kr) * a.scale, a.accumulate);
      }
    }
  }
}

// One launch for both roles.  Normally workgroups [0, kv_blocks) are dK/dV
// tiles and [kv_pad, kv_pad + q_blocks) dQ tiles, so the dQ workgroups start
// as the dK/dV ones drain; when the dQ role's longest walk is the longer
// one (a call over a few late segments: few query tiles, each against every
// earlier key), the dQ role goes first instead, so that its long walks start
// at once and the short dK/dV tiles fill in around them.  The second range
// starts at a multiple of the 8 XCDs so that both keep the head -> XCD map;
// the padding workgroups exit at once.
template <int D, typename InT, typename GT, bool DQ_FIRST>
__global__ __launch_bounds__(64 * kBwdKvWaves) void bwd_kernel(BwdArgs a) {
  static_assert(kBwdKvWaves == kBwdQWaves, "both roles use the same workgroup size");
  __shared__ __attribute__((aligned(16))) char smem[BwdLds<D>::kBytes];
  const int x = blockIdx.x;
  if constexpr (DQ_FIRST) {
    if (x < a.q_blocks)
      dq_body<D, InT, GT>(a, x, smem);
    else if (x >= a.q_pad)
      dkdv_body<D, InT, GT>(a, x - a.q_pad, smem);
  } else {
    if (x < a.kv_blocks)
      dkdv_body<D, InT, GT>(a, x, smem);
    else if (x >= a.kv_pad)
      dq_body<D, InT, GT>(a, x - a.kv_pad, smem);
  }
}

// Each role order is compiled in its own translation unit (this file, and
// bwd_dqfirst.hip, which includes it with SEGATTN_BWD_DQ_FIRST defined):
// with both kernels in one module the compiler inlined the shared helpers
// differently and the dK/dV-first kernel grew from 13 to 27 spilled scalar
// registers (+0.8% time).
#ifdef SEGATTN_BWD_DQ_FIRST
constexpr bool kDqFirstTU = true;
#else
constexpr bool kDqFirstTU = false;
#endif

template <int D, typename InT, typename GT>
static hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
  const int64_t grid = kDqFirstTU ? (int64_t)a.q_pad + a.kv_blocks : (int64_t)a.kv_pad + a.q_blocks;
  hipLaunchKernelGGL((bwd_kernel<D, InT, GT, kDqFirstTU>), dim3((unsigned)grid), dim3(64 * kBwdKvWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace dev

#define SEGATTN_DISPATCH(FN, a, d, in_dtype, g_dtype, s)                                   \
  do {                                                                                    \
    const bool ib = (in_dtype) == 0, gb = (g_dtype) == 0;                                 \
    if ((d) == 128) {                                                                     \
      if (ib) return gb ? dev::FN<128, __bf16, __bf16>(a, s) : dev::FN<128, __bf16, float>(a, s); \
      return gb ? dev::FN<128, float, __bf16>(a, s) : dev::FN<128, float, float>(a, s);   \
    }                                                                                     \
    if (ib) return gb ? dev::FN<64, __bf16, __bf16>(a, s) : dev::FN<64, __bf16, float>(a, s); \
    return gb ? dev::FN<64, float, __bf16>(a, s) : dev::FN<64, float, float>(a, s);       \
  } while (0)

#ifdef SEGATTN_BWD_DQ_FIRST
hipError_t launch_bwd_dq_first(const BwdArgs &a, int d, int in_dtype, int g_dtype, hipStream_t s) {
  SEGATTN_DISPATCH(launch_bwd_t, a, d, in_dtype, g_dtype, s);
}
#else
hipError_t launch_bwd(const BwdArgs &a, int d, int in_dtype, int g_dtype, hipStream_t s) {
  if (a.dq_first) return launch_bwd_dq_first(a, d, in_dtype, g_dtype, s);
  SEGATTN_DISPATCH(launch_bwd_t, a, d, in_dtype, g_dtype, s);
}
#endif

#undef SEGATTN_DISPATCH

}  // namespace segattn

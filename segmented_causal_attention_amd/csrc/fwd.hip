// Forward partial attention kernel for gfx950 (CDNA4), bf16 MFMA.
//
// One workgroup = one query tile of up to 256 rows of one work item and one
// query head: 8 wavefronts x 32 rows, two wavefronts per SIMD, so one
// wavefront's softmax overlaps the other's matrix products.  The item's
// visible keys are streamed in 64-key tiles that global_load_lds copies
// straight into swizzled LDS tiles (a ring of kFwdStages slots, copied up to
// kFwdStages - 1 tiles ahead) while the query rows stay in registers.  Scores are computed transposed, S^T = K Q^T, so that every
// lane owns one query row's scores: the row max needs only two cross-lane
// steps, and the probabilities are already in the B-operand layout of the
// second product O^T += V^T P^T, whose V^T operand comes from transposing LDS
// reads.
//
// What it computes (SPPO section 5.1 / Figure 9: a segment's queries against
// the resident K/V of all segments up to it; InfiniPipe section II-A: one
// step of the multi-step online self-attention): for each query row q of the
// item, over the visible keys j (k_lo <= j < k_hi, j <= q),
//   LSE_q = log sum_j exp(scale <Q_q, K_j>),   O_q = sum_j exp(scale <Q_q,K_j> - LSE_q) V_j,
// optionally merged into an existing fp32 (O, LSE) with the log-sum-exp rule.
#include <cstddef>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile.h"

namespace segattn {
namespace dev {

template <int D>
struct FwdCfg {
  static constexpr int W = kFwdWaves;      // wavefronts per workgroup
  static constexpr int BM = kFwdBM;        // query rows per workgroup
  static constexpr int BN = kFwdBN;        // keys per LDS tile (= kTileRows)
  static constexpr int NQ = kFwdWaveRows / 16;  // 16-row subtiles per wavefront
  static constexpr int KS = D / 32;        // depth steps of K Q^T
  static constexpr int MT = D / 16;        // 16-wide head-dim tiles of O^T
  static constexpr int KP = BN / 32;       // 32-key pairs per tile
  static constexpr int TSZ = BN * D;       // one swizzled tile (bf16 elements)
  static constexpr int BUF = 2 * TSZ;      // K (row tile), V (column tile)
  static constexpr int NS = kFwdStages;    // LDS ring depth
};
static_assert(kFwdBN == kTileRows && kFwdBM == kFwdWaves * kFwdWaveRows && kFwdWaveRows % 16 == 0,
              "forward tile shape");

// Tables are read through the constant address space (scalar loads):
// either a device table or one carried in the kernel arguments, whose
// explicit part starts at the kernel argument segment pointer.
typedef const __attribute__((address_space(4))) int32_t *ctab;
template <typename Args>
__device__ __forceinline__ ctab arg_table(const int32_t *dev, size_t inline_offset) {
  if (dev) return (ctab)dev;
  return (ctab)((const __attribute__((address_space(4))) char *)__builtin_amdgcn_kernarg_segment_ptr() + inline_offset);
}

// Index of the item whose unit range holds `rank` (unit_begin ascending).
__device__ __forceinline__ int find_item(ctab items, int n, int rank) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (items[mid * kItemWords + 5] <= rank)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <typename OutT>
__device__ __forceinline__ void store4(OutT *p, const f32x4 &v);
template <>
__device__ __forceinline__ void store4<float>(float *p, const f32x4 &v) {
  *reinterpret_cast<f32x4 *>(p) = v;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16 *p, const f32x4 &v) {
  *reinterpret_cast<u32x2 *>(p) = (u32x2){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

template <int D, typename InT, typename OutT>
__global__ __launch_bounds__(64 * kFwdWaves, kFwdWaveRows > 32 ? 1 : 2) void fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  constexpr int NS = C::NS;
  __shared__ __attribute__((aligned(16))) __bf16 lds[NS * C::BUF];
  const uint32_t lds0 = lds_addr(lds);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const XorLanes xl(lane);

  int rank, h;
  map_xcd(blockIdx.x, a.hq, a.n_units, rank, h);
  const ctab items = arg_table<FwdArgs>(a.items, offsetof(FwdArgs, inline_items));
  const ctab it = items + find_item(items, a.n_items, rank) * kItemWords;
  const int seq_off = it[0], q_lo = it[1], q_hi = it[2], k_lo = it[3], k_hi = it[4];
  // Work unit = (query tile, key piece): P pieces per query tile (P = 1
  // unless the launch splits key walks), part0 = the item's first partial.
  const int P = it[6], part0 = it[7];
  const int local = rank - it[5];
  const int tile = local / P, piece = local - tile * P;
  const int r1 = q_hi - tile * C::BM;             // heaviest (last) rows first
  const int r0 = max(q_lo, r1 - C::BM);
  const int hq = a.hq, hkv = a.hkv;
  const int g = (h * hkv) / hq;
  const int64_t T = a.tokens;

  const InT *__restrict__ qg = static_cast<const InT *>(a.q);
  const InT *__restrict__ kg = static_cast<const InT *>(a.k);
  const InT *__restrict__ vg = static_cast<const InT *>(a.v);

  // This wavefront's query rows [rw0, rw_end).
  const int rw0 = r0 + kFwdWaveRows * wave;
  const int rw_end = min(rw0 + kFwdWaveRows, r1);
  const bool has_rows = rw0 < rw_end;
  const int rw_max = rw_end - 1;

  // Query fragments (B operand of K Q^T): lane holds Q[row = l16][8*lg .. +8]
  // of each 32-dim step, matching the K row reads of logical chunk 4ks + lg.
  bf16x8 qf[C::NQ][C::KS];
#pragma unroll
  for (int nq = 0; nq < C::NQ; ++nq) {
    const int row = rw0 + 16 * nq + l16;
    const bool ok = has_rows && row < r1;
    const InT *qp = qg + ((int64_t)(seq_off + (ok ? row : r0)) * hq + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 w = ok ? load8<InT>(qp + 32 * ks) : (u32x4){0, 0, 0, 0};
      qf[nq][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Loop-invariant LDS byte offsets of this lane's reads.
  int roff[C::KS], coff[C::MT];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) roff[ks] = row_read_off<D>(ks, l16, lg);
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) coff[mt] = col_read_off<D>(mt, l16, lg);

  // This piece's 64-key tiles: its share [t0, t1) of the query tile's tiles.
  const int ke = min(k_hi, r1);
  const int nall = ke > k_lo ? (ke - k_lo + C::BN - 1) / C::BN : 0;
  const int t0 = piece * nall / P, t1 = (piece + 1) * nall / P;
  const int kb = k_lo + t0 * C::BN;
  const int ntiles = t1 - t0;

  float m_run[C::NQ];
  // Row sums of P on the matrix unit: an extra O^T block whose A operand is
  // all ones gives sum_k P^T[k][row] in every value of the lane of that row.
  // It sums the same bf16 P as the numerator, so the normalised weights add
  // up to one exactly and O's rounding error scales with V's spread around
  // O rather than with |V|.
  f32x4 lsum[C::NQ];
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (u32x4){0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  f32x4 o[C::NQ][C::MT];
#pragma unroll
  for (int nq = 0; nq < C::NQ; ++nq) {
    m_run[nq] = kNegInf;
    lsum[nq] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) o[nq][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // K and V tiles of 64 keys starting at key kvs, staged into ring slot `slot`.
  const int64_t kvstride = (int64_t)hkv * D;
  // The fragment loads above complete here, before the first tile copy: the
  // compiler then knows they are done, instead of waiting for vmcnt(0) (the
  // tile copies in flight included) before their first use in every step.
  wait_vm<0>();
  using Loader = TileLoader<D, InT, C::W>;
  // bf16 input: direct global -> LDS copies, NS - 1 tiles ahead.  fp32 input
  // (rounded to bf16 on the way): the tile NS - 1 ahead is fetched into
  // registers in one step and rounded into its slot in the next, so no step
  // waits for a global load of its own.
  constexpr bool kViaRegs = std::is_same<InT, float>::value;
  Loader lkv, lv;  // lv: the fp32 path's V registers
  lkv.init(wave, lane, kvstride);
  lv.init(wave, lane, kvstride);
  auto stage = [&](int kvs, int slot) __attribute__((always_inline)) {
    __bf16 *Ks = lds + slot * C::BUF;
    const uint32_t ka = lds0 + slot * C::BUF * 2;  // its LDS byte address
    const int64_t off = ((int64_t)(seq_off + kvs) * hkv + g) * D;
    lkv.template stage<kRowTile>(Ks, ka, kg + off, ke - kvs);
    lkv.template stage<kColTile>(Ks + C::TSZ, ka + C::TSZ * 2, vg + off, ke - kvs);
  };
  auto fetch = [&](int kvs) __attribute__((always_inline)) {
    if constexpr (kViaRegs) {
      const int64_t off = ((int64_t)(seq_off + kvs) * hkv + g) * D;
      lkv.fetch(kg + off, ke - kvs);
      lv.fetch(vg + off, ke - kvs);
    }
  };
  auto commit = [&](int slot) __attribute__((always_inline)) {
    if constexpr (kViaRegs) {
      __bf16 *Ks = lds + slot * C::BUF;
      lkv.template commit<kRowTile>(Ks);
      lv.template commit<kColTile>(Ks + C::TSZ);
    }
  };

  const float c2 = a.scale_log2;
  int issued = 0, j = 0;  // tiles staged (fp32: fetched) / steps done
  bool pending = false;   // fp32: a fetched tile waits for its slot
  if constexpr (kViaRegs) {
#pragma unroll
    for (int s = 0; s < NS - 2; ++s)
      if (issued < ntiles) {
        stage(kb + issued * C::BN, s);
        ++issued;
      }
    if (issued < ntiles) {
      fetch(kb + issued * C::BN);
      ++issued;
      pending = true;
    }
  } else {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (issued < ntiles) {
        stage(kb + issued * C::BN, s);
        ++issued;
      }
  }

  // One key tile.  The ring slot is a compile-time constant so every LDS
  // read is a precomputed lane offset plus an immediate.
  auto step = [&](auto slot) __attribute__((always_inline)) -> bool {
    constexpr int buf = decltype(slot)::value;
    if constexpr (!kViaRegs) wait_stages<2 * Loader::kInstr, NS>(issued - j - 1);
    ring_barrier();  // tile `buf` visible; the slot staged next is free
    if constexpr (kViaRegs) {
      // tile j + NS - 2 (fetched last step) into the slot tile j - 2 used;
      // the barriers of steps j + 1 .. j + NS - 2 publish it
      if (pending) {
        commit((buf + NS - 2) % NS);
        pending = false;
      }
      if (issued < ntiles) {
        fetch(kb + issued * C::BN);
        ++issued;
        pending = true;
      }
    } else if (issued < ntiles) {
      stage(kb + issued * C::BN, (buf + NS - 1) % NS);
      ++issued;
    }
    const int kv0 = kb + j * C::BN;
    const __bf16 *Ks = lds + buf * C::BUF;
    const __bf16 *Vs = Ks + C::TSZ;

    if (has_rows && kv0 <= rw_max) {
      // ---- S^T = K Q^T.  Pair kp covers keys 32kp..32kp+31; half ab of the
      // pair reads key rows 8*(m/4) + 4*ab + m%4 so that a lane's 8 values of
      // a pair are the keys 32kp + 8*lg + 0..7 of its query row.
      f32x4 s[C::NQ][C::KP][2];
#pragma unroll
      for (int nq = 0; nq < C::NQ; ++nq)
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp) {
          s[nq][kp][0] = (f32x4){0.f, 0.f, 0.f, 0.f};
          s[nq][kp][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      // sub-step ks: the 2 x KP key fragments of depth step ks
      pipelined<C::KS>(
          [&](auto ksc) __attribute__((always_inline)) {
            constexpr int ks = decltype(ksc)::value;
            struct {
              bf16x8 f[C::KP][2];
            } kf;
#pragma unroll
            for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
              for (int ab = 0; ab < 2; ++ab) kf.f[kp][ab] = lds_row8(Ks, roff[ks] + (32 * kp + 4 * ab) * 2 * D);
            return kf;
          },
          [&](auto ksc, const auto &kf) __attribute__((always_inline)) {
            constexpr int ks = decltype(ksc)::value;
#pragma unroll
            for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
              for (int ab = 0; ab < 2; ++ab)
#pragma unroll
                for (int nq = 0; nq < C::NQ; ++nq) s[nq][kp][ab] = mfma16(kf.f[kp][ab], qf[nq][ks], s[nq][kp][ab]);
          });

      // ---- masking (boundary tiles only: a separate code path, so that
      // interior tiles carry no per-element compares)
      const bool need_mask = (kv0 + C::BN - 1 > rw0) || (kv0 + C::BN > k_hi);
      if (need_mask) {
        // Key kv0 + 8lg + c (c = 32kp + 4ab + i) is visible to row qrow iff
        // c <= min(qrow, k_hi - 1) - kv0 - 8lg =: lim.  The sign of lim - c
        // picks +inf or -inf and min() applies it: no per-element compares,
        // each of which would hold a scalar register pair.
#pragma unroll
        for (int nq = 0; nq < C::NQ; ++nq) {
          const int lim = min(rw0 + 16 * nq + l16, k_hi - 1) - kv0 - 8 * lg;
#pragma unroll
          for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
            for (int ab = 0; ab < 2; ++ab)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t sign = (uint32_t)(lim - (32 * kp + 4 * ab + i)) & 0x80000000u;
                s[nq][kp][ab][i] = fminf(s[nq][kp][ab][i], __builtin_bit_cast(float, sign | 0x7f800000u));
              }
        }
      }

      // ---- online softmax (base 2), one query row per lane and subtile.
      // The row maxima of all subtiles first (their cross-lane steps
      // overlap), one wave-wide rescale test for all, then the exponentials.
      bf16x8 pf[C::NQ][C::KP];
      float mxs[C::NQ];
#pragma unroll
      for (int nq = 0; nq < C::NQ; ++nq) {
        float mx = kNegInf;
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[nq][kp][ab][i]);
        mxs[nq] = mx;
      }
#pragma unroll
      for (int nq = 0; nq < C::NQ; ++nq) mxs[nq] = wave_max_xor16_32(mxs[nq], xl) * c2;
      bool grow_any = false;
#pragma unroll
      for (int nq = 0; nq < C::NQ; ++nq) grow_any |= mxs[nq] > m_run[nq] + 8.f;
      if (__any(grow_any)) {
#pragma unroll
        for (int nq = 0; nq < C::NQ; ++nq) {
          const bool grow = mxs[nq] > m_run[nq] + 8.f;
          const float m_new = grow ? mxs[nq] : m_run[nq];
          const float alpha = grow ? fast_exp2(m_run[nq] - m_new) : 1.f;  // m_run = -inf -> 0
          lsum[nq] *= alpha;
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt) o[nq][mt] *= alpha;
          m_run[nq] = m_new;
        }
      }
#pragma unroll
      for (int nq = 0; nq < C::NQ; ++nq) {
        const float m_use = m_run[nq] == kNegInf ? 0.f : m_run[nq];
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[nq][kp][ab][i] = fast_exp2(fmaf(s[nq][kp][ab][i], c2, -m_use));
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp) pf[nq][kp] = pack_bf16x8(s[nq][kp][0], s[nq][kp][1]);
      }

      // ---- O^T += V^T P^T
      // sub-step mt: the V^T fragments of head-dim block mt
      pipelined<C::MT>(
          [&](auto mtc) __attribute__((always_inline)) {
            constexpr int mt = decltype(mtc)::value;
            struct {
              bf16x8 f[C::KP];
            } vf;
#pragma unroll
            for (int kp = 0; kp < C::KP; ++kp) vf.f[kp] = lds_col8<D>(Vs, coff[mt] + 32 * kp * 2 * D);
            return vf;
          },
          [&](auto mtc, const auto &vf) __attribute__((always_inline)) {
            constexpr int mt = decltype(mtc)::value;
#pragma unroll
            for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
              for (int nq = 0; nq < C::NQ; ++nq) o[nq][mt] = mfma16(vf.f[kp], pf[nq][kp], o[nq][mt]);
          });
#pragma unroll
      for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
        for (int nq = 0; nq < C::NQ; ++nq) lsum[nq] = mfma16(ones, pf[nq][kp], lsum[nq]);
    }
    ++j;
    return j < ntiles;
  };
  if (ntiles > 0)
    while (ring_pass<0, NS>(step)) {
    }

  // ---- epilogue: normalise; a key piece stores its partial; a whole
  // query tile merges into (O, LSE) if asked and stores its rows.
  float lse_row[C::NQ];
#pragma unroll
  for (int nq = 0; nq < C::NQ; ++nq) {
    const float lt = lsum[nq][0];
    lse_row[nq] = lt > 0.f ? (m_run[nq] + fast_log2(lt)) * kLn2 : kNegInf;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) o[nq][mt] *= inv;
  }
  if (P > 1) {
    // A key piece of a split query tile: its normalised partial goes to
    // partial (part0 + tile P + piece) of head h, rows local to the tile;
    // split_merge_kernel, next on the stream, combines the pieces.
    const int64_t pr0 = ((int64_t)(part0 + tile * P + piece) * hq + h) * C::BM;
#pragma unroll
    for (int nq = 0; nq < C::NQ; ++nq) {
      const int qrow = rw0 + 16 * nq + l16;
      if (has_rows && qrow < r1) {
        const int64_t pr = pr0 + (qrow - r0);
        if (lg == 0) a.part_lse[pr] = lse_row[nq];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) *reinterpret_cast<f32x4 *>(a.part_o + pr * D + 16 * mt + 4 * lg) = o[nq][mt];
      }
    }
    return;
  }
  OutT *__restrict__ og = static_cast<OutT *>(a.o);
#pragma unroll
  for (int nq = 0; nq < C::NQ; ++nq) {
    const int qrow = rw0 + 16 * nq + l16;
    const bool valid = has_rows && qrow < r1;
    const float lse_new = lse_row[nq];
    const int64_t grow = (int64_t)seq_off + (valid ? qrow : r0);
    float w_new = 1.f, w_old = 0.f, lse_out = lse_new;
    if (a.merge && valid) {
      const float lo_ = a.lse[(int64_t)h * T + grow];
      const float m = fmaxf(lo_, lse_new);
      if (m == kNegInf) {
        w_new = 0.f;
        lse_out = kNegInf;
      } else {
        const float eo = fast_exp2((lo_ - m) * kLog2e), en = fast_exp2((lse_new - m) * kLog2e);
        const float den = eo + en;
        w_old = eo / den;
        w_new = en / den;
        lse_out = m + fast_log2(den) * kLn2;
      }
    }
    if (valid) {
      OutT *op = og + (grow * hq + h) * D + 4 * lg;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        f32x4 val = o[nq][mt] * w_new;
        if constexpr (sizeof(OutT) == 4) {
          if (a.merge) val += *reinterpret_cast<const f32x4 *>(op + 16 * mt) * w_old;
        }
        store4<OutT>(op + 16 * mt, val);
      }
      if (lg == 0) a.lse[(int64_t)h * T + grow] = lse_out;
    }
  }
}

// Combines the key pieces of split query tiles (SEGATTN_SPLIT_KEYS): for
// each row, the log-sum-exp merge of its P partials in piece order (the
// rule of segattn_merge applied left to right), then, as the forward's own
// epilogue does, the optional merge into the (O, LSE) already held, and the
// stores.  One thread per (row, 4 columns) of a split query tile and head,
// D/4 workgroups per (tile, head): every load of a row is in flight at once
// (the pieces are few and the merge is latency-bound).
template <int D, typename OutT>
__global__ __launch_bounds__(256) void split_merge_kernel(SplitMergeArgs a) {
  constexpr int CPR = D / 4;  // 4-column chunks per row
  constexpr int BPT = kFwdBM * CPR / 256;  // workgroups per (tile, head)
  const int x = blockIdx.x, th = x / BPT, t = th / a.hq, h = th - t * a.hq;
  const ctab st = arg_table<SplitMergeArgs>(a.tiles, offsetof(SplitMergeArgs, inline_tiles)) + t * kSplitTileWords;
  const int seq_off = st[0], r0 = st[1], r1 = st[2], P = st[3], part = st[4];
  const int w = (x - th * BPT) * 256 + threadIdx.x;
  const int lr = w / CPR, c = w - lr * CPR;
  if (lr >= r1 - r0) return;
  const int64_t pstep = (int64_t)a.hq * kFwdBM;
  const int64_t pr0 = ((int64_t)part * a.hq + h) * kFwdBM + lr;
  float l[kFwdMaxPieces];
  f32x4 ov[kFwdMaxPieces];
#pragma unroll
  for (int p = 0; p < kFwdMaxPieces; ++p) {
    l[p] = p < P ? a.part_lse[pr0 + p * pstep] : kNegInf;
    ov[p] = p < P ? *reinterpret_cast<const f32x4 *>(a.part_o + (pr0 + p * pstep) * D + 4 * c)
                  : (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  float m = kNegInf;
#pragma unroll
  for (int p = 0; p < kFwdMaxPieces; ++p) m = fmaxf(m, l[p]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int p = 0; p < kFwdMaxPieces; ++p) {
      if (p < P) {
        const float wgt = fast_exp2((l[p] - m) * kLog2e);
        den += wgt;
        acc += wgt * ov[p];
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const float lse_new = den > 0.f ? m + fast_log2(den) * kLn2 : kNegInf;
  const int64_t grow = (int64_t)seq_off + r0 + lr;
  float w_new = 1.f, w_old = 0.f, lse_out = lse_new;
  if (a.merge) {
    const float lo_ = a.lse[(int64_t)h * a.tokens + grow];
    const float mm = fmaxf(lo_, lse_new);
    if (mm == kNegInf) {
      w_new = 0.f;
      lse_out = kNegInf;
    } else {
      const float eo = fast_exp2((lo_ - mm) * kLog2e), en = fast_exp2((lse_new - mm) * kLog2e);
      const float dd = eo + en;
      w_old = eo / dd;
      w_new = en / dd;
      lse_out = mm + fast_log2(dd) * kLn2;
    }
  }
  OutT *op = static_cast<OutT *>(a.o) + (grow * a.hq + h) * D + 4 * c;
  f32x4 val = acc * (inv * w_new);
  if constexpr (sizeof(OutT) == 4) {
    if (a.merge) val += *reinterpret_cast<const f32x4 *>(op) * w_old;
  }
  store4<OutT>(op, val);
  if (c == 0) a.lse[(int64_t)h * a.tokens + grow] = lse_out;
}

template <int D, typename InT, typename OutT>
static hipError_t launch_fwd_t(const FwdArgs &a, const SplitMergeArgs &m, hipStream_t s) {
  const int64_t grid = (int64_t)a.n_units * a.hq;
  hipLaunchKernelGGL((fwd_kernel<D, InT, OutT>), dim3((unsigned)grid), dim3(64 * FwdCfg<D>::W), 0, s, a);
  if (hipError_t e = hipGetLastError()) return e;
  if (m.n_tiles > 0) {
    constexpr int BPT = kFwdBM * (D / 4) / 256;
    hipLaunchKernelGGL((split_merge_kernel<D, OutT>), dim3((unsigned)((int64_t)m.n_tiles * m.hq * BPT)), dim3(256), 0,
                       s, m);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace dev

hipError_t launch_fwd(const FwdArgs &a, const SplitMergeArgs &m, int d, int in_dtype, int o_dtype, hipStream_t s) {
  using namespace dev;
  const bool in_bf = in_dtype == 0, out_bf = o_dtype == 0;
  if (d == 128) {
    if (in_bf) return out_bf ? launch_fwd_t<128, __bf16, __bf16>(a, m, s) : launch_fwd_t<128, __bf16, float>(a, m, s);
    return out_bf ? launch_fwd_t<128, float, __bf16>(a, m, s) : launch_fwd_t<128, float, float>(a, m, s);
  }
  if (in_bf) return out_bf ? launch_fwd_t<64, __bf16, __bf16>(a, m, s) : launch_fwd_t<64, __bf16, float>(a, m, s);
  return out_bf ? launch_fwd_t<64, float, __bf16>(a, m, s) : launch_fwd_t<64, float, float>(a, m, s);
}

}  // namespace segattn

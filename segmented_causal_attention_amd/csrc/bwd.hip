// Backward kernels for gfx950 (CDNA4), bf16 MFMA, fp32 accumulation.
//
// Gradients of f = sum(dO * O) for the items' attention, given the forward's
// final LSE and D = <dO, O> (computed beforehand):
//   P = exp(scale <Q, K> - LSE),  dV += P^T dO,  dP = dO V^T,
//   dS = P (dP - D),  dQ += scale dS K,  dK += scale dS^T Q.
// InfiniPipe section II-A: a slice's backward runs after those of the slices
// that follow it (a key's gradient needs every later query); section III-A3:
// dK/dV of earlier slices are completed by the later slices' backward.  Here
// one launch covers all items; each key tile's dK/dV accumulate in registers
// over the items in REVERSE item order, so no atomics are needed and the
// result is deterministic.
//
// dkdv_kernel: key-stationary.  A workgroup owns 128 keys of one KV head
//   (4 waves x 32 keys; K and V in registers) and walks every (item, query
//   head of the group, 64-row query tile) that can see them; per tile it
//   recomputes S, P, dP, dS and accumulates dV and dK (4 products).  Q and
//   dO tiles are staged row-major; the operands contracted over query rows
//   are read with transposing LDS reads.
// dq_kernel: query-stationary, like the forward.  A workgroup owns 128 query
//   rows of one head (4 waves x 32 rows; Q and dO in registers) and walks the
//   64-key tiles of every item of its query group; per tile it recomputes
//   S^T, P, dP^T, dS^T and accumulates dQ^T (3 products).
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

__device__ __forceinline__ int find_unit(const int32_t *tab, int words, int field, int n, int rank) {
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

__device__ __forceinline__ void map_head(int x, int nh, int &rank, int &h) {
  if ((nh & 7) == 0) {
    const int hpx = nh >> 3, xcd = x & 7, j = x >> 3;
    rank = j / hpx;
    h = xcd * hpx + j % hpx;
  } else {
    rank = x / nh;
    h = x % nh;
  }
}

// =================================================================== dK/dV

struct KvStep {
  int item;  // < 0: done
  int hh;    // query head within the group
  int qt0;   // first query row of the tile (sequence-local)
};

template <int D, typename InT, typename GT>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int BQ = kBwdKvBM;  // 64 query rows per tile
  constexpr int BUF = 2 * C::TSZ;  // Q tile, dO tile
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF];
  __shared__ __attribute__((aligned(16))) float stat[2][2][BQ];  // [buf][lse2 | D][row]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  int rank, g;
  map_head(blockIdx.x, a.hkv, rank, g);
  const int32_t *kv = a.kvg + find_unit(a.kvg, 4, 3, a.n_kvg, rank) * 4;
  const int seq_off = kv[0], kb = kv[1], ke = kv[2];
  const int kt0 = kb + (rank - kv[3]) * kBwdKvBN;
  const int kt1 = min(ke, kt0 + kBwdKvBN);
  const int G = a.hq / a.hkv;
  const int64_t T = a.tokens;
  const int32_t *__restrict__ items = a.items;
  const float *__restrict__ lse = a.lse;
  const float *__restrict__ delta = a.delta;
  const int hq = a.hq, hkv = a.hkv;
  const InT *qg = static_cast<const InT *>(a.q);
  const InT *kg = static_cast<const InT *>(a.k);
  const InT *vg = static_cast<const InT *>(a.v);
  const InT *dg = static_cast<const InT *>(a.d_o);

  // This wave's keys [kw0, kw0 + 32).
  const int kw0 = kt0 + 32 * wave;
  const bool has_keys = kw0 < kt1;

  // K and V fragments (B operands of Q K^T and dO V^T): lane holds
  // K[key = kw0 + 16nk + l16][32ks + 8lg .. +8].
  bf16x8 kf[2][C::KS], vf[2][C::KS];
#pragma unroll
  for (int nk = 0; nk < 2; ++nk) {
    const int key = kw0 + 16 * nk + l16;
    const bool ok = key < kt1;
    const int64_t base = ((int64_t)(seq_off + (ok ? key : kt0)) * hkv + g) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      kf[nk][ks] = __builtin_bit_cast(bf16x8, ok ? load8<InT>(kg + base + 32 * ks) : (u32x4){0, 0, 0, 0});
      vf[nk][ks] = __builtin_bit_cast(bf16x8, ok ? load8<InT>(vg + base + 32 * ks) : (u32x4){0, 0, 0, 0});
    }
  }

  f32x4 dk[2][C::NT], dv[2][C::NT];
#pragma unroll
  for (int nk = 0; nk < 2; ++nk)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      dk[nk][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
      dv[nk][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

  // ---- step iterator over (item in reverse order, head, query tile)
  auto item_sees = [&](int i) __attribute__((always_inline)) {
    const int32_t *it = items + i * kItemWords;
    return it[0] == seq_off && it[3] < kt1 && it[4] > kt0 && it[2] > kt0;
  };
  auto first_from = [&](int i) __attribute__((always_inline)) -> KvStep {
    for (; i >= 0; --i)
      if (item_sees(i)) return KvStep{i, 0, max(items[i * kItemWords + 1], kt0)};
    return KvStep{-1, 0, 0};
  };
  auto advance = [&](KvStep s) __attribute__((always_inline)) -> KvStep {
    const int32_t *it = items + s.item * kItemWords;
    s.qt0 += BQ;
    if (s.qt0 < it[2]) return s;
    if (++s.hh < G) {
      s.qt0 = max(it[1], kt0);
      return s;
    }
    return first_from(s.item - 1);
  };

  TileLoader<D, InT> lq, ldo;
  float st_lse = 0.f, st_d = 0.f;
  const int64_t qstride = (int64_t)hq * D;
  auto stage = [&](const KvStep &s, int buf) __attribute__((always_inline)) {
    const int32_t *it = items + s.item * kItemWords;
    const int h = g * G + s.hh;
    const int nvalid = min(BQ, it[2] - s.qt0);
    const int64_t row0 = (int64_t)seq_off + s.qt0;
    __bf16 *b = lds + buf * BUF;
    lq.issue(b, qg + (row0 * hq + h) * D, qstride, nvalid, wave, lane);
    ldo.issue(b + C::TSZ, dg + (row0 * hq + h) * D, qstride, nvalid, wave, lane);
    if (tid < BQ) {
      if (tid < nvalid) {
        const float l = lse[(int64_t)h * T + row0 + tid];
        // A row without visible keys (LSE = -inf) contributes nothing.
        st_lse = l == kNegInf ? __builtin_inff() : l * kLog2e;
        st_d = delta[(int64_t)h * T + row0 + tid];
      } else {
        st_lse = __builtin_inff();
        st_d = 0.f;
      }
    }
  };
  auto commit = [&](int buf) __attribute__((always_inline)) {
    __bf16 *b = lds + buf * BUF;
    lq.commit(b, tid);
    ldo.commit(b + C::TSZ, tid);
    if (tid < BQ) {
      stat[buf][0][tid] = st_lse;
      stat[buf][1][tid] = st_d;
    }
  };

  const float c2 = a.scale_log2;
  KvStep cur = first_from(a.n_items - 1);
  if (cur.item >= 0) {
    stage(cur, 0);
    commit(0);
  }
  wait_staged();
  __syncthreads();
  int buf = 0;
  while (cur.item >= 0) {
    const KvStep nxt = advance(cur);
    if (nxt.item >= 0) stage(nxt, buf ^ 1);
    const int32_t *it = items + cur.item * kItemWords;
    const int k_lo = it[3], k_hi = it[4], q_hi = it[2];
    const int qt0 = cur.qt0;
    const int qt1 = min(qt0 + BQ, q_hi);
    if (has_keys && kw0 < qt1) {
      const __bf16 *Qs = lds + buf * BUF, *dOs = Qs + C::TSZ;
      const bool need_mask = !(kw0 + 31 <= qt0 && kw0 >= k_lo && kw0 + 32 <= k_hi);
      // The 64 query rows are handled as two pairs of 32 (qp), one after the
      // other, to bound the live score registers.
#pragma unroll
      for (int qp = 0; qp < 2; ++qp) {
        // ---- S = Q K^T and dP = dO V^T.  Half ab reads query row
        // 32qp + 8*(m/4) + 4*ab + m%4, so a lane's 8 values of the pair are
        // the rows 32qp + 8*lg + 0..7 for its key 16nk + l16.
        f32x4 s[2][2], dp[2][2];
#pragma unroll
        for (int ab = 0; ab < 2; ++ab)
#pragma unroll
          for (int nk = 0; nk < 2; ++nk) {
            s[ab][nk] = (f32x4){0.f, 0.f, 0.f, 0.f};
            dp[ab][nk] = (f32x4){0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab) {
            const int row = 32 * qp + 8 * (l16 >> 2) + 4 * ab + (l16 & 3);
            const bf16x8 qa = tile_row8<D>(Qs, row, 32 * ks + 8 * lg);
            const bf16x8 da = tile_row8<D>(dOs, row, 32 * ks + 8 * lg);
#pragma unroll
            for (int nk = 0; nk < 2; ++nk) {
              s[ab][nk] = mfma16(qa, kf[nk][ks], s[ab][nk]);
              dp[ab][nk] = mfma16(da, vf[nk][ks], dp[ab][nk]);
            }
          }
        // ---- P and dS
        const f32x4 l0 = *reinterpret_cast<const f32x4 *>(&stat[buf][0][32 * qp + 8 * lg]);
        const f32x4 l1 = *reinterpret_cast<const f32x4 *>(&stat[buf][0][32 * qp + 8 * lg + 4]);
        const f32x4 d0 = *reinterpret_cast<const f32x4 *>(&stat[buf][1][32 * qp + 8 * lg]);
        const f32x4 d1 = *reinterpret_cast<const f32x4 *>(&stat[buf][1][32 * qp + 8 * lg + 4]);
        bf16x8 pa[2], dsa[2];
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) {
          const int key = kw0 + 16 * nk + l16;
          f32x4 p[2], ds[2];
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float lq = ab ? l1[i] : l0[i];
              const float dq = ab ? d1[i] : d0[i];
              float pv = fast_exp2(fmaf(s[ab][nk][i], c2, -lq));
              if (need_mask) {
                const int q = qt0 + 32 * qp + 8 * lg + 4 * ab + i;
                if (key > q || key < k_lo || key >= k_hi) pv = 0.f;
              }
              p[ab][i] = pv;
              ds[ab][i] = pv * (dp[ab][nk][i] - dq);
            }
          pa[nk] = pack_bf16x8(p[0], p[1]);
          dsa[nk] = pack_bf16x8(ds[0], ds[1]);
        }
        // ---- dV += P^T dO, dK += dS^T Q  (B operands read transposed from LDS)
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          const bf16x8 dob = tile_rows8<D>(dOs, 32 * qp, 16 * nt, l16, lg);
          const bf16x8 qb = tile_rows8<D>(Qs, 32 * qp, 16 * nt, l16, lg);
#pragma unroll
          for (int nk = 0; nk < 2; ++nk) {
            dv[nk][nt] = mfma16(pa[nk], dob, dv[nk][nt]);
            dk[nk][nt] = mfma16(dsa[nk], qb, dk[nk][nt]);
          }
        }
      }
    }
    if (nxt.item >= 0) commit(buf ^ 1);
    wait_staged();
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  // ---- epilogue: lane holds rows key = kw0 + 16nk + 4lg + i, column 16nt + l16
  GT *dkg = static_cast<GT *>(a.dk);
  GT *dvg = static_cast<GT *>(a.dv);
#pragma unroll
  for (int nk = 0; nk < 2; ++nk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kw0 + 16 * nk + 4 * lg + i;
      if (has_keys && key < kt1) {
        const int64_t base = ((int64_t)(seq_off + key) * hkv + g) * D + l16;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          put1<GT>(dkg + base + 16 * nt, dk[nk][nt][i] * a.scale, a.accumulate);
          put1<GT>(dvg + base + 16 * nt, dv[nk][nt][i], a.accumulate);
        }
      }
    }
}

// ====================================================================== dQ

struct QStep {
  int item;  // < 0: done
  int kv0;
};

template <int D, typename InT, typename GT>
__global__ __launch_bounds__(256) void dq_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int BN = kBwdQBN;  // 64 keys per tile
  constexpr int BUF = 2 * C::TSZ;  // K tile, V tile
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  int rank, h;
  map_head(blockIdx.x, a.hq, rank, h);
  const int32_t *__restrict__ items = a.items;
  const float *__restrict__ lse = a.lse;
  const float *__restrict__ delta = a.delta;
  const int hq = a.hq, hkv = a.hkv;
  const int32_t *grp = a.qg + find_unit(a.qg, 4, 2, a.n_qg, rank) * 4;
  const int first = grp[0], count = grp[1];
  const int32_t *it0 = items + first * kItemWords;
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

  bf16x8 qf[2][C::KS], dof[2][C::KS];
  float lse2[2], drow[2];
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
    drow[nq] = ok ? delta[(int64_t)h * T + grow] : 0.f;
  }

  f32x4 dq[2][C::NT];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) dq[nq][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // ---- step iterator over (item of the group in reverse order, key tile)
  auto item_end = [&](int i) __attribute__((always_inline)) { return min(items[i * kItemWords + 4], r1); };
  auto first_from = [&](int i) __attribute__((always_inline)) -> QStep {
    for (; i >= first; --i)
      if (item_end(i) > items[i * kItemWords + 3]) return QStep{i, items[i * kItemWords + 3]};
    return QStep{-1, 0};
  };
  auto advance = [&](QStep s) __attribute__((always_inline)) -> QStep {
    s.kv0 += BN;
    if (s.kv0 < item_end(s.item)) return s;
    return first_from(s.item - 1);
  };

  TileLoader<D, InT> lk, lv;
  const int64_t kstride = (int64_t)hkv * D;
  auto stage = [&](const QStep &s, int buf) __attribute__((always_inline)) {
    const int nvalid = min(BN, item_end(s.item) - s.kv0);
    const int64_t off = (((int64_t)seq_off + s.kv0) * hkv + g) * D;
    __bf16 *b = lds + buf * BUF;
    lk.issue(b, kg + off, kstride, nvalid, wave, lane);
    lv.issue(b + C::TSZ, vg + off, kstride, nvalid, wave, lane);
  };
  auto commit = [&](int buf) __attribute__((always_inline)) {
    __bf16 *b = lds + buf * BUF;
    lk.commit(b, tid);
    lv.commit(b + C::TSZ, tid);
  };

  const float c2 = a.scale_log2;
  QStep cur = first_from(first + count - 1);
  if (cur.item >= 0) {
    stage(cur, 0);
    commit(0);
  }
  wait_staged();
  __syncthreads();
  int buf = 0;
  while (cur.item >= 0) {
    const QStep nxt = advance(cur);
    if (nxt.item >= 0) stage(nxt, buf ^ 1);
    const int kv0 = cur.kv0;
    const int k_hi = items[cur.item * kItemWords + 4];
    if (has_rows && kv0 <= rw_end - 1) {
      const __bf16 *Ks = lds + buf * BUF, *Vs = Ks + C::TSZ;
      // ---- S^T = K Q^T, dP^T = V dO^T (key pair kp, half ab as in the forward)
      f32x4 s[2][2][2], dp[2][2][2];
#pragma unroll
      for (int nq = 0; nq < 2; ++nq)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab) {
            s[nq][kp][ab] = (f32x4){0.f, 0.f, 0.f, 0.f};
            dp[nq][kp][ab] = (f32x4){0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab) {
            const int kvr = 32 * kp + 8 * (l16 >> 2) + 4 * ab + (l16 & 3);
            const bf16x8 ka = tile_row8<D>(Ks, kvr, 32 * ks + 8 * lg);
            const bf16x8 va = tile_row8<D>(Vs, kvr, 32 * ks + 8 * lg);
#pragma unroll
            for (int nq = 0; nq < 2; ++nq) {
              s[nq][kp][ab] = mfma16(ka, qf[nq][ks], s[nq][kp][ab]);
              dp[nq][kp][ab] = mfma16(va, dof[nq][ks], dp[nq][kp][ab]);
            }
          }
      const bool need_mask = (kv0 + BN - 1 > rw0) || (kv0 + BN > k_hi);
      bf16x8 dsb[2][2];
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        const int qrow = rw0 + 16 * nq + l16;
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          f32x4 ds[2];
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float pv = fast_exp2(fmaf(s[nq][kp][ab][i], c2, -lse2[nq]));
              if (need_mask) {
                const int key = kv0 + 32 * kp + 8 * lg + 4 * ab + i;
                if (key > qrow || key >= k_hi) pv = 0.f;
              }
              ds[ab][i] = pv * (dp[nq][kp][ab][i] - drow[nq]);
            }
          dsb[nq][kp] = pack_bf16x8(ds[0], ds[1]);
        }
      }
      // ---- dQ^T += K^T dS^T
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const bf16x8 ka = tile_rows8<D>(Ks, 32 * kp, 16 * nt, l16, lg);
#pragma unroll
          for (int nq = 0; nq < 2; ++nq) dq[nq][nt] = mfma16(ka, dsb[nq][kp], dq[nq][nt]);
        }
    }
    if (nxt.item >= 0) commit(buf ^ 1);
    wait_staged();
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  // ---- epilogue: lane holds dQ[row = rw0 + 16nq + l16][16nt + 4lg + i]
  GT *dqg = static_cast<GT *>(a.dq);
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int row = rw0 + 16 * nq + l16;
    if (has_rows && row < r1) {
      GT *p = dqg + (((int64_t)seq_off + row) * hq + h) * D + 4 * lg;
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) put4<GT>(p + 16 * nt, dq[nq][nt] * a.scale, a.accumulate);
    }
  }
}

template <int D, typename InT, typename GT>
static hipError_t launch_dkdv_t(const BwdArgs &a, hipStream_t s) {
  const int64_t grid = (int64_t)a.n_kv_units * a.hkv;
  hipLaunchKernelGGL((dkdv_kernel<D, InT, GT>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, typename InT, typename GT>
static hipError_t launch_dq_t(const BwdArgs &a, hipStream_t s) {
  const int64_t grid = (int64_t)a.n_q_units * a.hq;
  hipLaunchKernelGGL((dq_kernel<D, InT, GT>), dim3((unsigned)grid), dim3(256), 0, s, a);
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

hipError_t launch_bwd_dkdv(const BwdArgs &a, int d, int in_dtype, int g_dtype, hipStream_t s) {
  SEGATTN_DISPATCH(launch_dkdv_t, a, d, in_dtype, g_dtype, s);
}

hipError_t launch_bwd_dq(const BwdArgs &a, int d, int in_dtype, int g_dtype, hipStream_t s) {
  SEGATTN_DISPATCH(launch_dq_t, a, d, in_dtype, g_dtype, s);
}

#undef SEGATTN_DISPATCH

}  // namespace segattn

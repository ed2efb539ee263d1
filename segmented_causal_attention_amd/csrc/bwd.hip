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
//   recomputes S, P, dP, dS and accumulates dV and dK (4 products).
// dq_kernel: query-stationary, like the forward.  A workgroup owns 128 query
//   rows of one head (4 waves x 32 rows; Q and dO in registers) and walks the
//   64-key tiles of every item of its query group; per tile it recomputes
//   S^T, P, dP^T, dS^T and accumulates dQ^T (3 products).
#include "device_common.h"
#include "kernels.h"

namespace segattn {
namespace dev {

template <int D>
struct BwdCfg {
  static constexpr int KS = D / 32;    // depth steps over the head dim
  static constexpr int NT = D / 16;    // 16-wide head-dim tiles
  static constexpr int ROW = D + 8;    // LDS row stride, row-major tiles (bf16)
  static constexpr int TROW = 64 + 8;  // LDS row stride, transposed 64-row tiles (bf16)
  static constexpr int STAGERS = 16 * (D / 8);  // threads staging a 64-row tile (4 rows x 8 dims each)
};

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

// Stages a 64-row tile of a [tokens][heads][D] tensor into LDS both
// row-major (rows x D) and transposed (D x 64 rows).  Each staging thread
// holds 4 consecutive rows x 8 dims.
template <int D, typename InT>
struct TileStager {
  using C = BwdCfg<D>;
  u32x4 r[4];
  __device__ __forceinline__ void load(const InT *base, int64_t row0, int nvalid, int heads, int h, int tid) {
    if (tid < C::STAGERS) {
      const int rq = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * rq + i;
        r[i] = rr < nvalid ? load8<InT>(base + ((row0 + rr) * heads + h) * D + 8 * dc) : (u32x4){0, 0, 0, 0};
      }
    }
  }
  __device__ __forceinline__ void store(__bf16 *rowmajor, __bf16 *trans, int tid) const {
    if (tid < C::STAGERS) {
      const int rq = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4 *>(rowmajor + (4 * rq + i) * C::ROW + 8 * dc) = r[i];
      if (trans) {
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int w = dd >> 1;
          u32x2 pk;
          if (dd & 1) {
            pk[0] = join_hi(r[0][w], r[1][w]);
            pk[1] = join_hi(r[2][w], r[3][w]);
          } else {
            pk[0] = join_lo(r[0][w], r[1][w]);
            pk[1] = join_lo(r[2][w], r[3][w]);
          }
          *reinterpret_cast<u32x2 *>(trans + (8 * dc + dd) * C::TROW + 4 * rq) = pk;
        }
      }
    }
  }
};

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
  constexpr int ROWS = BQ * C::ROW, TRANS = D * C::TROW;
  constexpr int BUF = 2 * ROWS + 2 * TRANS;  // Q, dO row-major + transposed (bf16 elements)
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
    const int64_t base = ((int64_t)(seq_off + (ok ? key : kt0)) * a.hkv + g) * D + 8 * lg;
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
  auto item_sees = [&](int i) {
    const int32_t *it = a.items + i * kItemWords;
    return it[0] == seq_off && it[3] < kt1 && it[4] > kt0 && it[2] > kt0;
  };
  auto first_from = [&](int i) -> KvStep {
    for (; i >= 0; --i)
      if (item_sees(i)) return KvStep{i, 0, max(a.items[i * kItemWords + 1], kt0)};
    return KvStep{-1, 0, 0};
  };
  auto advance = [&](KvStep s) -> KvStep {
    const int32_t *it = a.items + s.item * kItemWords;
    s.qt0 += BQ;
    if (s.qt0 < it[2]) return s;
    if (++s.hh < G) {
      s.qt0 = max(it[1], kt0);
      return s;
    }
    return first_from(s.item - 1);
  };

  TileStager<D, InT> sq, sdo;
  float st_lse = 0.f, st_d = 0.f;
  auto gload = [&](const KvStep &s) {
    const int32_t *it = a.items + s.item * kItemWords;
    const int h = g * G + s.hh;
    const int nvalid = min(BQ, it[2] - s.qt0);
    const int64_t row0 = (int64_t)seq_off + s.qt0;
    sq.load(qg, row0, nvalid, a.hq, h, tid);
    sdo.load(dg, row0, nvalid, a.hq, h, tid);
    if (tid < BQ) {
      if (tid < nvalid) {
        const float l = a.lse[(int64_t)h * T + row0 + tid];
        // A row without visible keys (LSE = -inf) contributes nothing.
        st_lse = l == kNegInf ? __builtin_inff() : l * kLog2e;
        st_d = a.delta[(int64_t)h * T + row0 + tid];
      } else {
        st_lse = __builtin_inff();
        st_d = 0.f;
      }
    }
  };
  auto sstore = [&](int buf) {
    __bf16 *b = lds + buf * BUF;
    sq.store(b, b + 2 * ROWS, tid);
    sdo.store(b + ROWS, b + 2 * ROWS + TRANS, tid);
    if (tid < BQ) {
      stat[buf][0][tid] = st_lse;
      stat[buf][1][tid] = st_d;
    }
  };

  const float c2 = a.scale_log2;
  KvStep cur = first_from(a.n_items - 1);
  if (cur.item >= 0) {
    gload(cur);
    sstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (cur.item >= 0) {
    const KvStep nxt = advance(cur);
    if (nxt.item >= 0) gload(nxt);
    const int32_t *it = a.items + cur.item * kItemWords;
    const int k_lo = it[3], k_hi = it[4], q_hi = it[2];
    const int qt0 = cur.qt0;
    const int qt1 = min(qt0 + BQ, q_hi);
    if (has_keys && kw0 < qt1) {
      const __bf16 *Qs = lds + buf * BUF, *dOs = Qs + ROWS, *Qt = Qs + 2 * ROWS, *dOt = Qt + TRANS;
      // ---- S = Q K^T and dP = dO V^T.  Query pair qp covers rows
      // 32qp..32qp+31; half ab reads row 8*(m/4) + 4*ab + m%4 so a lane's 8
      // values of a pair are the rows 32qp + 8*lg + 0..7 of its key.
      f32x4 s[2][2][2], dp[2][2][2];
#pragma unroll
      for (int qp = 0; qp < 2; ++qp)
#pragma unroll
        for (int ab = 0; ab < 2; ++ab)
#pragma unroll
          for (int nk = 0; nk < 2; ++nk) {
            s[qp][ab][nk] = (f32x4){0.f, 0.f, 0.f, 0.f};
            dp[qp][ab][nk] = (f32x4){0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int qp = 0; qp < 2; ++qp)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab) {
            const int row = 32 * qp + 8 * (l16 >> 2) + 4 * ab + (l16 & 3);
            const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(Qs + row * C::ROW + 32 * ks + 8 * lg);
            const bf16x8 da = *reinterpret_cast<const bf16x8 *>(dOs + row * C::ROW + 32 * ks + 8 * lg);
#pragma unroll
            for (int nk = 0; nk < 2; ++nk) {
              s[qp][ab][nk] = mfma16(qa, kf[nk][ks], s[qp][ab][nk]);
              dp[qp][ab][nk] = mfma16(da, vf[nk][ks], dp[qp][ab][nk]);
            }
          }
      // ---- P and dS (lane: key 16nk + l16, rows 32qp + 8lg + j)
      const bool need_mask = !(kw0 + 31 <= qt0 && kw0 >= k_lo && kw0 + 32 <= k_hi);
      bf16x8 pa[2][2], dsa[2][2];
#pragma unroll
      for (int qp = 0; qp < 2; ++qp) {
        const f32x4 l0 = *reinterpret_cast<const f32x4 *>(&stat[buf][0][32 * qp + 8 * lg]);
        const f32x4 l1 = *reinterpret_cast<const f32x4 *>(&stat[buf][0][32 * qp + 8 * lg + 4]);
        const f32x4 d0 = *reinterpret_cast<const f32x4 *>(&stat[buf][1][32 * qp + 8 * lg]);
        const f32x4 d1 = *reinterpret_cast<const f32x4 *>(&stat[buf][1][32 * qp + 8 * lg + 4]);
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
              float pv = fast_exp2(fmaf(s[qp][ab][nk][i], c2, -lq));
              if (need_mask) {
                const int q = qt0 + 32 * qp + 8 * lg + 4 * ab + i;
                if (key > q || key < k_lo || key >= k_hi) pv = 0.f;
              }
              p[ab][i] = pv;
              ds[ab][i] = pv * (dp[qp][ab][nk][i] - dq);
            }
          pa[qp][nk] = pack_bf16x8(p[0], p[1]);
          dsa[qp][nk] = pack_bf16x8(ds[0], ds[1]);
        }
      }
      // ---- dV += P^T dO, dK += dS^T Q  (B operands from the transposed tiles)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
          const bf16x8 dob = *reinterpret_cast<const bf16x8 *>(dOt + (16 * nt + l16) * C::TROW + 32 * qp + 8 * lg);
          const bf16x8 qb = *reinterpret_cast<const bf16x8 *>(Qt + (16 * nt + l16) * C::TROW + 32 * qp + 8 * lg);
#pragma unroll
          for (int nk = 0; nk < 2; ++nk) {
            dv[nk][nt] = mfma16(pa[qp][nk], dob, dv[nk][nt]);
            dk[nk][nt] = mfma16(dsa[qp][nk], qb, dk[nk][nt]);
          }
        }
    }
    if (nxt.item >= 0) sstore(buf ^ 1);
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
        const int64_t base = ((int64_t)(seq_off + key) * a.hkv + g) * D + l16;
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
  constexpr int ROWS = BN * C::ROW, TRANS = D * C::TROW;
  constexpr int BUF = 2 * ROWS + TRANS;  // K, V row-major + K transposed
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  int rank, h;
  map_head(blockIdx.x, a.hq, rank, h);
  const int32_t *grp = a.qg + find_unit(a.qg, 4, 2, a.n_qg, rank) * 4;
  const int first = grp[0], count = grp[1];
  const int32_t *it0 = a.items + first * kItemWords;
  const int seq_off = it0[0], q_lo = it0[1], q_hi = it0[2];
  const int r1 = q_hi - (rank - grp[2]) * kBwdQBM;
  const int r0 = max(q_lo, r1 - kBwdQBM);
  const int g = h / (a.hq / a.hkv);
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
    const int64_t base = (grow * a.hq + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[nq][ks] = __builtin_bit_cast(bf16x8, ok ? load8<InT>(qg + base + 32 * ks) : (u32x4){0, 0, 0, 0});
      dof[nq][ks] = __builtin_bit_cast(bf16x8, ok ? load8<InT>(dg + base + 32 * ks) : (u32x4){0, 0, 0, 0});
    }
    const float l = ok ? a.lse[(int64_t)h * T + grow] : kNegInf;
    lse2[nq] = l == kNegInf ? __builtin_inff() : l * kLog2e;
    drow[nq] = ok ? a.delta[(int64_t)h * T + grow] : 0.f;
  }

  f32x4 dq[2][C::NT];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) dq[nq][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // ---- step iterator over (item of the group in reverse order, key tile)
  auto item_end = [&](int i) { return min(a.items[i * kItemWords + 4], r1); };
  auto first_from = [&](int i) -> QStep {
    for (; i >= first; --i)
      if (item_end(i) > a.items[i * kItemWords + 3]) return QStep{i, a.items[i * kItemWords + 3]};
    return QStep{-1, 0};
  };
  auto advance = [&](QStep s) -> QStep {
    s.kv0 += BN;
    if (s.kv0 < item_end(s.item)) return s;
    return first_from(s.item - 1);
  };

  TileStager<D, InT> sk, sv;
  auto gload = [&](const QStep &s) {
    const int nvalid = min(BN, item_end(s.item) - s.kv0);
    const int64_t row0 = (int64_t)seq_off + s.kv0;
    sk.load(kg, row0, nvalid, a.hkv, g, tid);
    sv.load(vg, row0, nvalid, a.hkv, g, tid);
  };
  auto sstore = [&](int buf) {
    __bf16 *b = lds + buf * BUF;
    sk.store(b, b + 2 * ROWS, tid);
    sv.store(b + ROWS, nullptr, tid);
  };

  const float c2 = a.scale_log2;
  QStep cur = first_from(first + count - 1);
  if (cur.item >= 0) {
    gload(cur);
    sstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (cur.item >= 0) {
    const QStep nxt = advance(cur);
    if (nxt.item >= 0) gload(nxt);
    const int kv0 = cur.kv0;
    const int k_hi = a.items[cur.item * kItemWords + 4];
    if (has_rows && kv0 <= rw_end - 1) {
      const __bf16 *Ks = lds + buf * BUF, *Vs = Ks + ROWS, *Kt = Ks + 2 * ROWS;
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
            const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(Ks + kvr * C::ROW + 32 * ks + 8 * lg);
            const bf16x8 va = *reinterpret_cast<const bf16x8 *>(Vs + kvr * C::ROW + 32 * ks + 8 * lg);
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
          const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(Kt + (16 * nt + l16) * C::TROW + 32 * kp + 8 * lg);
#pragma unroll
          for (int nq = 0; nq < 2; ++nq) dq[nq][nt] = mfma16(ka, dsb[nq][kp], dq[nq][nt]);
        }
    }
    if (nxt.item >= 0) sstore(buf ^ 1);
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
      GT *p = dqg + (((int64_t)seq_off + row) * a.hq + h) * D + 4 * lg;
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

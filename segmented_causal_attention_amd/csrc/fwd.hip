// Forward partial attention kernel for gfx950 (CDNA4), bf16 MFMA.
//
// One workgroup = one query tile of up to 256 rows of one work item and one
// query head (4 waves x 64 rows).  The item's visible keys are streamed in
// 64-key tiles staged through LDS (K row-major, V transposed, double
// buffered) while the query rows stay in registers.  Scores are computed
// transposed, S^T = K Q^T, so that every lane owns one query row's scores:
// the row max and the row sum of the online softmax then need only two
// cross-lane steps, and the probabilities are already in the B-operand layout
// of the second product O^T += V^T P^T.
//
// What it computes (SPPO section 5.1 / Figure 9: a segment's queries against
// the resident K/V of all segments up to it; InfiniPipe section II-A: one
// step of the multi-step online self-attention): for each query row q of the
// item, over the visible keys j (k_lo <= j < k_hi, j <= q),
//   LSE_q = log sum_j exp(scale <Q_q, K_j>),   O_q = sum_j exp(scale <Q_q,K_j> - LSE_q) V_j,
// optionally merged into an existing fp32 (O, LSE) with the log-sum-exp rule.
#include "device_common.h"
#include "kernels.h"

namespace segattn {
namespace dev {

template <int D>
struct FwdCfg {
  static constexpr int BM = kFwdBM;        // query rows per workgroup
  static constexpr int BN = kFwdBN;        // keys per LDS tile
  static constexpr int NQ = 4;             // 16-row subtiles per wave (64 rows)
  static constexpr int KS = D / 32;        // depth steps of K Q^T
  static constexpr int MT = D / 16;        // 16-wide head-dim tiles of O^T
  static constexpr int KP = BN / 32;       // 32-key pairs per tile
  static constexpr int KROW = D + 8;       // LDS K row stride (bf16)
  static constexpr int VROW = BN + 8;      // LDS V^T row stride (bf16)
  static constexpr int KSZ = BN * KROW;
  static constexpr int VSZ = D * VROW;
  static constexpr int BUF = KSZ + VSZ;
  static constexpr int KCH = BN * D / 8 / 256;    // 16-byte K chunks per thread
  static constexpr int VBLK = (BN / 4) * (D / 8); // 4-key x 8-dim V blocks
};

// Workgroup index -> (tile rank, head).  Consecutive workgroups go to the 8
// XCDs in turn; when hq is a multiple of 8, XCD c gets the heads
// [c*hq/8, (c+1)*hq/8) so the workgroups sharing an XCD's L2 read the same
// K/V, while every XCD still receives the tile ranks heaviest-first.
__device__ __forceinline__ void map_unit(int x, int hq, int &rank, int &h) {
  if ((hq & 7) == 0) {
    const int hpx = hq >> 3, xcd = x & 7, j = x >> 3;
    rank = j / hpx;
    h = xcd * hpx + j % hpx;
  } else {
    rank = x / hq;
    h = x % hq;
  }
}

// Index of the item whose unit range holds `rank` (unit_begin ascending).
__device__ __forceinline__ int find_item(const int32_t *items, int n, int rank) {
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
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * C::BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  int rank, h;
  map_unit(blockIdx.x, a.hq, rank, h);
  const int32_t *it = a.items + find_item(a.items, a.n_items, rank) * kItemWords;
  const int seq_off = it[0], q_lo = it[1], q_hi = it[2], k_lo = it[3], k_hi = it[4];
  const int tile = rank - it[5];
  const int r1 = q_hi - tile * C::BM;             // heaviest (last) rows first
  const int r0 = max(q_lo, r1 - C::BM);
  const int g = (h * a.hkv) / a.hq;
  const int64_t T = a.tokens;

  const InT *__restrict__ qg = static_cast<const InT *>(a.q);
  const InT *__restrict__ kg = static_cast<const InT *>(a.k);
  const InT *__restrict__ vg = static_cast<const InT *>(a.v);

  // This wave's query rows [rw0, rw_end).
  const int rw0 = r0 + 64 * wave;
  const int rw_end = min(rw0 + 64, r1);
  const bool has_rows = rw0 < rw_end;
  const int rw_max = rw_end - 1;

  // Query fragments (B operand of K Q^T): lane holds Q[row = l16][8*lg .. +8].
  bf16x8 qf[C::NQ][C::KS];
#pragma unroll
  for (int nq = 0; nq < C::NQ; ++nq) {
    const int row = rw0 + 16 * nq + l16;
    const bool ok = has_rows && row < r1;
    const InT *qp = qg + ((int64_t)(seq_off + (ok ? row : r0)) * a.hq + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 w = ok ? load8<InT>(qp + 32 * ks) : (u32x4){0, 0, 0, 0};
      qf[nq][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kb = k_lo;
  const int ke = min(k_hi, r1);
  const int ntiles = ke > kb ? (ke - kb + C::BN - 1) / C::BN : 0;

  float m_run[C::NQ], l_run[C::NQ];
  f32x4 o[C::NQ][C::MT];
#pragma unroll
  for (int nq = 0; nq < C::NQ; ++nq) {
    m_run[nq] = kNegInf;
    l_run[nq] = 0.f;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) o[nq][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // Global -> register staging of one K/V tile starting at key kvs.
  u32x4 kreg[C::KCH], vreg[4];
  auto gload = [&](int kvs) {
#pragma unroll
    for (int r = 0; r < C::KCH; ++r) {
      const int c = tid + 256 * r, row = c / (D / 8), cc = c % (D / 8);
      const int kr = kvs + row;
      kreg[r] = kr < ke ? load8<InT>(kg + ((int64_t)(seq_off + kr) * a.hkv + g) * D + 8 * cc)
                        : (u32x4){0, 0, 0, 0};
    }
    if (tid < C::VBLK) {
      const int kvq = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = kvs + 4 * kvq + r;
        vreg[r] = kr < ke ? load8<InT>(vg + ((int64_t)(seq_off + kr) * a.hkv + g) * D + 8 * dc)
                          : (u32x4){0, 0, 0, 0};
      }
    }
  };
  // Register -> LDS: K row-major, V transposed (V^T[d][key]).
  auto sstore = [&](int buf) {
    __bf16 *Ks = lds + buf * C::BUF;
    __bf16 *Vt = Ks + C::KSZ;
#pragma unroll
    for (int r = 0; r < C::KCH; ++r) {
      const int c = tid + 256 * r, row = c / (D / 8), cc = c % (D / 8);
      *reinterpret_cast<u32x4 *>(Ks + row * C::KROW + 8 * cc) = kreg[r];
    }
    if (tid < C::VBLK) {
      const int kvq = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1;
        u32x2 pk;
        if (dd & 1) {
          pk[0] = join_hi(vreg[0][w], vreg[1][w]);
          pk[1] = join_hi(vreg[2][w], vreg[3][w]);
        } else {
          pk[0] = join_lo(vreg[0][w], vreg[1][w]);
          pk[1] = join_lo(vreg[2][w], vreg[3][w]);
        }
        *reinterpret_cast<u32x2 *>(Vt + (8 * dc + dd) * C::VROW + 4 * kvq) = pk;
      }
    }
  };

  const float c2 = a.scale_log2;

  if (ntiles > 0) {
    gload(kb);
    sstore(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = kb + j * C::BN;
    if (j + 1 < ntiles) gload(kv0 + C::BN);
    const __bf16 *Ks = lds + (j & 1) * C::BUF;
    const __bf16 *Vt = Ks + C::KSZ;

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
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab) {
            const int kvr = 32 * kp + 8 * (l16 >> 2) + 4 * ab + (l16 & 3);
            const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + kvr * C::KROW + 32 * ks + 8 * lg);
#pragma unroll
            for (int nq = 0; nq < C::NQ; ++nq) s[nq][kp][ab] = mfma16(kf, qf[nq][ks], s[nq][kp][ab]);
          }
      }

      // ---- online softmax (base 2), one query row per lane and subtile.
      const bool need_mask = (kv0 + C::BN - 1 > rw0) || (kv0 + C::BN > k_hi);
      bf16x8 pf[C::NQ][C::KP];
#pragma unroll
      for (int nq = 0; nq < C::NQ; ++nq) {
        const int qrow = rw0 + 16 * nq + l16;
        float mx = kNegInf;
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float val = s[nq][kp][ab][i];
              if (need_mask) {
                const int kv = kv0 + 32 * kp + 8 * lg + 4 * ab + i;
                if (kv > qrow || kv >= k_hi) val = kNegInf;
                s[nq][kp][ab][i] = val;
              }
              mx = fmaxf(mx, val);
            }
        mx = wave_max_xor16_32(mx);
        const float m_new = fmaxf(m_run[nq], mx * c2);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[nq] - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp)
#pragma unroll
          for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p = fast_exp2(fmaf(s[nq][kp][ab][i], c2, -m_use));
              s[nq][kp][ab][i] = p;
              rs += p;
            }
        l_run[nq] = fmaf(l_run[nq], alpha, rs);
        m_run[nq] = m_new;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) o[nq][mt] *= alpha;
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp) pf[nq][kp] = pack_bf16x8(s[nq][kp][0], s[nq][kp][1]);
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int kp = 0; kp < C::KP; ++kp) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8 *>(Vt + (16 * mt + l16) * C::VROW + 32 * kp + 8 * lg);
#pragma unroll
          for (int nq = 0; nq < C::NQ; ++nq) o[nq][mt] = mfma16(vf, pf[nq][kp], o[nq][mt]);
        }
    }

    if (j + 1 < ntiles) sstore((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, optional merge, write O rows and LSE.
  OutT *__restrict__ og = static_cast<OutT *>(a.o);
#pragma unroll
  for (int nq = 0; nq < C::NQ; ++nq) {
    const float lt = wave_sum_xor16_32(l_run[nq]);
    const int qrow = rw0 + 16 * nq + l16;
    const bool valid = has_rows && qrow < r1;
    const float lse_new = lt > 0.f ? (m_run[nq] + fast_log2(lt)) * kLn2 : kNegInf;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
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
      OutT *op = og + (grow * a.hq + h) * D + 4 * lg;
      const float sc = inv * w_new;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        f32x4 val = o[nq][mt] * sc;
        if constexpr (sizeof(OutT) == 4) {
          if (a.merge) val += *reinterpret_cast<const f32x4 *>(op + 16 * mt) * w_old;
        }
        store4<OutT>(op + 16 * mt, val);
      }
      if (lg == 0) a.lse[(int64_t)h * T + grow] = lse_out;
    }
  }
}

template <int D, typename InT, typename OutT>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t s) {
  const int64_t grid = (int64_t)a.n_units * a.hq;
  hipLaunchKernelGGL((fwd_kernel<D, InT, OutT>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dev

hipError_t launch_fwd(const FwdArgs &a, int d, int in_dtype, int o_dtype, hipStream_t s) {
  using namespace dev;
  const bool in_bf = in_dtype == 0, out_bf = o_dtype == 0;
  if (d == 128) {
    if (in_bf) return out_bf ? launch_fwd_t<128, __bf16, __bf16>(a, s) : launch_fwd_t<128, __bf16, float>(a, s);
    return out_bf ? launch_fwd_t<128, float, __bf16>(a, s) : launch_fwd_t<128, float, float>(a, s);
  }
  if (in_bf) return out_bf ? launch_fwd_t<64, __bf16, __bf16>(a, s) : launch_fwd_t<64, __bf16, float>(a, s);
  return out_bf ? launch_fwd_t<64, float, __bf16>(a, s) : launch_fwd_t<64, float, float>(a, s);
}

}  // namespace segattn

// Memory-bound kernels: log-sum-exp merge of partial results, the backward
// row reduction D = <dO, O>, and the stream-ordered table upload; and the
// device array behind segattn_bwd_noalloc.
#include <mutex>

#include "device_common.h"
#include "kernels.h"
#include "segattn.h"

namespace segattn {
namespace dev {

// ---------------------------------------------------------------- merge
// Softmax over a disjoint union of key sets A and B (InfiniPipe section II-A:
// the ring's partial results are combined by online self-attention):
//   m = max(l_a, l_b);  m = -inf -> (0, -inf);  w = e^(l - m);
//   LSE = m + log(w_a + w_b),  O = (w_a O_a + w_b O_b) / (w_a + w_b).
// One thread per 4 consecutive floats of a (row, head) vector; the d/4
// threads of one vector sit in one wavefront, which issues all its loads
// before any store, so an in-place merge reads the old LSE in every lane
// before a lane overwrites it.  A workgroup takes kMergeUnroll groups of
// 256/(d/4) consecutive vectors with all their loads in flight at once; the
// only 64-bit division is one per workgroup.  The O vectors are read and
// written once, so their loads and stores carry the nontemporal hint (5.77
// instead of 5.34 TB/s on 131072 x 32 x 128 partials); the LSE entries,
// 4 bytes per vector spread over the heads' rows, keep the default policy.
constexpr int kMergeUnroll = 4;

__device__ __forceinline__ void merge_one(const MergeArgs &a, int64_t vec, int64_t li, int c, const f32x4 &oa,
                                          const f32x4 &ob, float la, float lb) {
  const float m = fmaxf(la, lb);
  f32x4 out = {0.f, 0.f, 0.f, 0.f};
  float lse = kNegInf;
  if (m != kNegInf) {
    const float wa = fast_exp2((la - m) * kLog2e), wb = fast_exp2((lb - m) * kLog2e);
    const float den = wa + wb, inv = 1.f / den;
    out = oa * (wa * inv) + ob * (wb * inv);
    lse = m + fast_log2(den) * kLn2;
  }
  __builtin_nontemporal_store(out, reinterpret_cast<f32x4 *>(a.o_out + vec * a.d + 4 * c));
  if (c == 0) a.lse_out[li] = lse;
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int CPV = D / 4, VPB = 256 / CPV, U = kMergeUnroll;
  const int tid = threadIdx.x, c = tid % CPV, vl = tid / CPV;
  const int64_t nvec = a.rows * a.h;
  const int64_t nblk = (nvec + VPB * U - 1) / (VPB * U);
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
  const int64_t vbase = blk * (VPB * U);
  const int64_t r0 = vbase / a.h;
  const int hh0 = (int)(vbase - r0 * a.h);
  f32x4 oa[U], ob[U];
  float la[U], lb[U];
  int64_t li[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int v = u * VPB + vl;
    const int t = hh0 + v;
    const int64_t vec = vbase + v;
    li[u] = (int64_t)(t % a.h) * a.lse_stride + r0 + t / a.h;
    if (vec < nvec) {
      oa[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.o_a + vec * D + 4 * c));
      ob[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.o_b + vec * D + 4 * c));
      la[u] = a.lse_a[li[u]];
      lb[u] = a.lse_b[li[u]];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t vec = vbase + u * VPB + vl;
    if (vec < nvec) merge_one(a, vec, li[u], c, oa[u], ob[u], la[u], lb[u]);
  }
  }
}

// Any other d (a multiple of 4, at most 1024): a workgroup takes whole
// vectors, 256/(d/4) of them per pass, so all threads of a vector load
// before a barrier and store after it (in-place safe).
__global__ __launch_bounds__(256) void merge_kernel_any(MergeArgs a) {
  const int cpv = a.d >> 2, vpb = 256 / cpv;
  const int tid = threadIdx.x, vl = tid / cpv, c = tid - vl * cpv;
  const int64_t nvec = a.rows * a.h;
  for (int64_t vb = (int64_t)blockIdx.x * vpb; vb < nvec; vb += (int64_t)gridDim.x * vpb) {
    const int64_t vec = vb + vl;
    const bool ok = vl < vpb && vec < nvec;
    const int64_t r = ok ? vec / a.h : 0;
    const int64_t li = ok ? (vec - r * a.h) * a.lse_stride + r : 0;
    f32x4 oa = {0.f, 0.f, 0.f, 0.f}, ob = oa;
    float la = kNegInf, lb = kNegInf;
    if (ok) {
      oa = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.o_a + vec * a.d + 4 * c));
      ob = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.o_b + vec * a.d + 4 * c));
      la = a.lse_a[li];
      lb = a.lse_b[li];
    }
    __syncthreads();
    if (ok) merge_one(a, vec, li, c, oa, ob, la, lb);
    __syncthreads();
  }
}

// ------------------------------------------------------------- D = <dO, O>
// Rows [r0, r1) of one q unit of the items' q groups, one query head: d/8
// threads per row, one 8-element chunk each, reduced with xor shuffles
// inside the wavefront.
template <int D, typename OT, typename GT>
__global__ __launch_bounds__(256) void bwd_pre_kernel(PreArgs a) {
  constexpr int CPR = D / 8;      // chunks per row: 16 or 8
  constexpr int RPP = 256 / CPR;  // rows per pass
  const int x = blockIdx.x, rank = x / a.hq, h = x - rank * a.hq;
  int lo = 0, hi = a.n_qg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qg[mid * 4 + 2] <= rank)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int32_t *grp = a.qg + lo * 4;
  const int32_t *it = a.items + grp[0] * kItemWords;
  const int seq_off = it[0], q_lo = it[1], q_hi = it[2];
  const int r1 = q_hi - (rank - grp[2]) * kBwdQBM, r0 = max(q_lo, r1 - kBwdQBM);
  const int c = threadIdx.x % CPR;
  const OT *og = static_cast<const OT *>(a.o);
  const GT *dg = static_cast<const GT *>(a.d_o);
  for (int r = r0 + (int)threadIdx.x / CPR; r < r1; r += RPP) {
    const int64_t row = ((int64_t)seq_off + r) * a.hq + h;
    const OT *op = og + row * D + 8 * c;
    const GT *gp = dg + row * D + 8 * c;
    float ov[8], gv[8];
    if constexpr (sizeof(OT) == 4) {
      const f32x4 x0 = *reinterpret_cast<const f32x4 *>(op), x1 = *reinterpret_cast<const f32x4 *>(op + 4);
      for (int i = 0; i < 4; ++i) { ov[i] = x0[i]; ov[4 + i] = x1[i]; }
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4 *>(op);
      for (int i = 0; i < 4; ++i) { ov[2 * i] = bf16_lo(w[i]); ov[2 * i + 1] = bf16_hi(w[i]); }
    }
    if constexpr (sizeof(GT) == 4) {
      const f32x4 x0 = *reinterpret_cast<const f32x4 *>(gp), x1 = *reinterpret_cast<const f32x4 *>(gp + 4);
      for (int i = 0; i < 4; ++i) { gv[i] = x0[i]; gv[4 + i] = x1[i]; }
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4 *>(gp);
      for (int i = 0; i < 4; ++i) { gv[2 * i] = bf16_lo(w[i]); gv[2 * i + 1] = bf16_hi(w[i]); }
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(ov[i], gv[i], acc);
#pragma unroll
    for (int off = CPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (c == 0) a.delta[(int64_t)h * a.tokens + seq_off + r] = -acc;  // negated: the start value of dP
  }
}

// ---------------------------------------------------------------- upload
constexpr int kUploadWords = 1000;  // 4 KB of kernel arguments per launch
struct UploadChunk {
  int32_t n;
  int32_t pad;
  int32_t w[kUploadWords];
};

__global__ __launch_bounds__(1024) void upload_kernel(int32_t *dst, UploadChunk c) {
  const int i = threadIdx.x;
  if (i < c.n) dst[i] = c.w[i];
}

static unsigned grid_for(int64_t work, int64_t per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > 256 * 64) g = 256 * 64;  // grid-stride beyond 64 workgroups per CU
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace dev

hipError_t launch_merge(const MergeArgs &a, hipStream_t s) {
  using namespace dev;
  const int64_t nvec = a.rows * a.h;
  if (a.d == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid_for(nvec, (256 / 32) * kMergeUnroll)), dim3(256), 0, s, a);
  } else if (a.d == 64) {
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid_for(nvec, (256 / 16) * kMergeUnroll)), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(merge_kernel_any, dim3(grid_for(nvec, 256 / (a.d / 4))), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const PreArgs &a, int d, int o_dtype, int in_dtype, hipStream_t s) {
  using namespace dev;
  const dim3 grid((unsigned)((int64_t)a.n_q_units * a.hq)), block(256);
  const bool ob = o_dtype == 0, gb = in_dtype == 0;
#define SEGATTN_PRE(DD, OT, GT) hipLaunchKernelGGL((bwd_pre_kernel<DD, OT, GT>), grid, block, 0, s, a)
  if (d == 128) {
    if (ob) { if (gb) SEGATTN_PRE(128, __bf16, __bf16); else SEGATTN_PRE(128, __bf16, float); }
    else { if (gb) SEGATTN_PRE(128, float, __bf16); else SEGATTN_PRE(128, float, float); }
  } else {
    if (ob) { if (gb) SEGATTN_PRE(64, __bf16, __bf16); else SEGATTN_PRE(64, __bf16, float); }
    else { if (gb) SEGATTN_PRE(64, float, __bf16); else SEGATTN_PRE(64, float, float); }
  }
#undef SEGATTN_PRE
  return hipGetLastError();
}

// ---------------------------------------------------- no-allocation scratch
// segattn_bwd_noalloc keeps the backward's D and plan tables here instead of
// in a caller's workspace.  Host code never passes the array's name to a
// kernel (on the host it only names a stand-in): each device's address of
// it is taken once with hipGetSymbolAddress, with that device current, and
// kept in scratch_addr[].
static __device__ __align__(256) char scratch[SEGATTN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **out) {
  *out = nullptr;
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void *p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return hipSuccess;
}

hipError_t launch_upload(int32_t *dst, const int32_t *words, int64_t n, hipStream_t s) {
  using namespace dev;
  for (int64_t off = 0; off < n; off += kUploadWords) {
    UploadChunk c;
    c.n = (int32_t)((n - off) < kUploadWords ? (n - off) : kUploadWords);
    c.pad = 0;
    for (int i = 0; i < c.n; ++i) c.w[i] = words[off + i];
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(1024), 0, s, dst + off, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace segattn

// 64-row bf16 tiles in LDS shared by the forward and backward kernels.
//
// Layout: row-major, D columns, no padding.  The 16-byte chunk c of row r is
// stored at chunk position c ^ swz(r).  The swizzle spreads, over the 32 LDS
// banks, both read patterns the kernels use:
//   * 16-byte row reads (MFMA operands contracted over the head dim) whose
//     16 lanes visit rows 8a + b (a, b = 0..3): swz takes each value twice;
//   * 8-byte transposing reads (operands contracted over rows) whose 16 lanes
//     visit rows 8*lg + b.
// Without padding a wavefront can fill 1 KB of a tile with one
// global_load_lds_dwordx4 (global memory straight to LDS, no registers).
#pragma once

#include "device_common.h"

namespace segattn {
namespace dev {

constexpr int kTileRows = 64;

__device__ __forceinline__ int swz(int r) { return (r & 3) | ((r >> 1) & 4); }

// Element offset of (row r, column col) in a swizzled tile; col % 4 == 0.
template <int D>
__device__ __forceinline__ int toff(int r, int col) {
  return r * D + (((col >> 3) ^ swz(r)) << 3) + (col & 7);
}

// 16-byte read: tile[r][col .. col+7] (col % 8 == 0).
template <int D>
__device__ __forceinline__ bf16x8 tile_row8(const __bf16 *t, int r, int col) {
  return *reinterpret_cast<const bf16x8 *>(t + toff<D>(r, col));
}

// Operand of a contraction over ROWS: lane l receives
// tile[row0 + 8*(l/16) + j][col0 + l%16], j = 0..7.  ds_read_b64_tr_b16
// hands lane i of each 16-lane group element i%4 of the 8 bytes loaded by
// lane 4k + i/4 as its k-th value, so lane j points at row
// row0 + 8*(l/16) + j/4, columns col0 + 4*(j%4) .. +3 (col0 % 16 == 0).
template <int D>
__device__ __forceinline__ bf16x8 tile_rows8(const __bf16 *t, int row0, int col0, int l16, int lg) {
  const int r = row0 + 8 * lg + (l16 >> 2), c = col0 + 4 * (l16 & 3);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t + toff<D>(r, c)));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(t + toff<D>(r + 4, c)));
  return __builtin_bit_cast(bf16x8, (s16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
}

// Stages a 64-row tile of a token-major tensor into LDS.  Rows >= nvalid
// are filled from row nvalid-1 (bf16 path) or with zeros (fp32 path); the
// kernels mask them, they only need to be finite.
//   src: first row of the tile; stride: elements between consecutive rows.
// bf16: issue() starts direct global->LDS copies (each of the 4 waves copies
//   16 rows); the caller waits for them (vmcnt) before the barrier that
//   publishes the tile.  commit() does nothing.
// fp32: issue() loads into registers, commit() rounds to bf16 and stores.
template <int D, typename InT>
struct TileLoader;

template <int D>
struct TileLoader<D, __bf16> {
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;  // rows per wavefront instruction
  __device__ __forceinline__ void issue(__bf16 *tile, const __bf16 *src, int64_t stride, int nvalid, int wave,
                                        int lane) {
#pragma unroll
    for (int t = 0; t < 16 / RPI; ++t) {
      const int rb = wave * 16 + t * RPI;  // first row of this instruction (uniform)
      const int r = rb + lane / CPR;
      const int c = (lane % CPR) ^ swz(r);
      const int gr = max(0, min(r, nvalid - 1));
      __builtin_amdgcn_global_load_lds((const void *)(src + gr * stride + 8 * c),
                                       (__attribute__((address_space(3))) void *)(tile + rb * D), 16, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(__bf16 *, int) const {}
};

template <int D>
struct TileLoader<D, float> {
  static constexpr int CPR = D / 8;
  static constexpr int N = 64 * CPR / 256;  // chunks per thread
  u32x4 r_[N];
  __device__ __forceinline__ void issue(__bf16 *, const float *src, int64_t stride, int nvalid, int wave, int lane) {
    const int tid = wave * 64 + lane;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = tid + 256 * i, row = ch / CPR, c = ch % CPR;
      r_[i] = row < nvalid ? load8<float>(src + row * stride + 8 * c) : (u32x4){0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void commit(__bf16 *tile, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = tid + 256 * i, row = ch / CPR, c = ch % CPR;
      *reinterpret_cast<u32x4 *>(tile + toff<D>(row, 8 * c)) = r_[i];
    }
  }
};

// Waits for this wavefront's outstanding memory operations (including the
// direct global->LDS copies) before a barrier publishes a staged tile.
__device__ __forceinline__ void wait_staged() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace dev
}  // namespace segattn

// 64-row bf16 tiles in LDS shared by the forward and backward kernels.
//
// Layout: row-major, D columns, no padding; the 16-byte chunk c of row r is
// stored at chunk position c ^ swz<KIND>(r).  gfx950's LDS has 64 four-byte
// banks (a 256-byte row of a D = 128 tile spans all of them), and each tile is
// stored in the layout that suits the way the kernels read it:
//   KIND 0 (row tiles) -- 16-byte row reads of MFMA operands contracted over
//     the head dim; lanes visit rows 8a + b (a, b = 0..3) at one logical
//     chunk.  swz = (r & 3) | ((r >> 3) & 3) << 2.
//   KIND 1 (column tiles) -- 8-byte transposing reads of operands contracted
//     over rows; each half-wavefront visits rows 8g + b of g in {0,1} (or
//     {2,3}), two chunks each, and needs eight disjoint 32-byte bank windows.
//     swz = ((r >> 3) & 1) << 3 | (r & 3) << 1 | (r >> 4) & 1.
// Both were measured bank-conflict free on the device (SQ_LDS_BANK_CONFLICT);
// each is 2-way conflicted under the other access, so a tensor read both ways
// is staged twice.  For D = 64 (8 chunks per row) the swizzle is taken mod 8.
// Without padding a wavefront fills 1 KB of a tile with one
// global_load_lds_dwordx4 (global memory straight to LDS, no registers).
//
// The per-lane byte offsets of every read are loop invariant; kernels compute
// them once (row_read_off / col_read_off) and add compile-time immediates for
// the pair, half and buffer indices (the swizzles ignore row bits 2 and 5).
#pragma once

#include "device_common.h"

namespace segattn {
namespace dev {

constexpr int kTileRows = 64;

constexpr int kRowTile = 0;  // read with 16-byte row reads
constexpr int kColTile = 1;  // read with 8-byte transposing reads

template <int D, int KIND>
__device__ __forceinline__ int swz(int r) {
  const int f = KIND == kRowTile ? ((r & 3) | (((r >> 3) & 3) << 2))
                                 : ((((r >> 3) & 1) << 3) | ((r & 3) << 1) | ((r >> 4) & 1));
  return f & (D / 8 - 1);
}

// Byte offset, inside a tile of the given kind, of the 16-byte chunk c of row r.
template <int D, int KIND>
__device__ __forceinline__ int chunk_off(int r, int c) {
  return r * (2 * D) + ((c ^ swz<D, KIND>(r)) << 4);
}

// Row reads.  Lane (l16, lg) of step ks reads 8 consecutive columns of row
// rho(l16) = 8*(l16/4) + l16%4 (plus a multiple of 4 rows added as an
// immediate, which leaves f unchanged) at logical chunk 4*ks + lg.
// Returns the byte offset for step ks.
template <int D>
__device__ __forceinline__ int row_read_off(int ks, int l16, int lg) {
  const int r = 8 * (l16 >> 2) + (l16 & 3);
  return chunk_off<D, kRowTile>(r, 4 * ks + lg);
}

// Transposing reads.  For column block mt (16 columns) lane (l16, lg) points
// at row 8*lg + l16/4 (plus multiples of 4 rows as immediates), columns
// 16*mt + 4*(l16%4) .. +3.  Returns the byte offset.
template <int D>
__device__ __forceinline__ int col_read_off(int mt, int l16, int lg) {
  const int r = 8 * lg + (l16 >> 2);
  const int c = 2 * mt + ((l16 & 3) >> 1);
  return chunk_off<D, kColTile>(r, c) + 8 * (l16 & 1);
}

__device__ __forceinline__ const char *lds_at(const void *base, int byte_off) {
  return static_cast<const char *>(base) + byte_off;
}

// 16-byte row read at a precomputed byte offset.
__device__ __forceinline__ bf16x8 lds_row8(const void *base, int byte_off) {
  return *reinterpret_cast<const bf16x8 *>(lds_at(base, byte_off));
}

// Operand of a contraction over ROWS: lane l receives
// tile[row0 + 8*(l/16) + j][16*mt + l%16], j = 0..7, given
// off = col_read_off(mt) + row0 * 2D.  ds_read_b64_tr_b16 hands lane i of
// each 16-lane group element i%4 of the 8 bytes loaded by lane 4k + i/4 as
// its k-th value; the second read covers rows +4.
template <int D>
__device__ __forceinline__ bf16x8 lds_col8(const void *base, int byte_off) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)lds_at(base, byte_off));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)lds_at(base, byte_off + 4 * 2 * D));
  return __builtin_bit_cast(bf16x8, (s16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
}

// Stages 64-row tiles of a token-major tensor into LDS with W wavefronts.
// Rows >= nvalid are filled from row nvalid-1 (bf16 path) or with zeros
// (fp32 path); the kernels mask them, they only need to be finite.
//   init(): stride = elements between consecutive rows of the tensor;
//   issue<KIND>(): src = first row of the tile; KIND = tile layout.
// bf16: issue() starts direct global->LDS copies; the caller waits for them
//   (wait_staged) before the barrier that publishes the tile.  commit() does
//   nothing.
// fp32: issue() loads into a register slot, commit() rounds to bf16 and
//   stores (used only for fp32 inputs; one loader stages two tensors).
template <int D, typename InT, int W>
struct TileLoader;

template <int D, int W>
struct TileLoader<D, __bf16, W> {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;           // rows per wavefront instruction
  static constexpr int NI = kTileRows / RPI / W;  // instructions per wavefront
  static_assert(NI >= 1 && NI * RPI * W == kTileRows, "tile split");
  int row_[NI];     // lane's tile row per instruction
  int off_[2][NI];  // element offset of the lane's chunk in a full tile, per tile kind
  int stride_;      // elements between rows (< 2^31 / 64 is checked on the host)
  int wave_;        // wavefront index (scalar)
  __device__ __forceinline__ void init(int wave, int lane, int64_t stride) {
    stride_ = (int)stride;
    wave_ = wave;
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      row_[t] = (wave * NI + t) * RPI + lane / CPR;
      off_[kRowTile][t] = row_[t] * stride_ + 8 * ((lane % CPR) ^ swz<D, kRowTile>(row_[t]));
      off_[kColTile][t] = row_[t] * stride_ + 8 * ((lane % CPR) ^ swz<D, kColTile>(row_[t]));
    }
  }
  template <int KIND>
  __device__ __forceinline__ void issue(__bf16 *tile, const __bf16 *src, int nvalid, int, int = 0) const {
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      int off = off_[KIND][t];
      if (nvalid < kTileRows && row_[t] >= nvalid)  // partial tile: repeat the last valid row
        off += (nvalid - 1 - row_[t]) * stride_;
      __builtin_amdgcn_global_load_lds((const void *)(src + off),
                                       (__attribute__((address_space(3))) void *)(tile + (wave_ * NI + t) * RPI * D),
                                       16, 0, 0);
    }
  }
  template <int KIND>
  __device__ __forceinline__ void commit(__bf16 *, int, int = 0) const {}
};

template <int D, int W>
struct TileLoader<D, float, W> {
  static constexpr int CPR = D / 8;
  static constexpr int N = (kTileRows * CPR + 64 * W - 1) / (64 * W);  // chunks per thread
  u32x4 r_[2][N];  // two staged tensors (slot 0 / 1)
  int64_t stride_;
  __device__ __forceinline__ void init(int, int, int64_t stride) { stride_ = stride; }
  // fp32 path: issue<KIND>(...) loads into register slot `slot` (the tile
  // pointer is unused until commit).
  template <int KIND>
  __device__ __forceinline__ void issue(__bf16 *, const float *src, int nvalid, int wave, int slot = 0) {
    const int tid = wave * 64 + (int)(threadIdx.x & 63);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = tid + 64 * W * i, row = ch / CPR, c = ch % CPR;
      r_[slot][i] = (row < kTileRows && row < nvalid) ? load8<float>(src + row * stride_ + 8 * c) : (u32x4){0, 0, 0, 0};
    }
  }
  template <int KIND>
  __device__ __forceinline__ void commit(__bf16 *tile, int tid, int slot = 0) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = tid + 64 * W * i, row = ch / CPR, c = ch % CPR;
      if (row < kTileRows)
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(tile) + chunk_off<D, KIND>(row, c)) = r_[slot][i];
    }
  }
};

// Waits for this wavefront's outstanding memory operations (including the
// direct global->LDS copies) before a barrier publishes a staged tile.
__device__ __forceinline__ void wait_staged() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace dev
}  // namespace segattn

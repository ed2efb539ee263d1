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
// Each was measured bank-conflict free on the device for its own read
// pattern (SQ_LDS_BANK_CONFLICT).  A tensor that is read both ways (Q and dO
// in the dK/dV role, K in the dQ role) is staged once, in the column layout:
// its row reads then conflict and run at about 60% of the row layout's LDS
// rate, which costs far less than copying the tile from memory twice.  (XOR
// swizzles that are conflict-free both ways exist -- a timed search over all
// linear ones found many -- but removing those conflicts left the kernel
// times unchanged, so the two layouts above stay.)  For D = 64 (8 chunks per row) the
// swizzle is taken mod 8.  Without padding a wavefront fills 1 KB of a tile
// with one global_load_lds_dwordx4 (global memory straight to LDS, no
// registers).
//
// Those copies are issued from inline assembly (dma_to_lds) and the rings are
// published with ring_barrier() instead of __syncthreads().  With the
// compiler builtin, the compiler cannot tell which ring slot a copy writes,
// so it waits for every copy in flight (vmcnt 0) before the first LDS read
// that follows one and, through __syncthreads()'s release fence, before every
// barrier -- including the copies of the next 2-3 tiles, which defeats the
// ring.  The kernels count their own copies instead (wait_vm / wait_stages
// before each ring_barrier).  Vector-memory loads complete in issue order, so
// the compiler's own vmcnt waits for its loads stay correct with these extra
// copies outstanding (they only become stricter).
//
// The per-lane byte offsets of every read are loop invariant; kernels compute
// them once (row_read_off / col_read_off) and add compile-time immediates for
// the pair, half and buffer indices (the swizzles ignore row bits 2 and 5).
#pragma once

#include <type_traits>

#include "device_common.h"

namespace segattn {
namespace dev {

constexpr int kTileRows = 64;

// LDS byte address of a pointer into a __shared__ array.  Kernels take it
// once from the array itself and add compile-time offsets: converting
// computed generic pointers instead costs a null check per use and keeps
// 64-bit pointers in scalar registers.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Direct copy global -> LDS of BYTES (4 or 16) per lane: lane i's bytes at
// base + voff (base wave-uniform, held in scalar registers; voff the lane's
// byte offset) land at LDS byte address lds_dst + BYTES * i.  With the base
// in scalar registers a copy needs no per-lane address arithmetic.  M0 holds
// the wave-uniform LDS destination; no instruction the compiler generates in
// these kernels keeps a value in M0, so clobbering it here is safe.  ALT
// only changes the assembly text (a comment), so that the compiler does not
// merge copies on different paths into one with selected operands.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES, bool ALT = false>
__device__ __forceinline__ void dma_to_lds(const void *base, uint32_t voff, uint32_t lds_dst) {
  static_assert(BYTES == 4 || BYTES == 16, "copy width");
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
  if constexpr (BYTES == 16 && !ALT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(base) : "memory", "m0");
  else if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 ; partial" ::"s"(m0), "v"(voff), "s"(base)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(m0), "v"(voff), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier of the LDS rings: this wavefront's LDS reads and writes
// are complete (lgkmcnt 0), then s_barrier.  Its direct copies must already
// be covered by a vmcnt wait (wait_vm / wait_stages).  The asm statement is
// also a compiler barrier for memory accesses.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
// immediate, which leaves both swizzles unchanged) at logical chunk 4*ks + lg.
// Returns the byte offset for step ks in a tile of the given kind.
template <int D, int KIND = kRowTile>
__device__ __forceinline__ int row_read_off(int ks, int l16, int lg) {
  const int r = 8 * (l16 >> 2) + (l16 & 3);
  return chunk_off<D, KIND>(r, 4 * ks + lg);
}

// Transposing reads (column tiles).  For column block mt (16 columns) lane
// (l16, lg) points at row 8*lg + l16/4 (plus multiples of 4 rows as
// immediates), columns 16*mt + 4*(l16%4) .. +3.  Returns the byte offset.
template <int D>
__device__ __forceinline__ int col_read_off(int mt, int l16, int lg) {
  const int r = 8 * lg + (l16 >> 2);
  const int c = 2 * mt + ((l16 & 3) >> 1);
  return chunk_off<D, kColTile>(r, c) + 8 * (l16 & 1);
}

// The offsets of the other depth steps / column blocks follow from step 0 by
// an XOR: the step index only flips offset bits that the swizzle XORs and no
// other term sets (bits 6-7 for row reads, 5-7 for transposing reads, both
// at D = 64 and 128):
//   row_read_off(ks) == row_read_off(0) ^ row_step(ks),
//   col_read_off(mt) == col_read_off(0) ^ col_step(mt).
// A kernel short of registers keeps only the step-0 offsets.
__device__ __forceinline__ constexpr int row_step(int ks) { return ks << 6; }
__device__ __forceinline__ constexpr int col_step(int mt) { return mt << 5; }

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
//   stage<KIND>(): tile = the tile in LDS, as a pointer and as its LDS byte
//   address; src = first row of the tile; KIND = tile layout.
// bf16: stage() starts kInstr direct global->LDS copies per wavefront and
//   returns; wait_vm / wait_stages below wait for them before the barrier
//   that publishes the tile.
// fp32: stage() loads, rounds to bf16 and stores with ordinary LDS writes
//   (only used for fp32 inputs; the barrier publishes them).
template <int D, typename InT, int W>
struct TileLoader;

template <int D, int W>
struct TileLoader<D, __bf16, W> {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;           // rows per wavefront instruction
  static constexpr int NI = kTileRows / RPI / W;  // instructions per wavefront
  static constexpr int kInstr = NI;
  static_assert(NI >= 1 && NI * RPI * W == kTileRows, "tile split");
  // Instruction t copies the rows of instruction 0 plus t * RPI.  With NI <= 2
  // and RPI = 4 that only sets row bit 2, which neither swizzle reads, so its
  // lane offsets are instruction 0's plus t * RPI rows: that part goes on the
  // scalar base and the lanes keep one offset per tile kind.
  static_assert(NI == 1 || (NI == 2 && RPI == 4), "later instructions must keep the lane's swizzled chunk");
  int row0_;          // lane's tile row in instruction 0
  uint32_t boff_[2];  // byte offset of the lane's chunk in a full tile, per tile kind
  uint32_t rbytes_;   // bytes between rows (64 rows < 2^32 bytes: heads <= 65536, d <= 128)
  int wave_;          // wavefront index (scalar)
  __device__ __forceinline__ void init(int wave, int lane, int64_t stride) {
    rbytes_ = 2u * (uint32_t)stride;
    wave_ = wave;
    row0_ = wave * NI * RPI + lane / CPR;
    boff_[kRowTile] = row0_ * rbytes_ + 16u * ((lane % CPR) ^ swz<D, kRowTile>(row0_));
    boff_[kColTile] = row0_ * rbytes_ + 16u * ((lane % CPR) ^ swz<D, kColTile>(row0_));
  }
  template <int KIND>
  __device__ __forceinline__ void stage(__bf16 *, uint32_t tile, const __bf16 *src, int nvalid) const {
    if (nvalid >= kTileRows) {
      // full tile: the precomputed lane offsets as they are
#pragma unroll
      for (int t = 0; t < NI; ++t)
        dma_to_lds<16>(reinterpret_cast<const char *>(src) + (size_t)(t * RPI) * rbytes_, boff_[KIND],
                       tile + (wave_ * NI + t) * RPI * D * 2);
    } else {
      // partial tile: rows >= nvalid repeat the last valid row.  The lane
      // offset is an unsigned 32-bit byte offset from the unshifted base, so
      // it is formed as min(row, nvalid - 1) rows plus the lane's chunk,
      // never as a difference that could go below zero.
      const uint32_t chunk = boff_[KIND] - (uint32_t)row0_ * rbytes_;
#pragma unroll
      for (int t = 0; t < NI; ++t)
        dma_to_lds<16, true>(src, (uint32_t)min(row0_ + t * RPI, nvalid - 1) * rbytes_ + chunk,
                             tile + (wave_ * NI + t) * RPI * D * 2);
    }
  }
};

template <int D, int W>
struct TileLoader<D, float, W> {
  static constexpr int CPR = D / 8;
  static constexpr int N = (kTileRows * CPR + 64 * W - 1) / (64 * W);  // chunks per thread
  static constexpr int kInstr = 0;  // nothing left in flight after stage()
  int64_t stride_;
  int tid_;
  f32x4 raw_[N][2];  // a fetched tile, not yet rounded and written to LDS
  __device__ __forceinline__ void init(int wave, int lane, int64_t stride) {
    stride_ = stride;
    tid_ = wave * 64 + lane;
  }
  // Issues the loads of one tile into registers (rows >= nvalid read as
  // zeros); the compiler waits for them where commit() uses them.
  __device__ __forceinline__ void fetch(const float *src, int nvalid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = tid_ + 64 * W * i, row = ch / CPR, c = ch % CPR;
      const bool ok = row < kTileRows && row < nvalid;
      raw_[i][0] = ok ? *reinterpret_cast<const f32x4 *>(src + row * stride_ + 8 * c) : (f32x4){0.f, 0.f, 0.f, 0.f};
      raw_[i][1] = ok ? *reinterpret_cast<const f32x4 *>(src + row * stride_ + 8 * c + 4) : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  }
  // Rounds the fetched tile to bf16 (nearest even) and writes it to LDS in
  // layout KIND.
  template <int KIND>
  __device__ __forceinline__ void commit(__bf16 *tile) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = tid_ + 64 * W * i, row = ch / CPR, c = ch % CPR;
      if (row < kTileRows)
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(tile) + chunk_off<D, KIND>(row, c)) =
            __builtin_bit_cast(u32x4, pack_bf16x8(raw_[i][0], raw_[i][1]));
    }
  }
  template <int KIND>
  __device__ __forceinline__ void stage(__bf16 *tile, uint32_t, const float *src, int nvalid) {
    fetch(src, nvalid);
    commit<KIND>(tile);
  }
};

// 64 consecutive floats (one per lane; lanes >= nvalid repeat element
// nvalid-1) copied straight into LDS (byte address dst) by one wavefront.
__device__ __forceinline__ void stage_row_floats(uint32_t dst, const float *src, int nvalid, int lane) {
  dma_to_lds<4>(src, 4u * (uint32_t)min(lane, nvalid - 1), dst);
}

// Waits until at most N of this wavefront's vector memory operations are
// still outstanding (loads complete in issue order).  Only the vmcnt field is
// constrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Prefetch ring: before computing on stage j, wait for this wavefront's
// copies of stage j while `ahead` (0 .. NS-2, wave-uniform) later stages,
// L copies each, may stay in flight.  L = 0 (register staging) waits for all.
template <int L, int NS>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (L > 0 && NS >= 4) {
    if (ahead >= 2) {
      wait_vm<2 * L>();
      return;
    }
  }
  if constexpr (L > 0 && NS >= 3) {
    if (ahead >= 1) {
      wait_vm<L>();
      return;
    }
  }
  wait_vm<0>();
}

// Software pipeline over N unrolled sub-steps: the operands of sub-step i+1
// are loaded (load(ic<i+1>)) before sub-step i consumes its own
// (use(ic<i>, ops)), so LDS latency overlaps the matrix products instead of
// stalling before each group of them.
template <int I, int N, typename L, typename U, typename T>
__device__ __forceinline__ void pipe_step(L &load, U &use, const T &cur) {
  if constexpr (I + 1 < N) {
    const auto nxt = load(std::integral_constant<int, I + 1>{});
    // keep the compiler's scheduler from sinking those loads below the
    // products that follow
    __builtin_amdgcn_sched_barrier(0);
    use(std::integral_constant<int, I>{}, cur);
    pipe_step<I + 1, N>(load, use, nxt);
  } else {
    use(std::integral_constant<int, I>{}, cur);
  }
}
template <int N, typename L, typename U>
__device__ __forceinline__ void pipelined(L load, U use) {
  pipe_step<0, N>(load, use, load(std::integral_constant<int, 0>{}));
}

// Runs f(integral_constant<B>) for B = 0 .. NS-1 while it returns true; the
// ring slot of every step is a compile-time constant.
template <int B, int NS, typename F>
__device__ __forceinline__ bool ring_pass(F &f) {
  if constexpr (B == NS) {
    return true;
  } else {
    if (!f(std::integral_constant<int, B>{})) return false;
    return ring_pass<B + 1, NS>(f);
  }
}

}  // namespace dev
}  // namespace segattn

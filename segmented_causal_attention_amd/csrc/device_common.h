// Device helpers shared by the gfx950 kernels: vector types, bf16 packing,
// global/LDS 16-byte accesses and wavefront reductions.
//
// MFMA operand layout used throughout (v_mfma_f32_16x16x32_bf16, wave64):
//   A (16 x 32, rows m, depth k): lane l supplies A[l % 16][8 * (l / 16) + j], j = 0..7
//   B (32 x 16, depth k, cols n): lane l supplies B[8 * (l / 16) + j][l % 16]
//   C (16 x 16):                  lane l holds   C[4 * (l / 16) + i][l % 16], i = 0..3
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace segattn {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two floats -> two bf16 (round to nearest even) packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const f32x4 &a, const f32x4 &b) {
  u32x4 u = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
             pack_bf16x2(b[2], b[3])};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 consecutive input elements as packed bf16 (4 dwords).  For fp32 input
// the values are rounded to nearest-even bf16 here, while staging.
template <typename InT>
__device__ __forceinline__ u32x4 load8(const InT *p);

template <>
__device__ __forceinline__ u32x4 load8<__bf16>(const __bf16 *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

template <>
__device__ __forceinline__ u32x4 load8<float>(const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  return (u32x4){pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                 pack_bf16x2(b[2], b[3])};
}

// Operand of a contraction over ROWS of a row-major bf16 LDS tile: lane l
// receives tile[row0 + 8*(l/16) + j][col0 + l%16], j = 0..7 (the A layout
// with m = column, k = row; equally the B layout with n = column).
// ds_read_b64_tr_b16 hands lane i of each 16-lane group element i%4 of the
// 8 bytes loaded by lane 4k + i/4 as its k-th value, so lane j points at
// row 8*(l/16) + j/4, columns 4*(j%4) .. +3.  Needs col0 % 4 == 0.
__device__ __forceinline__ bf16x8 lds_rows8(const __bf16 *tile, int stride, int row0, int col0, int l16, int lg) {
  const __bf16 *p = tile + (row0 + 8 * lg + (l16 >> 2)) * stride + col0 + 4 * (l16 & 3);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * stride));
  return __builtin_bit_cast(bf16x8, (s16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
}

// c + lo + hi of the two bf16 values packed in w (v_dot2 against ones; the
// products are exact, the sum is fp32).
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), c,
                                         false);
}

// 4 consecutive input elements as floats holding their bf16 values (fp32
// input is rounded to nearest-even bf16, as when it is staged).
template <typename InT>
__device__ __forceinline__ f32x4 load4_bf16(const InT *p);
template <>
__device__ __forceinline__ f32x4 load4_bf16<__bf16>(const __bf16 *p) {
  const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
  return (f32x4){bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
}
template <>
__device__ __forceinline__ f32x4 load4_bf16<float>(const float *p) {
  const f32x4 x = *reinterpret_cast<const f32x4 *>(p);
  const uint32_t w0 = pack_bf16x2(x[0], x[1]), w1 = pack_bf16x2(x[2], x[3]);
  return (f32x4){bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
}

// Byte-select of two dwords: result byte i = byte sel_i of {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// low bf16 of x and low bf16 of y -> (y.lo << 16) | x.lo
__device__ __forceinline__ uint32_t join_lo(uint32_t x, uint32_t y) { return perm(y, x, 0x05040100u); }
// high bf16 of x and high bf16 of y -> (y.hi << 16) | x.hi
__device__ __forceinline__ uint32_t join_hi(uint32_t x, uint32_t y) { return perm(y, x, 0x07060302u); }

// Byte addresses for ds_bpermute of lane ^ 16 and lane ^ 32 (computed once).
struct XorLanes {
  int x16, x32;
  __device__ __forceinline__ XorLanes(int lane) : x16((lane ^ 16) << 2), x32((lane ^ 32) << 2) {}
};
__device__ __forceinline__ float bperm(int addr, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}
// Reductions over the lanes l, l^16, l^32, l^48 (the 4 lane groups that hold
// one row's scores).
__device__ __forceinline__ float wave_max_xor16_32(float v, const XorLanes &x) {
  v = fmaxf(v, bperm(x.x16, v));
  v = fmaxf(v, bperm(x.x32, v));
  return v;
}
__device__ __forceinline__ float wave_sum_xor16_32(float v, const XorLanes &x) {
  v += bperm(x.x16, v);
  v += bperm(x.x32, v);
  return v;
}

// Workgroup index -> (unit rank, head) for a grid of nunits x nh workgroups.
// Consecutive workgroups are dealt to the 8 XCDs in turn.  When nh is a
// multiple of 8, XCD c takes the heads [c*nh/8, (c+1)*nh/8) one after the
// other, each head's units in rank (heaviest-first) order, so the
// workgroups resident on one XCD at a time mostly belong to one head and
// stream the same tiles through that XCD's L2.
__device__ __forceinline__ void map_xcd(int x, int nh, int nunits, int &rank, int &h) {
  if ((nh & 7) == 0) {
    const int xcd = x & 7, j = x >> 3;
    h = xcd * (nh >> 3) + j / nunits;
    rank = j - (j / nunits) * nunits;
  } else {
    rank = x / nh;
    h = x - rank * nh;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

}  // namespace dev
}  // namespace segattn

// pba_device.h - device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core fragment layouts used throughout (CDNA3/CDNA4 MFMA, wave64,
// lane l, lane group g = l / 16, lane column n = l % 16):
//   v_mfma_f32_16x16x32_bf16  A[i][k]: lane (g, i) holds k = 8g..8g+7
//                             B[k][n]: lane (g, n) holds k = 8g..8g+7
//   v_mfma_f32_16x16x4_f32    A[i][k]: lane (g, i) holds k = g
//                             B[k][n]: lane (g, n) holds k = g
//   result D[i][n] (both): lane (g, n) holds rows i = 4g..4g+3.
// A and B pair their k slots by (lane group, register), so any relabelling of
// k that is applied to both operands leaves the product unchanged; the
// kernels use that freedom to match the register layout of a previous
// product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma4f(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ u16 f2bf(float x) { return __builtin_bit_cast(u16, (__bf16)x); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float sigmoidf_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x4 as_bf4(u32x2 v) { return __builtin_bit_cast(bf16x4, v); }

// Pack two 4-float result fragments into one 8-wide bf16 operand (RNE).
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
  u32x4 r;
  r[0] = pack2(a[0], a[1]);
  r[1] = pack2(a[2], a[3]);
  r[2] = pack2(b[0], b[1]);
  r[3] = pack2(b[2], b[3]);
  return as_bf8(r);
}

// Identity operands that move a bf16 bias tile into fp32 accumulator
// registers on the matrix core instead of spending VALU conversions on it.
// They are 16x16x32 operands on purpose: a product chained into the
// accumulator of the next product must use the same opcode (a 16x16x16
// product feeding a 16x16x32 accumulation was observed to hand over rows
// 2-3 of each result group before they were written).
//
// A operand, lane (g, i), register v: 1 where g == i/4 and v == 4*half + i%4.
// With B = 8 contiguous bf16 values per lane (lane (g, n) holds row n's
// entries 8 apart per lane group), D[i][n] = B(lane (i/4, n))[4*half + i%4]:
// half 0 picks elements 0..3, half 1 elements 4..7 of each lane's B operand.
__device__ __forceinline__ bf16x8 ident_rows_frag(int lane, int half) {
  const int g = lane >> 4, i = lane & 15;
  const uint32_t one = 0x3F80u;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (g == (i >> 2)) {
    const int v = 4 * half + (i & 3);  // element index 0..7
    r[v >> 1] = one << (16 * (v & 1));
  }
  return as_bf8(r);
}
// B operand, lane (g, n), register v: 1 where g < 2 and n == 8g + v.  With
// A lane (g, i) holding row i's entries 8g..8g+7 (lanes g >= 2 may hold any
// finite values), D[i][n] = A[i][n]: the transpose of the A tile lands in the
// result layout.
__device__ __forceinline__ bf16x8 ident_cols_frag(int lane) {
  const int g = lane >> 4, n = lane & 15;
  const uint32_t one = 0x3F80u;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (g < 2 && (n >> 3) == g) {
    const int v = n & 7;
    r[v >> 1] = one << (16 * (v & 1));
  }
  return as_bf8(r);
}
__device__ __forceinline__ bf16x8 ones_frag() {
  u32x4 r;
  r[0] = r[1] = r[2] = r[3] = 0x3F803F80u;
  return as_bf8(r);
}

// Reduction over the four lanes that share a lane column (l, l^16, l^32, l^48).
__device__ __forceinline__ float max_over_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Workgroup index remap so that consecutive logical tiles run on the same
// XCD.  The dispatcher hands workgroup w to XCD (w mod 8); with this remap a
// contiguous range of logical ids lands on one XCD and shares its L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int nx = 8;
  const int q = total / nx, r = total % nx;
  const int x = w % nx, idx = w / nx;
  return (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
}

}  // namespace pba

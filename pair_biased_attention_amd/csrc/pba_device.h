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
// log2(e) as a sum of two bf16 values, hi = 1.4453125 and lo = -0.00262451171875;
// hi + lo differs from log2(e) by 4.9e-6 relative.
constexpr uint32_t kLog2eHiBf16 = 0x3FB9u;
constexpr uint32_t kLog2eLoBf16 = 0xBB2Cu;

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma4f(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ u16 f2bf(float x) { return __builtin_bit_cast(u16, (__bf16)x); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two floats -> two bf16 (RNE) in one dword; a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
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
// `one` is the bf16 bit pattern placed on the diagonal (1.0 by default; a
// split constant such as log2(e) = hi + lo scales the moved tile exactly
// enough with two products).
__device__ __forceinline__ bf16x8 ident_rows_frag(int lane, int half, uint32_t one = 0x3F80u) {
  const int g = lane >> 4, i = lane & 15;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (g == (i >> 2)) {
    const int v = 4 * half + (i & 3);  // element index 0..7
    r[v >> 1] = one << (16 * (v & 1));
  }
  return as_bf8(r);
}
// B operand, lane (g, n), register v: 1 where g0 <= g < g0 + 2 and
// n == 8(g - g0) + v (g0 = 0 or 2).  With A lane (g, i) holding row i's
// entries 8g..8g+7 (the lanes of the other two groups may hold any finite
// values), D[i][n] = A[i][8 g0 + n]: the transpose of the half of the A
// tile that groups g0, g0+1 hold lands in the result layout.
__device__ __forceinline__ bf16x8 ident_cols_frag(int lane, uint32_t one = 0x3F80u, int g0 = 0) {
  const int g = lane >> 4, n = lane & 15;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (g >= g0 && g < g0 + 2 && (n >> 3) == g - g0) {
    const int v = n & 7;
    r[v >> 1] = one << (16 * (v & 1));
  }
  return as_bf8(r);
}
// ---- LDS transpose reads (gfx950 ds_read_b64_tr_b16)
// Within each 16-lane group, lane 4e+a supplies the address of 4 consecutive
// bf16 values of some row R(e) starting at column c+4a; lane j = 4a+v then
// receives the column c+j of the four rows R(0..3).  Two such reads build one
// 16x16x32 operand whose k axis runs down the rows of a row-major tile.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ u32x2 lds_tr16(const u16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Operand whose lane (g, j) holds X[rb0 + e][c0 + j] in element e and
// X[rb1 + e][c0 + j] in element 4 + e (e = 0..3), for a row-major LDS tile X
// with row stride RS elements; rb0/rb1 are this lane group's row bases.
template <int RS>
__device__ __forceinline__ bf16x8 tr_frag(const u16* tile, int rb0, int rb1, int c0, int lane) {
  const int j = lane & 15;
  const int e = j >> 2, a = j & 3;
  const u32x2 lo = lds_tr16(tile + (rb0 + e) * RS + c0 + 4 * a);
  const u32x2 hi = lds_tr16(tile + (rb1 + e) * RS + c0 + 4 * a);
  return as_bf8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// ---- LDS tile layouts of bf16 row-major tiles (rows of DP elements).
// TileLds<DP, MODE>::off(r, c) is the element offset of row r, column c.
// DP = 32: 64-byte rows, no padding; the four 16-byte units of row r sit at
// unit position u ^ f(r).  Under the 64-bank model (16 lanes per cycle for a
// 16-byte read, 32 lanes for an 8-byte one) f spreads both kinds of reads
// over every bank:
//   MODE 0 (query tiles: operand rows r = 16t + i, transposed reads of rows
//   4g + e and 16 + 4g + e):  f = 2 * bit2(r) + bit3(r)
//   MODE 1 (key tiles: operand rows 16(i/4) + i%4 + 4t, transposed reads of
//   rows 16g + 8m + e):        f = 2 * bit4(r) + bit5(r)
// For a fixed unit, the 16 rows of a 16-byte read fall on four 64-byte
// offsets (r mod 4) times four distinct units; the eight rows of a 32-lane
// transposed read fall on four offsets times two distinct unit pairs.
// DP = 64: rows padded to 72 elements (144 bytes).
template <int DP, int MODE>
struct TileLds {
  static constexpr int kRowElems = DP == 32 ? 32 : DP + 8;
  __device__ static __forceinline__ int f(int r) {
    return MODE == 0 ? 2 * ((r >> 2) & 1) + ((r >> 3) & 1) : 2 * ((r >> 4) & 1) + ((r >> 5) & 1);
  }
  __device__ static __forceinline__ int off(int r, int c) {
    if constexpr (DP == 32) return r * 32 + ((((c >> 3) ^ f(r)) & 3) << 3) + (c & 7);
    else return r * (DP + 8) + c;
  }
};

// 16 query rows x 64 keys of a bf16 bias block in LDS as 16-byte units:
// unit u (keys 8u .. 8u + 7) of row q sits at slot 8q + (u ^ ((q >> 1) & 7)).
// The two units a lane group reads from one row then fall on distinct banks
// for all 16 rows of a 16-lane read.
__device__ __forceinline__ int bias_rows_slot(int q, int u) { return 8 * q + (u ^ ((q >> 1) & 7)); }

// tr_frag for a TileLds layout: lane (g, j) gets rows rb0+e and rb1+e
// (e = 0..3) at column c0 + j of the tile.
template <class L>
__device__ __forceinline__ bf16x8 tr_frag_l(const u16* tile, int rb0, int rb1, int c0, int lane) {
  const int j = lane & 15;
  const int e = j >> 2, a = j & 3;
  const u32x2 lo = lds_tr16(tile + L::off(rb0 + e, c0 + 4 * a));
  const u32x2 hi = lds_tr16(tile + L::off(rb1 + e, c0 + 4 * a));
  return as_bf8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// ---- vector-memory waits for loads the compiler does not track as producers
// (buffer loads with an LDS destination): s_waitcnt with only the vector
// counter set, at most N of this wave's vector-memory operations outstanding.
typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource words (base, stride 0, num_records bytes, the same flags as
// make_rsrc) for the inline-asm loads below; every word is wave-uniform.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane((int)num_bytes), 0x00020000};
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes LDS bytes
// lds_base + 16 l .. + 15 (zeros where byte_off fails the range check).  It
// has no register results.  Written as asm so that the compiler, which cannot
// tell which LDS bytes such a load writes, does not drain every one of them
// before each later LDS read; callers order them with vm_wait and barriers.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t lds_base, uint32_t byte_off) {
  // the LDS base goes in through the m0 operand constraint, so the compiler
  // itself writes m0 and knows the register is taken by this statement
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(byte_off), "s"(rsrc), "{m0}"(lds_base)
               : "memory");
}
// 4 bytes per lane from a buffer straight into LDS: lane l writes LDS bytes
// lds_base + 4 l .. + 3 (zero where byte_off fails the range check); ordered
// like lds_dma16.
__device__ __forceinline__ void lds_dma4(i32x4 rsrc, uint32_t lds_base, uint32_t byte_off) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(byte_off), "s"(rsrc), "{m0}"(lds_base)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)(p);
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---- key-split staging: one wave's private copy of a 64-key block
// K and V rows in the TileLds<32, 1> layout (64-byte rows) and the bias of
// the wave's 16 query rows in the bias_rows_slot layout, 10 KB per wave.
struct KeySplitLds {
  u16 k[64 * 32];
  u16 v[64 * 32];
  u32x4 bias[128];
};

// Stage key block kb (64 keys) of one (b, h) into `my` with LDS-destination
// loads, ten per wave.  K and V: load i fills LDS units 64 i + lane, i.e. row
// r = 16 i + lane / 4 at slot lane % 4, which holds channel unit
// slot ^ f(r); units past d read as zeros and rows past N fail the range
// check of the (b, h) plane.  Bias: load i fills slots 64 i + lane, i.e. query
// row q = 8 i + lane / 8 at slot lane % 8, holding keys kb + 8u .. + 7 with
// u = slot ^ ((q >> 1) & 7); rows past N read as zeros, keys past N land in
// masked columns.  The loads are ordered by the caller's vm_wait.
__device__ __forceinline__ void key_split_stage(KeySplitLds& my, i32x4 krs, i32x4 vrs, i32x4 brs, int q0, int N,
                                                int d, int kb, int lane) {
  constexpr uint32_t kOob = 0xFFFFFFF0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * i + (lane >> 2);
    const int c8 = ((lane & 3) ^ TileLds<32, 1>::f(r)) & 3;
    const uint32_t off = 8 * c8 < d ? (uint32_t)(((kb + r) * d + 8 * c8) * 2) : kOob;
    lds_dma16(krs, lds_addr(my.k) + 1024 * i, off);
    lds_dma16(vrs, lds_addr(my.v) + 1024 * i, off);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = 8 * i + (lane >> 3);
    const int u = (lane & 7) ^ ((q >> 1) & 7);
    const uint32_t off = q0 + q < N ? (uint32_t)(((size_t)(q0 + q) * N + kb + 8 * u) * 2) : kOob;
    lds_dma16(brs, lds_addr(my.bias) + 1024 * i, off);
  }
}

// ---- bounds-checked global loads through a buffer resource: any byte past
// num_bytes reads as zero, so ragged tiles need no per-element guards.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}
// The whole offset goes in the per-lane operand: that is the part the range
// check sees.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_u8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, byte_off, 0, 0);
}
__device__ __forceinline__ float2 buf_load_f32x2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// s_waitcnt immediate: vmcnt = 0, expcnt and lgkmcnt left at their maxima
// (no wait on them).
constexpr int kWaitVmcnt0 = 0x0F70;

// Most negative finite bf16 (-3.39e38), packed twice: the bias value given to
// masked keys so their scores stay finite through the identity product
// (0 * -inf would be NaN) and their probabilities underflow to exactly 0.
constexpr uint32_t kMaskedBias2 = 0xFF7FFF7Fu;
constexpr float kMaskedThreshold = -1.0e38f;

__device__ __forceinline__ bf16x8 ones_frag() {
  u32x4 r;
  r[0] = r[1] = r[2] = r[3] = 0x3F803F80u;
  return as_bf8(r);
}

// Reduction over the four lanes that share a lane column (l, l^16, l^32, l^48),
// with the gfx950 row-swap permutes (VALU, no LDS round trip): swapping the
// two 32-lane halves (then the odd/even 16-lane rows) between two copies of x
// leaves each lane with its partner's value in one of the two results.
__device__ __forceinline__ float max_over_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const uint32_t w = __float_as_uint(x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

// Wave index within the workgroup, marked wave-uniform so that values
// derived from it stay in scalar registers.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

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

// bias_proj.hip - the pair-bias projection bias = Linear(LayerNorm(z)) and its
// backward on gfx950.
//
// AlphaFold3 open-source implementation page (molayo1419.me), section "Model
// Efficiency": each attention projects its pair bias from the pair
// representation z [N, N, c], and that projection needs a gradient; the
// Protenix page counts LayerNorm among the kernels worth a custom
// implementation.  Per pair position p (= i N + j):
//   xhat = (z[p] - mean) / sqrt(var + eps)      biased variance over c channels
//   y    = gamma * xhat + beta,   bias[h, p] = sum_c w[h, c] y[c]
// Backward, given dbias [H, N, N]:
//   dy[p, c] = sum_h dbias[h, p] w[h, c],   dxhat = gamma * dy
//   dz       = rstd * (dxhat - mean_c(dxhat) - xhat * mean_c(dxhat * xhat))
//   dw[h, c] = sum_p dbias[h, p] y[p, c], dgamma = sum_p dy xhat, dbeta = sum_p dy
//
// Layout of the work (the kernels are HBM-bound: 2c bytes of z per position
// against 2H bytes of bias):
//  * A wave owns 16 consecutive positions.  Lane (g, i) holds position i and
//    channels 32kt + 8g .. 32kt + 8g + 7 of every 32-channel slice kt, read
//    straight from HBM as 16-byte loads.  That register layout is the A
//    operand of a 16x16x32 product over channels, so the projection runs on
//    the matrix cores from the loaded registers, and the LayerNorm statistics
//    need only the four lanes of one lane column.
//  * gamma is folded into the projection weights (gamma * w on the matrix
//    core, w . beta added to the result), so the forward never forms y.
//  * Backward: dxhat = (gamma w)^T dbias is a 16x16x16 product over heads
//    whose result rows are relabelled channels, chosen so that the result
//    lands in the z layout above and the LayerNorm backward stays lane-local.
//    dw, dgamma and dbeta follow from X[h, c] = sum_p dbias[h, p] xhat[p, c]
//    and s[h] = sum_p dbias[h, p] (dw = gamma X + beta s, dgamma = sum_h w X,
//    dbeta = sum_h w s): one more product per tile on an LDS transpose of
//    xhat, accumulated per wave, summed per workgroup in wave order, then over
//    workgroups in a fixed order by a small kernel.  No atomics: results are
//    bitwise reproducible.
#include <algorithm>

#include "pba.h"
#include "pba_device.h"
#include "pba_kernels.h"

namespace pba {
namespace {

constexpr uint32_t kOob = 0xFFFFFFF0u;
constexpr int kFwdWaves = 4;
constexpr int kFwdMaxWg = 512;
constexpr int kStages = 3;      // register sets in the load ring of both kernels
constexpr int kRedCh = 4;       // channels per reduction workgroup
constexpr int kRedGroups = 12;  // partial-row groups per reduction workgroup
constexpr int kRedElems = kRedCh * 16 + 16;

__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}

// Sum over the four lanes of a lane column (l, l^16, l^32, l^48); every one
// of them gets the same bits.
__device__ __forceinline__ float sum_over_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  const uint32_t v = __float_as_uint(x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
}

template <int KT>
__device__ __forceinline__ void unpack_z(const u32x4 (&u)[KT], float (&x)[KT][8]) {
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[kt][2 * q] = __uint_as_float(u[kt][q] << 16);
      x[kt][2 * q + 1] = __uint_as_float(u[kt][q] & 0xFFFF0000u);
    }
}

// In place z -> xhat for the position of this lane column; returns rstd.
template <int KT>
__device__ __forceinline__ float normalise(float (&x)[KT][8], float eps) {
  constexpr float inv_c = 1.0f / (32 * KT);
  float s = 0.f;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int v = 0; v < 8; ++v) s += x[kt][v];
  const float mean = sum_over_groups(s) * inv_c;
  float q = 0.f;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      x[kt][v] -= mean;
      q = fmaf(x[kt][v], x[kt][v], q);
    }
  const float rstd = rsqrtf(sum_over_groups(q) * inv_c + eps);
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int v = 0; v < 8; ++v) x[kt][v] *= rstd;
  return rstd;
}

// z rows of tile tt: lane (g, i) gets position 16 tt + i, channels 32kt + 8g ..
// +7.  Positions past the end (and tiles past the last) read as zeros.
template <int C>
__device__ __forceinline__ void load_z(__amdgpu_buffer_rsrc_t rz, u32x4 (&dst)[C / 32], uint32_t tt,
                                       uint32_t ntiles, int g, int i) {
  const bool ok = tt < ntiles;
  const uint32_t base = ((tt * 16u + i) * C + 8u * g) * 2u;
#pragma unroll
  for (int kt = 0; kt < C / 32; ++kt) dst[kt] = buf_load16(rz, ok ? base + 64u * kt : kOob);
}

}  // namespace

template <int KT>
__global__ __launch_bounds__(kFwdWaves * 64) void bias_proj_fwd_kernel(ProjArgs a) {
  constexpr int C = 32 * KT;
  const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
  const uint32_t P = (uint32_t)a.N * (uint32_t)a.N;
  const int H = a.H;
  const uint32_t ntiles = (P + 15u) >> 4;
  const uint32_t nw = gridDim.x * kFwdWaves;
  uint32_t t = blockIdx.x * kFwdWaves + wave_index();
  if (t >= ntiles) return;

  const auto rz = make_rsrc(a.z, P * C * 2u);
  const auto rb = make_rsrc(a.bias, (uint32_t)H * P * 2u);
  // A ring of kStages register sets: while one tile is processed the z of the
  // next kStages - 1 tiles is in flight.  The ring is unrolled, so no copy
  // between sets (which would wait for their loads) is ever needed.  Its
  // first loads go out before the parameters are read.
  u32x4 zr[kStages][KT];
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) load_z<C>(rz, zr[s], t + s * nw, ntiles, g, i);

  // B operand of the projection: lane (g, h) holds gamma * w[h] on channels
  // 32kt + 8g + v (zero for h >= H); wb[h] = w[h] . beta.  Branch-free
  // 16-byte loads: lanes with h >= H read row 0 and scale it by zero.
  const bool hv = i < H;
  const float hm = hv ? 1.f : 0.f;
  const float* const wrow = a.w + (hv ? i : 0) * C;
  u32x4 bw[KT];
  float wb = 0.f;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int c0 = 32 * kt + 8 * g;
    float wv[8], gv[8], bv[8];
    *reinterpret_cast<float4*>(wv) = *reinterpret_cast<const float4*>(wrow + c0);
    *reinterpret_cast<float4*>(wv + 4) = *reinterpret_cast<const float4*>(wrow + c0 + 4);
    *reinterpret_cast<float4*>(gv) = *reinterpret_cast<const float4*>(a.gamma + c0);
    *reinterpret_cast<float4*>(gv + 4) = *reinterpret_cast<const float4*>(a.gamma + c0 + 4);
    *reinterpret_cast<float4*>(bv) = *reinterpret_cast<const float4*>(a.beta + c0);
    *reinterpret_cast<float4*>(bv + 4) = *reinterpret_cast<const float4*>(a.beta + c0 + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bw[kt][q] = pack2(hm * wv[2 * q] * gv[2 * q], hm * wv[2 * q + 1] * gv[2 * q + 1]);
      wb = fmaf(wv[2 * q], bv[2 * q], wb);
      wb = fmaf(wv[2 * q + 1], bv[2 * q + 1], wb);
    }
  }
  wb = sum_over_groups(wb) * hm;

  auto tile = [&](const u32x4 (&z)[KT], uint32_t tt) {
    float x[KT][8];
    unpack_z<KT>(z, x);
    normalise<KT>(x, a.eps);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      u32x4 p;
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = pack2(x[kt][2 * q], x[kt][2 * q + 1]);
      acc = mfma32(as_bf8(p), as_bf8(bw[kt]), acc);
    }
    // result lane (g, h) holds positions 16tt + 4g + r of head h
    const uint32_t p0 = tt * 16u + 4u * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = (hv && p0 + r < P) ? ((uint32_t)i * P + p0 + r) * 2u : kOob;
      __builtin_amdgcn_raw_buffer_store_b16(f2bf(acc[r] + wb), rb, off, 0, 0);
    }
  };
  bool more = true;
  while (more) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      if (more) {
        load_z<C>(rz, zr[(s + kStages - 1) % kStages], t + (kStages - 1) * nw, ntiles, g, i);
        __builtin_amdgcn_sched_barrier(0);
        tile(zr[s], t);
        t += nw;
        more = t < ntiles;
      }
    }
  }
}

// EVEN: N is even, so N^2 is a multiple of 4 and the four dbias values of a
// lane are one aligned 8-byte load, either wholly inside the tensor or wholly
// past its end.  Odd N takes four 2-byte loads.
template <int KT, bool EVEN>
__global__ __launch_bounds__(proj_bwd_waves(32 * KT) * 64) void bias_proj_bwd_kernel(ProjArgs a) {
  constexpr int C = 32 * KT;
  constexpr int RS = C + 16;   // xhat tile row stride (positions x channels)
  constexpr int DRS = 24;      // dbias tile row stride (heads x positions)
  constexpr int R = 16 * C + 16;
  constexpr int NW = proj_bwd_waves(C);
  constexpr float inv_c = 1.0f / C;
  __shared__ __attribute__((aligned(16))) u16 sx[NW][16 * RS];
  __shared__ __attribute__((aligned(16))) u16 sd[NW][16 * DRS];
  __shared__ __attribute__((aligned(16))) float red[R];
  const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
  const int wave = wave_index();
  const uint32_t P = (uint32_t)a.N * (uint32_t)a.N;
  const int H = a.H;
  const uint32_t ntiles = (P + 15u) >> 4;
  const uint32_t nw = gridDim.x * NW;

  const auto rz = make_rsrc(a.z, P * C * 2u);
  const auto rd = make_rsrc(a.dbias, (uint32_t)H * P * 2u);
  const auto rdz = make_rsrc(a.dz, P * C * 2u);
  // dbias of tile tt: lane (g, h) gets positions 16 tt + 4g .. +3 of head h
  // (zeros past the end and for h >= H): the A operand of X.
  auto load_db = [&](u32x2& d, uint32_t tt) {
    const uint32_t p0 = tt * 16u + 4u * g;
    if constexpr (EVEN) {
      d = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rd, (i < H && p0 < P) ? ((uint32_t)i * P + p0) * 2u : kOob,
                                                      0, 0));
    } else {
      uint32_t v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t off = (i < H && p0 + e < P) ? ((uint32_t)i * P + p0 + e) * 2u : kOob;
        v[e] = __builtin_amdgcn_raw_buffer_load_b16(rd, off, 0, 0);
      }
      d = u32x2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
    }
  };

  uint32_t t = blockIdx.x * NW + wave;
  // register ring as in the forward kernel; its first loads go out before the
  // parameters are read
  u32x4 zr[kStages][KT];
  u32x2 dr[kStages];
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    load_z<C>(rz, zr[s], t + s * nw, ntiles, g, i);
    load_db(dr[s], t + s * nw);
  }

  // A operand of dxhat = (gamma w)^T dbias: lane (g, r) holds row r of channel
  // tile ct -- channel 32(ct/2) + 8(r/4) + 4(ct%2) + r%4 -- on heads 4g..4g+3.
  // The result lane (g, p) then holds channels 32kt + 8g + 0..7 of position p
  // in tiles ct = 2kt (first four) and 2kt + 1 (last four): the z layout.
  u32x2 aw[2 * KT];
#pragma unroll
  for (int ct = 0; ct < 2 * KT; ++ct) {
    const int ch = 32 * (ct >> 1) + 8 * (i >> 2) + 4 * (ct & 1) + (i & 3);
    const float gm = a.gamma[ch];
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // branch-free: heads h >= H read row 0, scaled by zero
      const int h = 4 * g + e;
      v[e] = a.w[(h < H ? h : 0) * C + ch] * (h < H ? gm : 0.f);
    }
    aw[ct] = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
  }

  f32x4 xacc[2 * KT];
#pragma unroll
  for (int ct = 0; ct < 2 * KT; ++ct) xacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sacc = 0.f;
  u16* const mx = sx[wave];
  u16* const md = sd[wave];
  // transposed-read addressing: lane 4e + a4 of each group reads row 4g + e at column 4 a4
  const int e4 = (lane & 15) >> 2, a4 = lane & 3;

  auto tile = [&](const u32x4 (&z)[KT], const u32x2 dcur, uint32_t tt) {
    // the tile stays private to this wave: LDS accesses of one wave run in order
    *reinterpret_cast<u32x2*>(md + i * DRS + 4 * g) = dcur;
    float x[KT][8];
    unpack_z<KT>(z, x);
    const float rstd = normalise<KT>(x, a.eps);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      u32x4 p;
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = pack2(x[kt][2 * q], x[kt][2 * q + 1]);
      *reinterpret_cast<u32x4*>(mx + i * RS + 32 * kt + 8 * g) = p;
    }
    sacc += (__uint_as_float(dcur[0] << 16) + __uint_as_float(dcur[0] & 0xFFFF0000u)) +
            (__uint_as_float(dcur[1] << 16) + __uint_as_float(dcur[1] & 0xFFFF0000u));

    // dxhat: B operand lane (g, p) = dbias[4g..4g+3][p]
    const u32x2 bdb = lds_tr16(md + (4 * g + e4) * DRS + 4 * a4);
    float dx[KT][8];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const f32x4 lo = mfma16(aw[2 * kt], bdb, f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 hi = mfma16(aw[2 * kt + 1], bdb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dx[kt][r] = lo[r];
        dx[kt][4 + r] = hi[r];
      }
    }
    // X[h][c] += sum_p dbias[h][p] xhat[p][c]: B operand lane (g, c) = xhat[4g..4g+3][c]
#pragma unroll
    for (int ct = 0; ct < 2 * KT; ++ct)
      xacc[ct] = mfma16(dcur, lds_tr16(mx + (4 * g + e4) * RS + 16 * ct + 4 * a4), xacc[ct]);

    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        s1 += dx[kt][v];
        s2 = fmaf(dx[kt][v], x[kt][v], s2);
      }
    const float m1 = sum_over_groups(s1) * inv_c, m2 = sum_over_groups(s2) * inv_c;
    const float k1 = -rstd * m1, k2 = -rstd * m2;
    const uint32_t zoff = (tt * 16u + i) * C * 2u + 16u * g;  // past the end for positions >= P
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack2(fmaf(dx[kt][2 * q], rstd, fmaf(x[kt][2 * q], k2, k1)),
                     fmaf(dx[kt][2 * q + 1], rstd, fmaf(x[kt][2 * q + 1], k2, k1)));
      // streaming (nontemporal) store: dz, as large as z, would otherwise
      // displace the z lines this launch and the next forward read
      __builtin_amdgcn_raw_buffer_store_b128(o, rdz, zoff + 64u * kt, 0, 2);
    }
  };
  bool more = t < ntiles;
  while (more) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      if (more) {
        const int n = (s + kStages - 1) % kStages;
        load_z<C>(rz, zr[n], t + (kStages - 1) * nw, ntiles, g, i);
        load_db(dr[n], t + (kStages - 1) * nw);
        __builtin_amdgcn_sched_barrier(0);
        tile(zr[s], dr[s], t);
        t += nw;
        more = t < ntiles;
      }
    }
  }

  // workgroup sum in wave order: X at red[c * 16 + h], s at red[16 C + h]
  const float s_h = sum_over_groups(sacc);
  for (int w = 0; w < NW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int ct = 0; ct < 2 * KT; ++ct) {
        f32x4* const r = reinterpret_cast<f32x4*>(red + (16 * ct + i) * 16 + 4 * g);
        *r = w ? *r + xacc[ct] : xacc[ct];
      }
      if (g == 0) red[16 * C + i] = w ? red[16 * C + i] + s_h : s_h;
    }
    __syncthreads();
  }
  float* const part = a.partial + (size_t)blockIdx.x * R;
  for (int e = threadIdx.x; e < R; e += NW * 64) part[e] = red[e];
}

// Sum of the workgroup partials in partial-index order, then
// dw = gamma X + beta s, dgamma = sum_h w X, dbeta = sum_h w s.
template <int KT>
__global__ __launch_bounds__(kRedElems * kRedGroups) void bias_proj_reduce_kernel(ProjArgs a) {
  constexpr int C = 32 * KT;
  constexpr int R = 16 * C + 16;
  __shared__ float tot[kRedGroups][kRedElems];
  const int tid = threadIdx.x, e = tid % kRedElems, rg = tid / kRedElems;
  const int c0 = blockIdx.x * kRedCh;
  const int src = e < kRedCh * 16 ? c0 * 16 + e : 16 * C + (e - kRedCh * 16);
  // every load is issued before the first add: one memory round trip
  constexpr int kPer = (kProjBwdMaxWg + kRedGroups - 1) / kRedGroups;
  const auto rp = make_rsrc(a.partial, (uint32_t)a.nwg * R * 4u);
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int k = rg + j * kRedGroups;
    v[j] = buf_load_f32(rp, k < a.nwg ? (uint32_t)(k * R + src) * 4u : kOob);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) s += v[j];
  tot[rg][e] = s;
  __syncthreads();
  if (tid < kRedElems) {
    float v = tot[0][tid];
    for (int r = 1; r < kRedGroups; ++r) v += tot[r][tid];
    tot[0][tid] = v;
  }
  __syncthreads();
  const float* const X = tot[0];            // X[h][c0 + cl] at 16 cl + h
  const float* const S = tot[0] + kRedCh * 16;
  if (tid < kRedCh * 16) {
    const int cl = tid >> 4, h = tid & 15, c = c0 + cl;
    if (h < a.H) a.dw[h * C + c] = fmaf(a.gamma[c], X[tid], a.beta[c] * S[h]);
  }
  if (tid < kRedCh) {
    const int c = c0 + tid;
    float dg = 0.f, db = 0.f;
    for (int h = 0; h < a.H; ++h) {
      const float wv = a.w[h * C + c];
      dg = fmaf(wv, X[16 * tid + h], dg);
      db = fmaf(wv, S[h], db);
    }
    a.dgamma[c] = dg;
    a.dbeta[c] = db;
  }
}

template <int KT>
hipError_t launch_fwd_t(const ProjArgs& a, hipStream_t s, KernelTimer* timer) {
  const long long ntiles = ((long long)a.N * a.N + 15) / 16;
  const int grid = (int)std::min<long long>((ntiles + kFwdWaves - 1) / kFwdWaves, kFwdMaxWg);
  timer_start(timer, s);
  hipLaunchKernelGGL(bias_proj_fwd_kernel<KT>, dim3(grid), dim3(kFwdWaves * 64), 0, s, a);
  timer_mark(timer, s);
  return hipGetLastError();
}

template <int KT>
hipError_t launch_bwd_t(const ProjArgs& a, hipStream_t s, KernelTimer* timer) {
  timer_start(timer, s);
  const dim3 block(proj_bwd_waves(32 * KT) * 64);
  if (a.N % 2 == 0)
    hipLaunchKernelGGL((bias_proj_bwd_kernel<KT, true>), dim3(a.nwg), block, 0, s, a);
  else
    hipLaunchKernelGGL((bias_proj_bwd_kernel<KT, false>), dim3(a.nwg), block, 0, s, a);
  timer_mark(timer, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bias_proj_reduce_kernel<KT>, dim3(32 * KT / kRedCh), dim3(kRedElems * kRedGroups), 0, s, a);
  timer_mark(timer, s);
  return hipGetLastError();
}

int proj_bwd_workgroups(int N, int c) {
  const long long ntiles = ((long long)N * N + 15) / 16;
  const int nw = proj_bwd_waves(c);
  return (int)std::min<long long>((ntiles + nw - 1) / nw, kProjBwdMaxWg);
}

size_t proj_bwd_workspace_bytes(int N, int c) {
  return (size_t)proj_bwd_workgroups(N, c) * (16 * (size_t)c + 16) * sizeof(float);
}

hipError_t launch_proj_fwd(const ProjArgs& a, hipStream_t s, KernelTimer* timer) {
  switch (a.c) {
    case 32: return launch_fwd_t<1>(a, s, timer);
    case 64: return launch_fwd_t<2>(a, s, timer);
    case 128: return launch_fwd_t<4>(a, s, timer);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_proj_bwd(const ProjArgs& a, hipStream_t s, KernelTimer* timer) {
  switch (a.c) {
    case 32: return launch_bwd_t<1>(a, s, timer);
    case 64: return launch_bwd_t<2>(a, s, timer);
    case 128: return launch_bwd_t<4>(a, s, timer);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pba

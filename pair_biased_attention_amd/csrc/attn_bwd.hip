// attn_bwd.hip - backward pass of pair-biased gated attention for gfx950.
//
// The bias gradient equals the gradient of the scaled QK^T product, dS, and
// because the bias is broadcast over the batch axis in the forward pass its
// gradient is the sum of dS over that axis ("Model Efficiency" section of the
// AlphaFold3 open-source implementation page, molayo1419.me).  P is recomputed
// from Q, K, bias and the forward logsumexp instead of being stored.
//
// Four launches on the caller's stream, no host synchronisation:
//   1. attn_bwd_pre      dA = dO*sigmoid(G), dG = dO*O*(1-sigmoid(G)),
//                        D = rowsum(dO*O)  (= rowsum(P*dP), so dS = P*(dP-D))
//   2. attn_bwd_dkdv     key-stationary: each workgroup owns 32 keys of one
//                        head for a chunk of C batch rows; per row it walks all
//                        queries, accumulates dK, dV in registers, and adds dS
//                        into an LDS slab [N x 32] that sums over the chunk.
//                        The slab is written once per chunk as an fp32 partial.
//   3. attn_bwd_dq       query-stationary: recomputes P and dP per key block
//                        and accumulates dQ = dS K in registers.
//   4. bias_grad_reduce  dBias = sum of the P partials in index order.
// No floating-point atomics reach global memory; the only LDS atomics add into
// slab cells owned by a single wave, in program order, so results are bitwise
// repeatable (the deterministic-reduction principle the Design-CP page states
// for atomic float reductions).
#include "pba_device.h"
#include "pba_kernels.h"

namespace pba {

namespace {

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void kperm_slot(int kappa, int& t, int& i) {
  t = (kappa & 15) >> 2;
  i = ((kappa >> 4) << 2) | (kappa & 3);
}
__device__ __forceinline__ u16 lo16(uint32_t w) { return (u16)(w & 0xFFFFu); }
__device__ __forceinline__ u16 hi16(uint32_t w) { return (u16)(w >> 16); }
__device__ __forceinline__ float sigmoid_precise(float x) { return 1.0f / (1.0f + expf(-x)); }

// 16 bias values plane[q][k0 .. k0+15] with element-wise guards (any N);
// entries outside the [N, N] plane read as zero.
__device__ __forceinline__ void bias_row16(const u16* plane, int q, int k0, int N, u32x4& lo, u32x4& hi) {
  uint32_t w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = k0 + 2 * e;
    const uint32_t x = (q < N && k < N) ? plane[(size_t)q * N + k] : 0u;
    const uint32_t y = (q < N && k + 1 < N) ? plane[(size_t)q * N + k + 1] : 0u;
    w[e] = x | (y << 16);
  }
  lo = u32x4{w[0], w[1], w[2], w[3]};
  hi = u32x4{w[4], w[5], w[6], w[7]};
}

// 8 contiguous bf16 bias values row[k0..k0+7] (zero past N) as a u32x4.
__device__ __forceinline__ u32x4 load_bias8(const u16* row, int k0, int N, bool vec_ok) {
  if (vec_ok && k0 + 8 <= N) return ld16(row + k0);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = k0 + 2 * e;
    const uint32_t x = (k < N) ? row[k] : 0u;
    const uint32_t y = (k + 1 < N) ? row[k + 1] : 0u;
    w[e] = x | (y << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace

// ------------------------------------------------------------------ 1. pre
template <bool BF16>
__global__ void __launch_bounds__(256) attn_bwd_pre_kernel(BwdArgs a) {
  const long long rows = (long long)a.B * a.H * a.N;
  const long long row = (long long)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int d = a.d;
  float D = 0.f;
  if constexpr (BF16) {
    const u16* dO = static_cast<const u16*>(a.dout) + row * d;
    const u16* O = static_cast<const u16*>(a.out) + row * d;
    const u16* G = static_cast<const u16*>(a.g) + row * d;
    u16* dA = static_cast<u16*>(a.da) + row * d;
    u16* dG = static_cast<u16*>(a.dg) + row * d;
    for (int c = 0; c < d; c += 8) {
      const u32x4 xo = ld16(dO + c), xv = ld16(O + c), xg = ld16(G + c);
      u32x4 ra, rg;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float f[2], s[2], o[2], ga[2], gg[2];
        f[0] = bf2f(lo16(xo[e])); f[1] = bf2f(hi16(xo[e]));
        o[0] = bf2f(lo16(xv[e])); o[1] = bf2f(hi16(xv[e]));
        s[0] = sigmoid_precise(bf2f(lo16(xg[e]))); s[1] = sigmoid_precise(bf2f(hi16(xg[e])));
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          ga[z] = f[z] * s[z];
          gg[z] = f[z] * o[z] * (1.f - s[z]);
          D = fmaf(f[z], o[z], D);
        }
        ra[e] = pack2(ga[0], ga[1]);
        rg[e] = pack2(gg[0], gg[1]);
      }
      *reinterpret_cast<u32x4*>(dA + c) = ra;
      *reinterpret_cast<u32x4*>(dG + c) = rg;
    }
  } else {
    const float* dO = static_cast<const float*>(a.dout) + row * d;
    const float* O = static_cast<const float*>(a.out) + row * d;
    const float* G = static_cast<const float*>(a.g) + row * d;
    float* dA = static_cast<float*>(a.da) + row * d;
    float* dG = static_cast<float*>(a.dg) + row * d;
    for (int c = 0; c < d; ++c) {
      const float f = dO[c], o = O[c], s = sigmoid_precise(G[c]);
      dA[c] = f * s;
      dG[c] = f * o * (1.f - s);
      D = fmaf(f, o, D);
    }
  }
  a.drow[row] = D;
}

// ------------------------------------------------------------------ 2. dK, dV, dBias (bf16)
// One workgroup = 4 waves = 32 keys of one head, for a chunk of C batch rows.
// Wave (kt, qh) owns keys kb+16kt..+15 and query half qh of every 64-query
// block.  Per (row b, query block) the workgroup stages Q (scaled by
// 1/sqrt(d), exactly as the forward rounds it) and dA in row-major LDS tiles;
//   S  = Q K^T   and dP = dA V^T   read them row-wise (A operands),
//   dK^T = Q^T dS and dV^T = dA^T P read them through the transpose read.
// The next iteration's tiles, bias fragments and K/V rows are prefetched
// into registers while the current one is computed.  dS is added into an LDS
// slab [Npad x 32] (row stride 36 floats) that sums over the chunk; each slab
// cell belongs to one lane of one wave, so plain read-add-write is race free
// and ordered.  (This is the path for N > 768; shorter rows keep the sums in
// registers, see attn_bwd_dkdv_rs_kernel.)
constexpr int kSlabStride = 36;

template <int DP>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_bf16_kernel(BwdArgs a) {
  constexpr int KC = DP / 32, CT = DP / 16, RS = DP + 8;
  constexpr int NCH = DP / 32;
  // staging tiles; at batch-row boundaries the same space holds the
  // (key tile, dK|dV, ct, lane) partials of the odd query half
  constexpr int kStageBytes = 2 * 64 * RS * 2;
  constexpr int kCombBytes = 2 * 2 * CT * 64 * 16;
  static_assert(kCombBytes <= kStageBytes, "combine area must fit in the staging tiles");
  __shared__ __attribute__((aligned(16))) u16 sQA[2 * 64 * RS];  // [Q tile | dA tile]
  __shared__ __attribute__((aligned(16))) float sL[64];          // log2(e) * LSE (+inf: no keys)
  __shared__ __attribute__((aligned(16))) float sD[64];          // D = rowsum(dO * O)
  extern __shared__ float slab[];                               // [Npad][kSlabStride] when a.slab
  u16* const sQ = sQA;
  u16* const sA = sQA + 64 * RS;
  f32x4* const comb = reinterpret_cast<f32x4*>(sQA);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int kt = wave & 1, qh = wave >> 1;
  const int N = a.N, d = a.d, H = a.H;
  const int nkb = (N + 31) / 32;
  const int nqb = (N + 63) / 64;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kblk = L % nkb;
  const int hp = L / nkb;
  const int p = hp % a.P, h = hp / a.P;
  const int kb = kblk * 32;
  const int key = kb + 16 * kt + n;          // this lane's key (result column)
  const int b0 = p * a.C, b1 = min(a.B, b0 + a.C);
  const int T = (b1 - b0) * nqb;              // iterations (row, query block)
  const u16* BiasH = static_cast<const u16*>(a.bias) + (size_t)h * N * N;
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(BiasH, (uint32_t)((size_t)N * N * 2));
  const bool bias_vec = (N % 8) == 0;

  const bool keep_lane = key < N && (a.mask == nullptr || a.mask[key] != 0);
  const bool wave_masked = __any(!keep_lane);

  if (a.slab) {
    for (int idx = tid; idx < nqb * 64 * kSlabStride; idx += 256) slab[idx] = 0.f;
  }

  // ---- prefetch state (registers)
  u32x4 rq[NCH], ra[NCH];
  float rl = kPosInf, rd = 0.f;
  u32x4 rb[2];                    // bias fragments of the wave's two query tiles
  u32x4 rkn[KC], rvn[KC];         // K, V rows of the next batch row
  auto fetch = [&](int it) {      // global -> registers for iteration it
    const int b = b0 + it / nqb, qbase = (it % nqb) * 64;
    const size_t bh = (size_t)b * H + h;
#pragma unroll
    for (int c8i = 0; c8i < NCH; ++c8i) {
      const int c = tid + 256 * c8i;
      const int kappa = c / (DP / 8), c8 = c % (DP / 8);
      const int q = qbase + kappa;
      if (q < N && 8 * c8 < d) {
        rq[c8i] = ld16(static_cast<const u16*>(a.q) + (bh * N + q) * d + 8 * c8);
        ra[c8i] = ld16(static_cast<const u16*>(a.da) + (bh * N + q) * d + 8 * c8);
      } else {
        rq[c8i] = u32x4{0, 0, 0, 0};
        ra[c8i] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < 64) {
      const int q = qbase + tid;
      rl = kPosInf;
      rd = 0.f;
      if (q < N) {
        const float l = a.lse[bh * N + q];
        rl = (l == kNegInf) ? kPosInf : l * kLog2e;
        rd = a.drow[bh * N + q];
      }
    }
    // lanes g and g+2 both fetch row qa's keys kb+16kt+8(g&1)..+7; the
    // identity B operand keeps lane groups 0-1
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int qa = qbase + 16 * (2 * qh + j) + n;
      const int k0 = kb + 16 * kt + 8 * (g & 1);
      if (bias_vec) {
        rb[j] = buf_load16(brs, (uint32_t)(((size_t)qa * N + k0) * 2));
      } else {
        rb[j] = (qa < N) ? load_bias8(BiasH + (size_t)qa * N, k0, N, false) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto fetch_kv = [&](int b) {
    const size_t bh = (size_t)b * H + h;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int c0 = 32 * kc + 8 * g;
      rkn[kc] = u32x4{0, 0, 0, 0};
      rvn[kc] = u32x4{0, 0, 0, 0};
      if (key < N && c0 < d) {
        rkn[kc] = ld16(static_cast<const u16*>(a.k) + (bh * N + key) * d + c0);
        rvn[kc] = ld16(static_cast<const u16*>(a.v) + (bh * N + key) * d + c0);
      }
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int c8i = 0; c8i < NCH; ++c8i) {
      const int c = tid + 256 * c8i;
      const int kappa = c / (DP / 8), c8 = c % (DP / 8);
      u32x4 qs;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qs[e] = pack2(bf2f(lo16(rq[c8i][e])) * a.scale, bf2f(hi16(rq[c8i][e])) * a.scale);
      *reinterpret_cast<u32x4*>(&sQ[kappa * RS + 8 * c8]) = qs;
      *reinterpret_cast<u32x4*>(&sA[kappa * RS + 8 * c8]) = ra[c8i];
    }
    if (tid < 64) {
      sL[tid] = rl;
      sD[tid] = rd;
    }
  };

  const bf16x8 ident = ident_cols_frag(lane);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  bf16x8 kf[KC], vf[KC];
  f32x4 dk[CT], dv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;

  if (T > 0) {
    fetch(0);
    fetch_kv(b0);
    commit();
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      kf[kc] = as_bf8(rkn[kc]);
      vf[kc] = as_bf8(rvn[kc]);
    }
  }
  __syncthreads();

  for (int it = 0; it < T; ++it) {
    const int b = b0 + it / nqb;
    const int qblk = it % nqb, qbase = qblk * 64;
    const bool last_q = qblk == nqb - 1;
    const u32x4 bcur0 = rb[0], bcur1 = rb[1];
    if (it + 1 < T) {
      fetch(it + 1);
      if (last_q) fetch_kv(b + 1);
    }

    // ---- two 16-query tiles per wave: S, P, dP, dS
    f32x4 pj[2], dsj[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int qtile = 2 * qh + j;
      f32x4 s = mfma32(as_bf8(j == 0 ? bcur0 : bcur1), ident, zero4);
      f32x4 dp = zero4;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        s = mfma32(as_bf8(*reinterpret_cast<const u32x4*>(&sQ[(16 * qtile + n) * RS + 32 * kc + 8 * g])), kf[kc], s);
        dp = mfma32(as_bf8(*reinterpret_cast<const u32x4*>(&sA[(16 * qtile + n) * RS + 32 * kc + 8 * g])), vf[kc], dp);
      }
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[16 * qtile + 4 * g]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[16 * qtile + 4 * g]);
      f32x4 pp, ds;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pr = exp2_fast(fmaf(s[r], kLog2e, -l4[r]));
        if (wave_masked && !keep_lane) pr = 0.f;
        pp[r] = pr;
        ds[r] = pr * (dp[r] - d4[r]);
      }
      pj[j] = pp;
      dsj[j] = ds;
      if (a.slab) {
#pragma unroll
        for (int r = 0; r < 4; ++r) slab[(qbase + 16 * qtile + 4 * g + r) * kSlabStride + 16 * kt + n] += ds[r];
      } else {
        float* part = a.partial + ((size_t)b * H + h) * N * N;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = qbase + 16 * qtile + 4 * g + r;
          if (q < N && key < N) part[(size_t)q * N + key] = ds[r];
        }
      }
    }
    // ---- dV^T += dA^T P, dK^T += Q^T dS over this wave's 32 queries; the k
    // slot (g, v) is query row 32qh + 16(v/4) + 4g + v%4 on both sides
    const bf16x8 pb = pack8(pj[0], pj[1]);
    const bf16x8 dsb = pack8(dsj[0], dsj[1]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int r0 = 32 * qh + 4 * g;
      dv[ct] = mfma32(tr_frag<RS>(sA, r0, r0 + 16, 16 * ct, lane), pb, dv[ct]);
      dk[ct] = mfma32(tr_frag<RS>(sQ, r0, r0 + 16, 16 * ct, lane), dsb, dk[ct]);
    }
    __syncthreads();  // every wave is done with this iteration's tiles

    if (last_q) {
      // ---- combine the two query halves and store dK, dV of row b
      if (qh == 1) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          comb[((kt * 2 + 0) * CT + ct) * 64 + lane] = dk[ct];
          comb[((kt * 2 + 1) * CT + ct) * 64 + lane] = dv[ct];
        }
      }
      __syncthreads();
      if (qh == 0 && key < N) {
        const size_t bh = (size_t)b * H + h;
        u16* dK = static_cast<u16*>(a.dk) + bh * N * d;
        u16* dV = static_cast<u16*>(a.dv) + bh * N * d;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int c = 16 * ct + 4 * g;
          if (c >= d) continue;
          // Q was staged pre-scaled, so dK needs no further scale
          const f32x4 sk = dk[ct] + comb[((kt * 2 + 0) * CT + ct) * 64 + lane];
          const f32x4 sv = dv[ct] + comb[((kt * 2 + 1) * CT + ct) * 64 + lane];
          *reinterpret_cast<u32x2*>(dK + (size_t)key * d + c) = u32x2{pack2(sk[0], sk[1]), pack2(sk[2], sk[3])};
          *reinterpret_cast<u32x2*>(dV + (size_t)key * d + c) = u32x2{pack2(sv[0], sv[1]), pack2(sv[2], sv[3])};
        }
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        kf[kc] = as_bf8(rkn[kc]);
        vf[kc] = as_bf8(rvn[kc]);
      }
      __syncthreads();  // the combine area is the staging space
    }
    if (it + 1 < T) {
      commit();
      __syncthreads();
    }
  }

  if (a.slab) {
    __syncthreads();
    float* part = a.partial + ((size_t)p * H + h) * N * N;
    for (int idx = tid; idx < N * 32; idx += 256) {
      const int q = idx >> 5, col = idx & 31;
      if (kb + col < N) part[(size_t)q * N + kb + col] = slab[q * kSlabStride + col];
    }
  }
}

// Register-slab variant for N <= 768 (ceil(N/64) <= NQB_T): the query-block
// loop is unrolled, so each wave keeps the dBias sums of its 16 keys x (its
// half of every query block) in accumulator registers; dS of every batch row
// is added there with an identity product (no VALU, no LDS).  The sums of the
// chunk are stored once, as this workgroup's slice of partial p.
template <int DP, int NQB_T>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_rs_kernel(BwdArgs a) {
  constexpr int KC = DP / 32, CT = DP / 16, RS = DP + 8;
  constexpr int NCH = DP / 32;
  constexpr int kStageBytes = 2 * 64 * RS * 2;
  constexpr int kCombBytes = 2 * 2 * CT * 64 * 16;
  static_assert(kCombBytes <= kStageBytes, "combine area must fit in the staging tiles");
  __shared__ __attribute__((aligned(16))) u16 sQA[2 * 64 * RS];  // [Q tile | dA tile]
  __shared__ __attribute__((aligned(16))) float sL[64];
  __shared__ __attribute__((aligned(16))) float sD[64];
  u16* const sQ = sQA;
  u16* const sA = sQA + 64 * RS;
  f32x4* const comb = reinterpret_cast<f32x4*>(sQA);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int kt = wave & 1, qh = wave >> 1;
  const int N = a.N, d = a.d, H = a.H;
  const int nkb = (N + 31) / 32;
  const int nqb = (N + 63) / 64;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kblk = L % nkb;
  const int hp = L / nkb;
  const int p = hp % a.P, h = hp / a.P;
  const int kb = kblk * 32;
  const int key = kb + 16 * kt + n;
  const int b0 = p * a.C, b1 = min(a.B, b0 + a.C);
  const u16* BiasH = static_cast<const u16*>(a.bias) + (size_t)h * N * N;
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(BiasH, (uint32_t)((size_t)N * N * 2));
  const bool bias_vec = (N % 8) == 0;
  const bool keep_lane = key < N && (a.mask == nullptr || a.mask[key] != 0);
  const bool wave_masked = __any(!keep_lane);

  u32x4 rq[NCH], ra[NCH];
  float rl = kPosInf, rd = 0.f;
  u32x4 rb[2];
  u32x4 rkn[KC], rvn[KC];
  auto fetch = [&](int b, int qbase) {
    const size_t bh = (size_t)b * H + h;
#pragma unroll
    for (int c8i = 0; c8i < NCH; ++c8i) {
      const int c = tid + 256 * c8i;
      const int kappa = c / (DP / 8), c8 = c % (DP / 8);
      const int q = qbase + kappa;
      if (q < N && 8 * c8 < d) {
        rq[c8i] = ld16(static_cast<const u16*>(a.q) + (bh * N + q) * d + 8 * c8);
        ra[c8i] = ld16(static_cast<const u16*>(a.da) + (bh * N + q) * d + 8 * c8);
      } else {
        rq[c8i] = u32x4{0, 0, 0, 0};
        ra[c8i] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < 64) {
      const int q = qbase + tid;
      rl = kPosInf;
      rd = 0.f;
      if (q < N) {
        const float l = a.lse[bh * N + q];
        rl = (l == kNegInf) ? kPosInf : l * kLog2e;
        rd = a.drow[bh * N + q];
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int qa = qbase + 16 * (2 * qh + j) + n;
      const int k0 = kb + 16 * kt + 8 * (g & 1);
      if (bias_vec) rb[j] = buf_load16(brs, (uint32_t)(((size_t)qa * N + k0) * 2));
      else rb[j] = (qa < N) ? load_bias8(BiasH + (size_t)qa * N, k0, N, false) : u32x4{0, 0, 0, 0};
    }
  };
  auto fetch_kv = [&](int b) {
    const size_t bh = (size_t)b * H + h;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int c0 = 32 * kc + 8 * g;
      rkn[kc] = u32x4{0, 0, 0, 0};
      rvn[kc] = u32x4{0, 0, 0, 0};
      if (key < N && c0 < d) {
        rkn[kc] = ld16(static_cast<const u16*>(a.k) + (bh * N + key) * d + c0);
        rvn[kc] = ld16(static_cast<const u16*>(a.v) + (bh * N + key) * d + c0);
      }
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int c8i = 0; c8i < NCH; ++c8i) {
      const int c = tid + 256 * c8i;
      const int kappa = c / (DP / 8), c8 = c % (DP / 8);
      u32x4 qs;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qs[e] = pack2(bf2f(lo16(rq[c8i][e])) * a.scale, bf2f(hi16(rq[c8i][e])) * a.scale);
      *reinterpret_cast<u32x4*>(&sQ[kappa * RS + 8 * c8]) = qs;
      *reinterpret_cast<u32x4*>(&sA[kappa * RS + 8 * c8]) = ra[c8i];
    }
    if (tid < 64) {
      sL[tid] = rl;
      sD[tid] = rd;
    }
  };

  const bf16x8 ident = ident_cols_frag(lane);
  const bf16x8 id_lo = ident_rows_frag(lane, 0), id_hi = ident_rows_frag(lane, 1);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  bf16x8 kf[KC], vf[KC];
  f32x4 dk[CT], dv[CT];
  f32x4 sacc[NQB_T][2];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;
#pragma unroll
  for (int qb = 0; qb < NQB_T; ++qb) sacc[qb][0] = sacc[qb][1] = zero4;

  if (b0 < b1) {
    fetch(b0, 0);
    fetch_kv(b0);
    commit();
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      kf[kc] = as_bf8(rkn[kc]);
      vf[kc] = as_bf8(rvn[kc]);
    }
  }
  __syncthreads();

  for (int b = b0; b < b1; ++b) {
#pragma unroll
    for (int qblk = 0; qblk < NQB_T; ++qblk) {
      if (qblk < nqb) {
        const int qbase = qblk * 64;
        const bool last_q = qblk == nqb - 1;
        const bool has_next = !(last_q && b + 1 >= b1);
        const u32x4 bcur0 = rb[0], bcur1 = rb[1];
        if (has_next) {
          if (last_q) {
            fetch(b + 1, 0);
            fetch_kv(b + 1);
          } else {
            fetch(b, qbase + 64);
          }
        }

        f32x4 pj[2], dsj[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int qtile = 2 * qh + j;
          f32x4 s = mfma32(as_bf8(j == 0 ? bcur0 : bcur1), ident, zero4);
          f32x4 dp = zero4;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            s = mfma32(as_bf8(*reinterpret_cast<const u32x4*>(&sQ[(16 * qtile + n) * RS + 32 * kc + 8 * g])), kf[kc], s);
            dp = mfma32(as_bf8(*reinterpret_cast<const u32x4*>(&sA[(16 * qtile + n) * RS + 32 * kc + 8 * g])), vf[kc], dp);
          }
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[16 * qtile + 4 * g]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[16 * qtile + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float pr = exp2_fast(fmaf(s[r], kLog2e, -l4[r]));
            if (wave_masked && !keep_lane) pr = 0.f;
            pj[j][r] = pr;
            dsj[j][r] = pr * (dp[r] - d4[r]);
          }
        }
        const bf16x8 pb = pack8(pj[0], pj[1]);
        const bf16x8 dsb = pack8(dsj[0], dsj[1]);
        // dBias sums: rows of query tile 2qh+j, the same rounded dS as dK uses
        sacc[qblk][0] = mfma32(id_lo, dsb, sacc[qblk][0]);
        sacc[qblk][1] = mfma32(id_hi, dsb, sacc[qblk][1]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int r0 = 32 * qh + 4 * g;
          dv[ct] = mfma32(tr_frag<RS>(sA, r0, r0 + 16, 16 * ct, lane), pb, dv[ct]);
          dk[ct] = mfma32(tr_frag<RS>(sQ, r0, r0 + 16, 16 * ct, lane), dsb, dk[ct]);
        }
        __syncthreads();

        if (last_q) {
          if (qh == 1) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              comb[((kt * 2 + 0) * CT + ct) * 64 + lane] = dk[ct];
              comb[((kt * 2 + 1) * CT + ct) * 64 + lane] = dv[ct];
            }
          }
          __syncthreads();
          if (qh == 0 && key < N) {
            const size_t bh = (size_t)b * H + h;
            u16* dK = static_cast<u16*>(a.dk) + bh * N * d;
            u16* dV = static_cast<u16*>(a.dv) + bh * N * d;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              const int c = 16 * ct + 4 * g;
              if (c >= d) continue;
              const f32x4 sk = dk[ct] + comb[((kt * 2 + 0) * CT + ct) * 64 + lane];
              const f32x4 sv = dv[ct] + comb[((kt * 2 + 1) * CT + ct) * 64 + lane];
              *reinterpret_cast<u32x2*>(dK + (size_t)key * d + c) = u32x2{pack2(sk[0], sk[1]), pack2(sk[2], sk[3])};
              *reinterpret_cast<u32x2*>(dV + (size_t)key * d + c) = u32x2{pack2(sv[0], sv[1]), pack2(sv[2], sv[3])};
            }
          }
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            kf[kc] = as_bf8(rkn[kc]);
            vf[kc] = as_bf8(rvn[kc]);
          }
          __syncthreads();
        }
        if (has_next) {
          commit();
          __syncthreads();
        }
      }
    }
  }

  // this chunk's dBias sums -> partial p
  if (key < N) {
    float* part = a.partial + ((size_t)p * H + h) * N * N;
#pragma unroll
    for (int qblk = 0; qblk < NQB_T; ++qblk) {
      if (qblk < nqb) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = qblk * 64 + 16 * (2 * qh + j) + 4 * g + r;
            if (q < N) part[(size_t)q * N + key] = sacc[qblk][j][r];
          }
      }
    }
  }
}

// ------------------------------------------------------------------ 3. dQ (bf16)
// Same decomposition as the forward kernel: 4 waves x 16*QT queries of one
// (b, h), 64-key blocks of K and V double-buffered in LDS in row-major form.
// S^T = K Q^T and dP^T = V dA^T read K and V row-wise; dQ^T = K^T dS^T reads
// K through the transpose read.
template <int DP, int QT, bool ALIGNED>
__global__ void __launch_bounds__(256) attn_bwd_dq_bf16_kernel(BwdArgs a, int nqblocks) {
  constexpr int KC = DP / 32, CT = DP / 16, RS = DP + 8;
  constexpr int QW = 16 * QT, QBLK = 4 * QW;
  constexpr int NCH = DP / 32;
  __shared__ __attribute__((aligned(16))) u16 sK[2][64 * RS];
  __shared__ __attribute__((aligned(16))) u16 sV[2][64 * RS];
  __shared__ uint32_t sKeep[2][16];
  __shared__ int sAny[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, ln = lane & 15;
  const int N = a.N, d = a.d;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = L % nqblocks;
  const int bh_lin = L / nqblocks;
  const int h = bh_lin / a.B, b = bh_lin % a.B;
  const size_t bh = (size_t)b * a.H + h;
  const u16* Q = static_cast<const u16*>(a.q) + bh * N * d;
  const u16* K = static_cast<const u16*>(a.k) + bh * N * d;
  const u16* V = static_cast<const u16*>(a.v) + bh * N * d;
  const u16* dA = static_cast<const u16*>(a.da) + bh * N * d;
  const u16* BiasH = static_cast<const u16*>(a.bias) + (size_t)h * N * N;
  const float* lse = a.lse + bh * N;
  const float* drow = a.drow + bh * N;
  u16* dQ = static_cast<u16*>(a.dq) + bh * N * d;
  const int q0 = qb * QBLK + wave * QW;
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(BiasH, (uint32_t)((size_t)N * N * 2));

  u32x4 rk[NCH], rv[NCH];
  bool rkeep = true;
  auto fetch = [&](int kb) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int c = tid + 256 * it;
      const int kappa = c / (DP / 8), c8 = c % (DP / 8);
      const int key = kb + kappa;
      if (key < N && 8 * c8 < d) {
        rk[it] = ld16(K + (size_t)key * d + 8 * c8);
        rv[it] = ld16(V + (size_t)key * d + 8 * c8);
      } else {
        rk[it] = u32x4{0, 0, 0, 0};
        rv[it] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < 64) {
      const int key = kb + tid;
      rkeep = key < N && (a.mask == nullptr || a.mask[key] != 0);
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int c = tid + 256 * it;
      const int kappa = c / (DP / 8), c8 = c % (DP / 8);
      *reinterpret_cast<u32x4*>(&sK[buf][kappa * RS + 8 * c8]) = rk[it];
      *reinterpret_cast<u32x4*>(&sV[buf][kappa * RS + 8 * c8]) = rv[it];
    }
    if (tid < 64) {
      reinterpret_cast<uint8_t*>(&sKeep[buf][0])[tid] = rkeep ? 1 : 0;
      const unsigned long long bal = __ballot(!rkeep);
      if (tid == 0) sAny[buf] = bal != 0ull;
    }
  };

  bf16x8 qf[QT][KC], daf[QT][KC];
  float l2[QT], dd[QT];
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    const int qrow = q0 + 16 * s + ln;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int c0 = 32 * kc + 8 * g;
      u32x4 raw = u32x4{0, 0, 0, 0}, rda = u32x4{0, 0, 0, 0};
      if (qrow < N && c0 < d) {
        raw = ld16(Q + (size_t)qrow * d + c0);
        rda = ld16(dA + (size_t)qrow * d + c0);
      }
      u32x4 sc;
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = pack2(bf2f(lo16(raw[e])) * a.scale, bf2f(hi16(raw[e])) * a.scale);
      qf[s][kc] = as_bf8(sc);
      daf[s][kc] = as_bf8(rda);
    }
    float l = kNegInf, dv = 0.f;
    if (qrow < N) {
      l = lse[qrow];
      dv = drow[qrow];
    }
    l2[s] = (l == kNegInf) ? kPosInf : l * kLog2e;  // rows without keys: P = 0
    dd[s] = dv;
  }

  const bf16x8 id_lo = ident_rows_frag(lane, 0), id_hi = ident_rows_frag(lane, 1);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 dq[QT][CT];
#pragma unroll
  for (int s = 0; s < QT; ++s)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) dq[s][ct] = zero4;
  const int krow = 16 * (ln >> 2) + (ln & 3);

  const int nkb = (N + 63) / 64;
  fetch(0);
  commit(0);
  __syncthreads();
  for (int blk = 0; blk < nkb; ++blk) {
    const int buf = blk & 1;
    const int kb = blk * 64;
    if (blk + 1 < nkb) fetch(kb + 64);

    bf16x8 kf[4][KC], vf[4][KC], kt[CT][2];
    const u16* tK = sK[buf];
    const u16* tV = sV[buf];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        kf[t][kc] = as_bf8(*reinterpret_cast<const u32x4*>(tK + (krow + 4 * t) * RS + 32 * kc + 8 * g));
        vf[t][kc] = as_bf8(*reinterpret_cast<const u32x4*>(tV + (krow + 4 * t) * RS + 32 * kc + 8 * g));
      }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int m = 0; m < 2; ++m) kt[ct][m] = tr_frag<RS>(tK, 16 * g + 8 * m, 16 * g + 8 * m + 4, 16 * ct, lane);

    const bool masked_blk = sAny[buf] != 0;
    u32x4 mlo = u32x4{0, 0, 0, 0}, mhi = u32x4{0, 0, 0, 0};
    if (masked_blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kw = sKeep[buf][4 * g + e];
        const uint32_t m01 = ((kw & 0xFFu) ? 0u : 0xFFFFu) | ((kw & 0xFF00u) ? 0u : 0xFFFF0000u);
        const uint32_t m23 = ((kw & 0xFF0000u) ? 0u : 0xFFFFu) | ((kw & 0xFF000000u) ? 0u : 0xFFFF0000u);
        if (e < 2) { mlo[2 * e] = m01; mlo[2 * e + 1] = m23; }
        else { mhi[2 * (e - 2)] = m01; mhi[2 * (e - 2) + 1] = m23; }
      }
    }
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      const int qrow = q0 + 16 * s + ln;
      u32x4 blo, bhi;
      if constexpr (ALIGNED) {
        const uint32_t boff = (uint32_t)(((size_t)qrow * N + kb + 16 * g) * 2);
        blo = buf_load16(brs, boff);
        bhi = buf_load16(brs, boff + 16);
      } else {
        bias_row16(BiasH, qrow, kb + 16 * g, N, blo, bhi);
      }
      if (masked_blk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          blo[e] = (blo[e] & ~mlo[e]) | (kMaskedBias2 & mlo[e]);
          bhi[e] = (bhi[e] & ~mhi[e]) | (kMaskedBias2 & mhi[e]);
        }
      }
      f32x4 acc[4], dp[4];
      acc[0] = mfma32(id_lo, as_bf8(blo), zero4);
      acc[1] = mfma32(id_hi, as_bf8(blo), zero4);
      acc[2] = mfma32(id_lo, as_bf8(bhi), zero4);
      acc[3] = mfma32(id_hi, as_bf8(bhi), zero4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        dp[t] = zero4;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          acc[t] = mfma32(kf[t][kc], qf[s][kc], acc[t]);
          dp[t] = mfma32(vf[t][kc], daf[s][kc], dp[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = exp2_fast(fmaf(acc[t][r], kLog2e, -l2[s]));
          acc[t][r] = pr * (dp[t][r] - dd[s]);
        }
      const bf16x8 s0 = pack8(acc[0], acc[1]);
      const bf16x8 s1 = pack8(acc[2], acc[3]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        dq[s][ct] = mfma32(kt[ct][0], s0, dq[s][ct]);
        dq[s][ct] = mfma32(kt[ct][1], s1, dq[s][ct]);
      }
    }
    if (blk + 1 < nkb) commit(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int s = 0; s < QT; ++s) {
    const int qrow = q0 + 16 * s + ln;
    if (qrow >= N) continue;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = 16 * ct + 4 * g;
      if (c >= d) continue;
      const f32x4 o = dq[s][ct] * a.scale;
      *reinterpret_cast<u32x2*>(dQ + (size_t)qrow * d + c) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
    }
  }
}

// ------------------------------------------------------------------ fp32 variants
// fp32 inputs use v_mfma_f32_16x16x4_f32 with the same decomposition; these
// kernels keep plain row-major LDS tiles (the fp32 case is the small one).
template <int DP>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_f32_kernel(BwdArgs a) {
  constexpr int CT = DP / 16, KC4 = DP / 4, RS = DP + 1;
  __shared__ float sq[64 * RS];    // Q (unscaled) rows of the query block
  __shared__ float sda[64 * RS];   // dA rows
  __shared__ float slse2[64], sdd[64];
  __shared__ f32x4 comb[2 * 2 * CT * 64];
  extern __shared__ float slab[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int kt = wave & 1, qh = wave >> 1;
  const int N = a.N, d = a.d, H = a.H;
  const int nkb = (N + 31) / 32, nqb = (N + 63) / 64;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kblk = L % nkb;
  const int hp = L / nkb;
  const int p = hp % a.P, h = hp / a.P;
  const int kb = kblk * 32;
  const int key = kb + 16 * kt + n;
  const int b0 = p * a.C, b1 = min(a.B, b0 + a.C);
  const float* Bias = static_cast<const float*>(a.bias) + (size_t)h * N * N;
  const bool keep_lane = key < N && (a.mask == nullptr || a.mask[key] != 0);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  if (a.slab) {
    for (int idx = tid; idx < nqb * 64 * kSlabStride; idx += 256) slab[idx] = 0.f;
  }
  for (int b = b0; b < b1; ++b) {
    const size_t bh = (size_t)b * H + h;
    const float* Q = static_cast<const float*>(a.q) + bh * N * d;
    const float* K = static_cast<const float*>(a.k) + bh * N * d;
    const float* V = static_cast<const float*>(a.v) + bh * N * d;
    const float* dA = static_cast<const float*>(a.da) + bh * N * d;
    float kf[KC4], vf[KC4];
#pragma unroll
    for (int kc = 0; kc < KC4; ++kc) {
      const int c = 4 * kc + g;
      kf[kc] = (key < N && c < d) ? K[(size_t)key * d + c] : 0.f;
      vf[kc] = (key < N && c < d) ? V[(size_t)key * d + c] : 0.f;
    }
    f32x4 dk[CT], dv[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;
    for (int qblk = 0; qblk < nqb; ++qblk) {
      const int qbase = qblk * 64;
      __syncthreads();
      for (int idx = tid; idx < 64 * DP; idx += 256) {
        const int r = idx / DP, c = idx % DP, q = qbase + r;
        const bool ok = q < N && c < d;
        sq[r * RS + c] = ok ? Q[(size_t)q * d + c] : 0.f;
        sda[r * RS + c] = ok ? dA[(size_t)q * d + c] : 0.f;
      }
      if (tid < 64) {
        const int q = qbase + tid;
        float l2 = kPosInf, dd = 0.f;
        if (q < N) {
          const float l = a.lse[bh * N + q];
          l2 = (l == kNegInf) ? kPosInf : l * kLog2e;
          dd = a.drow[bh * N + q];
        }
        slse2[tid] = l2;
        sdd[tid] = dd;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int qtile = 2 * qh + j;
        const int qt0 = 16 * qtile;  // row offset inside the block
        f32x4 s, dp = zero4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = qbase + qt0 + 4 * g + r;
          s[r] = (q < N && key < N) ? Bias[(size_t)q * N + key] : 0.f;
        }
#pragma unroll
        for (int kc = 0; kc < KC4; ++kc) {
          s = mfma4f(sq[(qt0 + n) * RS + 4 * kc + g] * a.scale, kf[kc], s);
          dp = mfma4f(sda[(qt0 + n) * RS + 4 * kc + g], vf[kc], dp);
        }
        f32x4 pp, ds;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = qt0 + 4 * g + r;
          float pr = exp2_fast(fmaf(s[r], kLog2e, -slse2[row]));
          if (!keep_lane) pr = 0.f;
          pp[r] = pr;
          ds[r] = pr * (dp[r] - sdd[row]);
        }
        if (a.slab) {
#pragma unroll
          for (int r = 0; r < 4; ++r) slab[(qbase + qt0 + 4 * g + r) * kSlabStride + 16 * kt + n] += ds[r];
        } else {
          float* part = a.partial + ((size_t)b * H + h) * N * N;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = qbase + qt0 + 4 * g + r;
            if (q < N && key < N) part[(size_t)q * N + key] = ds[r];
          }
        }
        // dV^T += dA^T P and dK^T += Q^T dS, one query (k slot) per lane group
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = qt0 + 4 * g + r;
            dv[ct] = mfma4f(sda[row * RS + 16 * ct + n], pp[r], dv[ct]);
            dk[ct] = mfma4f(sq[row * RS + 16 * ct + n], ds[r], dk[ct]);
          }
      }
    }
    __syncthreads();
    if (qh == 1) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        comb[((kt * 2 + 0) * CT + ct) * 64 + lane] = dk[ct];
        comb[((kt * 2 + 1) * CT + ct) * 64 + lane] = dv[ct];
      }
    }
    __syncthreads();
    if (qh == 0 && key < N) {
      float* dK = static_cast<float*>(a.dk) + bh * N * d;
      float* dV = static_cast<float*>(a.dv) + bh * N * d;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 16 * ct + 4 * g;
        if (c >= d) continue;
        const f32x4 sk = (dk[ct] + comb[((kt * 2 + 0) * CT + ct) * 64 + lane]) * a.scale;
        const f32x4 sv = dv[ct] + comb[((kt * 2 + 1) * CT + ct) * 64 + lane];
        *reinterpret_cast<f32x4*>(dK + (size_t)key * d + c) = sk;
        *reinterpret_cast<f32x4*>(dV + (size_t)key * d + c) = sv;
      }
    }
  }
  if (a.slab) {
    __syncthreads();
    float* part = a.partial + ((size_t)p * H + h) * N * N;
    for (int idx = tid; idx < N * 32; idx += 256) {
      const int q = idx >> 5, col = idx & 31;
      if (kb + col < N) part[(size_t)q * N + kb + col] = slab[q * kSlabStride + col];
    }
  }
}

template <int DP>
__global__ void __launch_bounds__(256) attn_bwd_dq_f32_kernel(BwdArgs a, int nqblocks) {
  constexpr int CT = DP / 16, KC4 = DP / 4, RS = DP + 1;
  __shared__ float sk[64 * RS];
  __shared__ float sv[64 * RS];
  __shared__ uint8_t skeep[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, ln = lane & 15;
  const int N = a.N, d = a.d;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = L % nqblocks;
  const int bh_lin = L / nqblocks;
  const int h = bh_lin / a.B, b = bh_lin % a.B;
  const size_t bh = (size_t)b * a.H + h;
  const float* Q = static_cast<const float*>(a.q) + bh * N * d;
  const float* K = static_cast<const float*>(a.k) + bh * N * d;
  const float* V = static_cast<const float*>(a.v) + bh * N * d;
  const float* dA = static_cast<const float*>(a.da) + bh * N * d;
  const float* Bias = static_cast<const float*>(a.bias) + (size_t)h * N * N;
  float* dQ = static_cast<float*>(a.dq) + bh * N * d;
  const int qrow = qb * 64 + wave * 16 + ln;

  float qf[KC4], daf[KC4];
#pragma unroll
  for (int kc = 0; kc < KC4; ++kc) {
    const int c = 4 * kc + g;
    const bool ok = qrow < N && c < d;
    qf[kc] = ok ? Q[(size_t)qrow * d + c] * a.scale : 0.f;
    daf[kc] = ok ? dA[(size_t)qrow * d + c] : 0.f;
  }
  float l2 = kPosInf, dd = 0.f;
  if (qrow < N) {
    const float l = a.lse[bh * N + qrow];
    l2 = (l == kNegInf) ? kPosInf : l * kLog2e;
    dd = a.drow[bh * N + qrow];
  }
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 dq[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) dq[ct] = zero4;

  const int nkb = (N + 63) / 64;
  for (int blk = 0; blk < nkb; ++blk) {
    const int kb = blk * 64;
    __syncthreads();
    for (int idx = tid; idx < 64 * DP; idx += 256) {
      const int r = idx / DP, c = idx % DP, key = kb + r;
      const bool ok = key < N && c < d;
      sk[r * RS + c] = ok ? K[(size_t)key * d + c] : 0.f;
      sv[r * RS + c] = ok ? V[(size_t)key * d + c] : 0.f;
    }
    if (tid < 64) {
      const int key = kb + tid;
      skeep[tid] = (key < N && (a.mask == nullptr || a.mask[key] != 0)) ? 1 : 0;
    }
    __syncthreads();
    // S^T and dP^T tiles: key row 16g' + 4t + r of the block is result row i = 4g'+r of tile t
    f32x4 acc[4], dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 16 * g + 4 * t + r;
        acc[t][r] = (qrow < N && key < N) ? Bias[(size_t)qrow * N + key] : 0.f;
      }
      dp[t] = zero4;
      const int krow = 16 * (ln >> 2) + 4 * t + (ln & 3);  // A-operand row i = ln
#pragma unroll
      for (int kc = 0; kc < KC4; ++kc) {
        acc[t] = mfma4f(sk[krow * RS + 4 * kc + g], qf[kc], acc[t]);
        dp[t] = mfma4f(sv[krow * RS + 4 * kc + g], daf[kc], dp[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kl = 16 * g + 4 * t + r;
        float pr = exp2_fast(fmaf(acc[t][r], kLog2e, -l2));
        if (!skeep[kl]) pr = 0.f;
        acc[t][r] = pr * (dp[t][r] - dd);
      }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[ct] = mfma4f(sk[(16 * g + 4 * t + r) * RS + 16 * ct + ln], acc[t][r], dq[ct]);
  }
  if (qrow < N) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = 16 * ct + 4 * g;
      if (c >= d) continue;
      *reinterpret_cast<f32x4*>(dQ + (size_t)qrow * d + c) = dq[ct] * a.scale;
    }
  }
}

// ------------------------------------------------------------------ 4. reduce
template <bool BF16>
__global__ void __launch_bounds__(256) bias_grad_reduce_kernel(const float* partial, int P, size_t count, void* out) {
  const size_t i4 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= count) return;
  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 s = {0.f, 0.f, 0.f, 0.f};
  if (i4 + 4 <= count && (count & 3) == 0) {  // every partial plane stays 16-byte aligned
    for (int p = 0; p < P; ++p) s += *reinterpret_cast<const f4*>(partial + (size_t)p * count + i4);
  } else {
    for (int p = 0; p < P; ++p)
      for (int e = 0; e < 4; ++e)
        if (i4 + e < count) s[e] += partial[(size_t)p * count + i4 + e];
  }
  for (int e = 0; e < 4; ++e) {
    if (i4 + e >= count) break;
    if constexpr (BF16) static_cast<u16*>(out)[i4 + e] = f2bf(s[e]);
    else static_cast<float*>(out)[i4 + e] = s[e];
  }
}

// ------------------------------------------------------------------ plan + launch
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static int slab_bytes(int N) { return ((N + 63) / 64) * 64 * kSlabStride * 4; }

// Batch rows per chunk so that the dK/dV launch has about 1024 workgroups.
static void pick_chunks(int B, long long per_chunk, int& P, int& C) {
  P = (int)std::min<long long>(B, std::max<long long>(1, (1024 + per_chunk - 1) / per_chunk));
  C = (B + P - 1) / P;
  P = (B + C - 1) / C;
}

BwdPlan plan_attn_bwd(int B, int H, int N, int d, bool bf16) {
  BwdPlan pl{};
  const size_t rows = (size_t)B * H * N;
  const long long per_chunk = (long long)H * ((N + 31) / 32);
  if (bf16 && N <= 768) {
    pl.slab = 2;  // dBias sums in registers
    pick_chunks(B, per_chunk, pl.P, pl.C);
  } else if (B > 1 && slab_bytes(N) <= 112 * 1024) {
    pl.slab = 1;  // dBias sums in an LDS slab
    pick_chunks(B, per_chunk, pl.P, pl.C);
  } else {
    pl.slab = 0;  // one partial per batch row
    pl.C = 1;
    pl.P = B;
  }
  size_t off = 0;
  pl.off_da = off;
  off = align256(off + rows * d * (bf16 ? 2 : 4));
  pl.off_drow = off;
  off = align256(off + rows * 4);
  pl.off_partial = off;
  off = align256(off + (size_t)pl.P * H * N * N * 4);
  pl.total = off;
  return pl;
}

hipError_t launch_attn_bwd(const BwdArgs& args, bool bf16, hipStream_t stream) {
  BwdArgs a = args;
  const int dp = a.d <= 32 ? 32 : 64;
  const long long rows = (long long)a.B * a.H * a.N;
  const long long bhs = (long long)a.B * a.H;
  hipError_t e;

  // 1. preprocess
  {
    const dim3 grid((unsigned)((rows + 255) / 256));
    if (bf16) hipLaunchKernelGGL(attn_bwd_pre_kernel<true>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(attn_bwd_pre_kernel<false>, grid, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 2. dK, dV, dBias partials
  {
    const int nkb = (a.N + 31) / 32;
    const dim3 grid((unsigned)((long long)a.H * a.P * nkb));
    if (a.slab == 2) {
      const int nqb = (a.N + 63) / 64;
      const int nt = nqb <= 4 ? 4 : nqb <= 6 ? 6 : nqb <= 8 ? 8 : 12;
#define PBA_RS_LAUNCH(DPV, NQV) \
  hipLaunchKernelGGL((attn_bwd_dkdv_rs_kernel<DPV, NQV>), grid, dim3(256), 0, stream, a)
      if (dp == 32) {
        if (nt == 4) PBA_RS_LAUNCH(32, 4); else if (nt == 6) PBA_RS_LAUNCH(32, 6);
        else if (nt == 8) PBA_RS_LAUNCH(32, 8); else PBA_RS_LAUNCH(32, 12);
      } else {
        if (nt == 4) PBA_RS_LAUNCH(64, 4); else if (nt == 6) PBA_RS_LAUNCH(64, 6);
        else if (nt == 8) PBA_RS_LAUNCH(64, 8); else PBA_RS_LAUNCH(64, 12);
      }
#undef PBA_RS_LAUNCH
    } else {
      const size_t shmem = a.slab ? (size_t)slab_bytes(a.N) : 0;
      if (shmem > 64 * 1024) {
        // the slab can exceed the default 64 KiB dynamic LDS limit
        const void* fns[4] = {reinterpret_cast<const void*>(&attn_bwd_dkdv_bf16_kernel<32>),
                              reinterpret_cast<const void*>(&attn_bwd_dkdv_bf16_kernel<64>),
                              reinterpret_cast<const void*>(&attn_bwd_dkdv_f32_kernel<32>),
                              reinterpret_cast<const void*>(&attn_bwd_dkdv_f32_kernel<64>)};
        for (const void* f : fns) {
          if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem)) != hipSuccess)
            return e;
        }
      }
      if (bf16) {
        if (dp == 32) hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<32>, grid, dim3(256), shmem, stream, a);
        else hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<64>, grid, dim3(256), shmem, stream, a);
      } else {
        if (dp == 32) hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<32>, grid, dim3(256), shmem, stream, a);
        else hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<64>, grid, dim3(256), shmem, stream, a);
      }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 3. dQ
  {
    if (bf16) {
      const bool qt2 = dp == 32 && bhs * ((a.N + 127) / 128) >= 1024;
      const bool al = (a.N % 8) == 0;
      const int nqb = qt2 ? (a.N + 127) / 128 : (a.N + 63) / 64;
      const dim3 grid((unsigned)(bhs * nqb));
#define PBA_DQ_LAUNCH(DPV, QTV, ALV) \
  hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<DPV, QTV, ALV>), grid, dim3(256), 0, stream, a, nqb)
      if (dp == 32) {
        if (qt2) { if (al) PBA_DQ_LAUNCH(32, 2, true); else PBA_DQ_LAUNCH(32, 2, false); }
        else { if (al) PBA_DQ_LAUNCH(32, 1, true); else PBA_DQ_LAUNCH(32, 1, false); }
      } else {
        if (qt2) { if (al) PBA_DQ_LAUNCH(64, 2, true); else PBA_DQ_LAUNCH(64, 2, false); }
        else { if (al) PBA_DQ_LAUNCH(64, 1, true); else PBA_DQ_LAUNCH(64, 1, false); }
      }
#undef PBA_DQ_LAUNCH
    } else {
      const int nqb = (a.N + 63) / 64;
      const dim3 grid((unsigned)(bhs * nqb));
      if (dp == 32) hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<32>, grid, dim3(256), 0, stream, a, nqb);
      else hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<64>, grid, dim3(256), 0, stream, a, nqb);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 4. dBias = sum of partials
  {
    const size_t count = (size_t)a.H * a.N * a.N;
    const dim3 grid((unsigned)((count / 4 + 255) / 256 + 1));
    if (bf16) hipLaunchKernelGGL(bias_grad_reduce_kernel<true>, grid, dim3(256), 0, stream, a.partial, a.P, count, a.dbias);
    else hipLaunchKernelGGL(bias_grad_reduce_kernel<false>, grid, dim3(256), 0, stream, a.partial, a.P, count, a.dbias);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pba

// attn_bwd.hip - backward pass of pair-biased gated attention for gfx950.
//
// The bias gradient equals the gradient of the scaled QK^T product, dS, and
// because the bias is broadcast over the batch axis in the forward pass its
// gradient is the sum of dS over that axis ("Model Efficiency" section of the
// AlphaFold3 open-source implementation page, molayo1419.me).  P is recomputed
// from Q, K, bias and the forward logsumexp instead of being stored.
//
// Launches on the caller's stream, no host synchronisation:
//   1. attn_bwd_pre      dA = dO*sigmoid(G), dG = dO*O*(1-sigmoid(G)),
//                        D = rowsum(dO*O)  (= rowsum(P*dP), so dS = P*(dP-D)),
//                        and (bf16) the row seeds (-log2(e) * LSE, -D) of the
//                        two gradient roles
//   2. one launch with two roles (bf16; two launches of the same kernel when
//      the dK/dV role's LDS slab leaves room for only one workgroup per CU):
//      - key-stationary dK/dV tiles, first in the grid: a workgroup owns 32
//        keys of one head for a chunk of C batch rows; per row it walks all
//        queries in 64-query blocks, accumulates dK, dV in registers and adds
//        dS into a dBias slab [N x 32] (registers for d <= 32 and an even count
//        of at most six query blocks, LDS otherwise) that sums over the chunk
//        and is written once per chunk as an fp32 partial.  On grids that
//        fill the chip with N <= 384, N % 8 == 0 and d <= 32 the tile takes
//        128-query steps instead, its operands staged by LDS-destination loads;
//      - query-stationary dQ tiles, filling the rest: P and dP recomputed per
//        64-key block, dQ = dS K accumulated in registers.  Grids too small
//        to fill the chip (B H ceil(N/64) < 512) take key-split dQ tiles
//        instead: one 16-query tile per workgroup, its four waves each over a
//        quarter of the key blocks, partial dQ summed in wave order.  When
//        the two launches are separate, the dQ launch runs a kernel instance
//        without the dK/dV role (fewer registers).
//      (fp32: attn_bwd_dkdv_f32 and attn_bwd_dq_f32, two launches.)
//   3. bias_grad_reduce  dBias = sum of the P partials in index order (skipped
//                        for one batch row, where dS is stored as dBias).
// No floating-point atomics anywhere; every slab cell is owned by a single
// wave and updated in program order, so results are bitwise repeatable (the
// deterministic-reduction principle the Design-CP page states for atomic
// float reductions).
#include <algorithm>
#include <type_traits>

#include "pba_device.h"
#include "pba_kernels.h"

namespace pba {

namespace {

// fp32 dK/dV kernel: LDS slab row stride (floats) for 32 keys, padded
constexpr int kSlabStride = 36;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
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
// bf16: one lane per 16-byte chunk of a row (L = d/8 lanes per row, 256/L
// rows per workgroup), so every load and store is a coalesced 16-byte access;
// D is summed over a row's lanes by a butterfly in a fixed order.
__global__ void __launch_bounds__(256) attn_bwd_pre_bf16_kernel(BwdArgs a, int lanes_log2) {
  // each row takes 2^lanes_log2 consecutive lanes (d / 8 rounded up to a
  // power of two), lane c its channels 8c .. 8c + 7; the row sum D is a
  // butterfly over those lanes, so there is no LDS and no barrier, and the
  // row's LSE is requested together with the other loads
  const int tid = threadIdx.x;
  const int lanes = 1 << lanes_log2;
  const long long rows = (long long)a.B * a.H * a.N;
  const long long row = (long long)blockIdx.x * (256 >> lanes_log2) + (tid >> lanes_log2);
  const int c = tid & (lanes - 1);
  const bool live = row < rows && 8 * c < a.d;
  const float l = (row < rows && c == 0) ? a.lse[row] : 0.f;
  float D = 0.f;
  if (live) {
    // dO, O and G are read only here and dG is written only here, so they go
    // through the caches as streaming (nontemporal) accesses and do not evict
    // the tensors the next launch reads again (Q, K, V, dA, bias, seeds)
    const size_t off = (size_t)row * a.d + 8 * c;
    const u32x4 xo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const u16*>(a.dout) + off));
    const u32x4 xv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const u16*>(a.out) + off));
    const u32x4 xg = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const u16*>(a.g) + off));
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
    *reinterpret_cast<u32x4*>(static_cast<u16*>(a.da) + off) = ra;
    __builtin_nontemporal_store(rg, reinterpret_cast<u32x4*>(static_cast<u16*>(a.dg) + off));
  }
  for (int m = 1; m < lanes; m <<= 1) D += __shfl_xor(D, m);
  // rows without keys (LSE = -inf) get the seed -inf, so P = exp2(-inf) = 0
  if (row < rows && c == 0) a.seed[row] = make_float2(l == kNegInf ? kNegInf : -l * kLog2e, -D);
}

__global__ void __launch_bounds__(256) attn_bwd_pre_f32_kernel(BwdArgs a) {
  const long long rows = (long long)a.B * a.H * a.N;
  const long long row = (long long)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int d = a.d;
  float D = 0.f;
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
  a.drow[row] = D;
}

// ------------------------------------------------------------------ 2. dK, dV, dBias (bf16)
// One workgroup = 4 waves = 32 keys of one head, for a chunk of C batch rows.
// Wave (kt, qh) owns keys kb+16kt..+15 and query half qh of every 64-query
// block.  Iteration `it` covers (row b, query block); its Q tile, dA tile,
// -log2(e)*LSE and -D rows sit in one of two LDS buffers, and the loads of iteration it+2 are in
// flight in registers while iteration it computes, so one barrier per
// iteration suffices and HBM latency is hidden behind two iterations.
//   S' = log2(e) * (Q K^T / sqrt(d) + bias) - log2(e) * LSE: K is held
//        pre-multiplied by log2(e)/sqrt(d), the bias enters through two
//        identity products (log2(e) split into bf16 hi + lo) and
//        -log2(e) * LSE as the accumulator's initial value, so P = exp2(S').
//   dP - D = dA V^T accumulated onto -D;  dS = P * (dP - D).
//   dV^T += dA^T P and dK^T += Q^T dS read the staged tiles through the
//   transpose read; dK takes the 1/sqrt(d) factor at the store.
// dBias: with `slab`, each wave adds dS of every row of the chunk into an LDS
// slab kept in accumulator layout (16 bytes per lane per tile, so no bank
// conflicts), through an identity product that reads the slab tile as its
// accumulator: no VALU, no atomics, one owner per cell, fixed order.  The
// chunk's sums are stored once as this workgroup's slice of partial p.
// With NQR > 0 the same slab tiles live in registers instead (each wave owns
// its tiles: NQR query blocks x 2 tiles x 4 floats per lane), which takes the
// slab's read and write of every iteration off the LDS; the row loop is then
// unrolled over the query blocks so every tile index is a constant.
// Without `slab` (one row per chunk) dS goes straight to partial b.
template <int DP>
struct DkdvStage {
  u32x4 q[DP / 32], da[DP / 32];  // Q and dA chunks of the staged tile
  u32x4 k[DP / 32], v[DP / 32];   // this lane's K and V row (fetched with a row's first query block)
  u32x4 bias;                     // bias of the wave's query tiles: lane groups 0-1 tile 0, 2-3 tile 1
  float2 seed;                    // (-log2(e) LSE, -D) of query `lane` of the block (wave 0)
};

template <int DP>
struct DkdvSmem {
  static constexpr int kTile = 64 * TileLds<DP, 0>::kRowElems;
  u16 sQA[2][2 * kTile];  // [buffer][Q tile | dA tile]
  float sLD[2][2][64];    // [buffer][-log2(e) LSE | -D]
  // query-half combine area of dK, dV at the end of a row; written again
  // only nqb >= 1 iterations (and barriers) later, so one barrier suffices
  f32x4 comb[2 * 2 * (DP / 16) * 64];
};

// One workgroup's tile: wg is its index among the nwg dK/dV workgroups, which
// take the first slots of the backward grid (the dispatcher sends slot w to
// XCD w mod 8); slab is the dynamic LDS [nqb][4 query tiles][2 key tiles]
// [64 lanes] when SLAB and NQR == 0.  NQR > 0 (with SLAB): the slab is held
// in registers; the host only picks it for an even number of 64-query blocks,
// at most NQR.
template <int DP, bool ALIGNED, bool SLAB, int NQR>
__device__ __forceinline__ void attn_dkdv_tile(int wg, int nwg, DkdvSmem<DP>& sm, f32x4* const slab,
                                               const BwdArgs& a) {
  constexpr int KC = DP / 32, CT = DP / 16;
  constexpr int NCH = DP / 32;
  constexpr int kTile = DkdvSmem<DP>::kTile;
  using LQ = TileLds<DP, 0>;
  auto& sQA = sm.sQA;
  auto& sLD = sm.sLD;
  auto& comb = sm.comb;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, n = lane & 15;
  const int kt = wave & 1, qh = wave >> 1;
  const int N = a.N, d = a.d, H = a.H;
  const int nkb = (N + 31) / 32;
  const int nqb = (N + 63) / 64;
  const int L = xcd_remap(wg, nwg);
  const int kblk = L % nkb;
  const int hp = L / nkb;
  const int p = hp % a.P, h = hp / a.P;
  const int kb = kblk * 32;
  const int key = kb + 16 * kt + n;          // this lane's key (result column)
  const int b0 = p * a.C, b1 = min(a.B, b0 + a.C);
  const int T = (b1 - b0) * nqb;              // iterations (row, query block)
  const u16* BiasH = static_cast<const u16*>(a.bias) + (size_t)h * N * N;
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(BiasH, (uint32_t)((size_t)N * N * 2));
  const size_t plane = (size_t)N * d;
  const uint32_t plane_bytes = (uint32_t)(plane * 2);

  const bool keep_lane = key < N && (a.mask == nullptr || a.mask[key] != 0);
  const bool wave_masked = __any(!keep_lane);

  static_assert(NQR == 0 || (SLAB && NQR % 2 == 0 && NQR <= 6), "register slab: SLAB, even, at most 6 blocks");
  f32x4 rslab[NQR > 0 ? NQR : 1][2];
  if constexpr (NQR > 0) {
#pragma unroll
    for (int i = 0; i < NQR; ++i) rslab[i][0] = rslab[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if constexpr (SLAB) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int idx = tid; idx < nqb * 8 * 64; idx += 256) slab[idx] = z;
  }

  // Every load below goes through a buffer resource that spans one (b, h)
  // plane (the whole offset in the per-lane register, which the range check
  // covers), so rows past N read as zeros and no load sits under a branch:
  // the compiler can then wait for exactly the stage it needs.  Columns
  // d..DP-1 of a staged Q/dA chunk hold the next row's leading values; they
  // only ever meet the zeroed K/V columns or land in dK/dV columns that are
  // not stored.
  uint32_t chunk_off[NCH];  // byte offset of this thread's chunks in a query block
  int kap[NCH], col[NCH];
#pragma unroll
  for (int c8i = 0; c8i < NCH; ++c8i) {
    const int c = tid + 256 * c8i;
    kap[c8i] = c / (DP / 8);
    col[c8i] = 8 * (c % (DP / 8));
    chunk_off[c8i] = (uint32_t)((kap[c8i] * d + col[c8i]) * 2);
  }
  // this lane's bias: query row 16(2qh+j)+n of the block with j = g/2, keys
  // k0..k0+7.  One 16-byte load per lane covers both query tiles of the wave;
  // the identity product of tile j reads lane groups 2j and 2j+1.
  const int k0 = kb + 16 * kt + 8 * (g & 1);
  const int bq = 16 * (2 * qh + (g >> 1)) + n;
  const uint32_t bias_off = (uint32_t)((bq * N + k0) * 2);
  bool colok[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) colok[kc] = 32 * kc + 8 * g < d;

  DkdvStage<DP> R[2];
  // Buffer resources of the next fetch's (b, h) plane.  Past the chunk they
  // are empty (zeros, no traffic).  Every buffer load costs address-unit time
  // whatever it moves, so only the loads a step needs are issued: K and V
  // rows with a row's first query block, the row seeds by wave 0.  Both
  // conditions are uniform across the wave.
  const size_t row_step = (size_t)H * plane;
  const u16* fK = static_cast<const u16*>(a.k) + ((size_t)b0 * H + h) * plane;
  const u16* fV = static_cast<const u16*>(a.v) + ((size_t)b0 * H + h) * plane;
  const u16* fQ = static_cast<const u16*>(a.q) + ((size_t)b0 * H + h) * plane;
  const u16* fdA = static_cast<const u16*>(a.da) + ((size_t)b0 * H + h) * plane;
  const float2* fS = a.seed + ((size_t)b0 * H + h) * N;
  uint32_t rec_plane = plane_bytes, rec_row = (uint32_t)N * 8u;
  auto next_row = [&]() {
    fQ += row_step;
    fdA += row_step;
    fK += row_step;
    fV += row_step;
    fS += (size_t)H * N;
  };
  int fb = b0, fq = 0;
  auto advance_fetch = [&]() {
    if (++fq == nqb) {
      fq = 0;
      ++fb;
      next_row();
      if (fb >= b1) rec_plane = rec_row = 0u;
    }
  };
  auto fetch = [&](DkdvStage<DP>& st, int qblk) {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(fQ, rec_plane);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(fdA, rec_plane);
    const uint32_t qoff = (uint32_t)(qblk * 64 * d * 2);
#pragma unroll
    for (int c8i = 0; c8i < NCH; ++c8i) {
      st.q[c8i] = buf_load16(rq, chunk_off[c8i] + qoff);
      st.da[c8i] = buf_load16(ra, chunk_off[c8i] + qoff);
    }
    if (qblk == 0) {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(fK, rec_plane);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(fV, rec_plane);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint32_t off = (uint32_t)((key * d + 32 * kc + 8 * g) * 2);
        st.k[kc] = buf_load16(rk, off);
        st.v[kc] = buf_load16(rv, off);
      }
    }
    if (wave == 0) st.seed = buf_load_f32x2(make_rsrc(fS, rec_row), (uint32_t)((qblk * 64 + lane) * 8));
    if constexpr (ALIGNED) {
      st.bias = buf_load16(brs, bias_off + (uint32_t)(qblk * 64 * N * 2));
    } else {
      const int qa = qblk * 64 + bq;
      st.bias = (qa < N) ? load_bias8(BiasH + (size_t)qa * N, k0, N, false) : u32x4{0, 0, 0, 0};
    }
  };
  auto commit = [&](const DkdvStage<DP>& st, int buf, int qblk) {
    u16* tQ = sQA[buf];
#pragma unroll
    for (int c8i = 0; c8i < NCH; ++c8i) {
      *reinterpret_cast<u32x4*>(&tQ[LQ::off(kap[c8i], col[c8i])]) = st.q[c8i];
      *reinterpret_cast<u32x4*>(&tQ[kTile + LQ::off(kap[c8i], col[c8i])]) = st.da[c8i];
    }
    if (tid < 64) {
      // queries past N get P = exp2(-inf) = 0 (rows without keys carry a -inf seed)
      sLD[buf][0][tid] = qblk * 64 + tid < N ? st.seed.x : kNegInf;
      sLD[buf][1][tid] = st.seed.y;
    }
  };

  const bf16x8 id_l2hi[2] = {ident_cols_frag(lane, kLog2eHiBf16, 0), ident_cols_frag(lane, kLog2eHiBf16, 2)};
  const bf16x8 id_l2lo[2] = {ident_cols_frag(lane, kLog2eLoBf16, 0), ident_cols_frag(lane, kLog2eLoBf16, 2)};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const u32x4 zero_u4 = {0u, 0u, 0u, 0u};
  bf16x8 kf[KC], vf[KC];
  f32x4 dk[CT], dv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;
  // S' = c1 * Q K^T + (log2(e) * bias - log2(e) * LSE), c1 = log2(e) * scale:
  // the score product takes the unscaled bf16 operands and is scaled in fp32
  // by one FMA, so no operand is rounded after scaling
  const float c1 = a.scale * kLog2e;
  auto take_kv = [&](const DkdvStage<DP>& st) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      kf[kc] = as_bf8(colok[kc] ? st.k[kc] : zero_u4);
      vf[kc] = as_bf8(colok[kc] ? st.v[kc] : zero_u4);
    }
  };

  // position of the current iteration (the next fetch is two ahead)
  int cb = b0, cq = 0;
  if (T > 0) {
    fetch(R[0], fq);
    advance_fetch();
    fetch(R[1], fq);
    advance_fetch();
    commit(R[0], 0, 0);
    take_kv(R[0]);
  }
  __syncthreads();

  // S_c: it & 1, the LDS buffer and register set of this iteration; QB_c:
  // the query block (== cq) when the slab is in registers, else unused
  auto step = [&](auto S_c, auto QB_c) {
    constexpr int S = decltype(S_c)::value;
    constexpr int QB = decltype(QB_c)::value;
    const int b = cb, qblk = cq;
    const bool last_q = qblk == nqb - 1;
    const u16* tQ = sQA[S];
    const u16* tA = tQ + kTile;
    // all LDS operands of the two 16-query tiles first, so that the four
    // independent product chains (S and dP of both tiles) interleave
    f32x4 sacc[2], dp[2];
    bf16x8 qfr[2][KC], afr[2][KC];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int qtile = 2 * qh + j;
      sacc[j] = *reinterpret_cast<const f32x4*>(&sLD[S][0][16 * qtile + 4 * g]);
      dp[j] = *reinterpret_cast<const f32x4*>(&sLD[S][1][16 * qtile + 4 * g]);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        qfr[j][kc] = as_bf8(*reinterpret_cast<const u32x4*>(&tQ[LQ::off(16 * qtile + n, 32 * kc + 8 * g)]));
        afr[j][kc] = as_bf8(*reinterpret_cast<const u32x4*>(&tA[LQ::off(16 * qtile + n, 32 * kc + 8 * g)]));
      }
    }
    // the transposed operands of the dV and dK products depend only on the
    // staged tiles: read them with the others, so their latency is not on
    // the path after the exponentials
    bf16x8 trA[CT], trQ[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int r0 = 32 * qh + 4 * g;
      trA[ct] = tr_frag_l<LQ>(tA, r0, r0 + 16, 16 * ct, lane);
      trQ[ct] = tr_frag_l<LQ>(tQ, r0, r0 + 16, 16 * ct, lane);
    }
    f32x4 slab0, slab1;
    f32x4* const st = slab + ((qblk * 4 + 2 * qh) * 2 + kt) * 64 + lane;
    if constexpr (SLAB && NQR == 0) {
      slab0 = st[0];
      slab1 = st[128];
    }
    // the bias of this iteration is read from its register stage before the
    // loads of iteration it+2 reuse the stage
#pragma unroll
    for (int j = 0; j < 2; ++j) sacc[j] = mfma32(as_bf8(R[S].bias), id_l2hi[j], sacc[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) sacc[j] = mfma32(as_bf8(R[S].bias), id_l2lo[j], sacc[j]);
    fetch(R[S], fq);  // iteration it+2
    advance_fetch();
    f32x4 qk[2] = {zero4, zero4};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        qk[j] = mfma32(qfr[j][kc], kf[kc], qk[j]);
        dp[j] = mfma32(afr[j][kc], vf[kc], dp[j]);
      }
    // P = exp2(S'), dS = P * (dP - D)
    f32x4 pj[2], dsj[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pj[j][r] = exp2_fast(fmaf(qk[j][r], c1, sacc[j][r]));
        dsj[j][r] = pj[j][r] * dp[j][r];
      }
    if (wave_masked && !keep_lane) {  // masked keys: P = dS = 0
      pj[0] = pj[1] = dsj[0] = dsj[1] = zero4;
    }
    if constexpr (!SLAB) {
      if (a.direct) {  // b == 0: dS is dBias
        u16* db = static_cast<u16*>(a.dbias) + (size_t)h * N * N;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = qblk * 64 + 16 * (2 * qh + j) + 4 * g + r;
            if (q < N && key < N) db[(size_t)q * N + key] = f2bf(dsj[j][r]);
          }
      } else {
        float* part = a.partial + ((size_t)b * H + h) * N * N;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = qblk * 64 + 16 * (2 * qh + j) + 4 * g + r;
            if (q < N && key < N) part[(size_t)q * N + key] = dsj[j][r];
          }
      }
    }
    // P and dS as 16x16x32 operands: k slot (g, v) is query row
    // 32qh + 16(v/4) + 4g + v%4 of the block
    const bf16x8 pb = pack8(pj[0], pj[1]);
    const bf16x8 dsb = pack8(dsj[0], dsj[1]);
    // slab tiles (qblk, 2qh+j, kt) += dS of query tile 2qh+j, in fp32 and in
    // the result layout (lane (g, n): queries 4g..4g+3 at key n)
    if constexpr (NQR > 0) {
      rslab[QB][0] += dsj[0];
      rslab[QB][1] += dsj[1];
    } else if constexpr (SLAB) {
      st[0] = slab0 + dsj[0];
      st[128] = slab1 + dsj[1];
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      dv[ct] = mfma32(trA[ct], pb, dv[ct]);
      dk[ct] = mfma32(trQ[ct], dsb, dk[ct]);
    }
    // ---- stage iteration it+1 into the other buffer (its loads were issued
    // one iteration ago)
    if (++cq == nqb) {
      cq = 0;
      ++cb;
    }
    commit(R[S ^ 1], S ^ 1, cq);
    if (last_q) take_kv(R[S ^ 1]);  // iteration it+1 starts the next row
    __syncthreads();

    if (last_q) {
      // ---- combine the two query halves and store dK, dV of row b.  The
      // next write of `comb` comes a row later, after at least one more
      // barrier, so the readers below need no closing barrier.
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
        u16* dK = static_cast<u16*>(a.dk) + bh * plane;
        u16* dV = static_cast<u16*>(a.dv) + bh * plane;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int c = 16 * ct + 4 * g;
          if (c >= d) continue;
          const f32x4 sk = (dk[ct] + comb[((kt * 2 + 0) * CT + ct) * 64 + lane]) * a.scale;
          const f32x4 sv = dv[ct] + comb[((kt * 2 + 1) * CT + ct) * 64 + lane];
          *reinterpret_cast<u32x2*>(dK + (size_t)key * d + c) = u32x2{pack2(sk[0], sk[1]), pack2(sk[2], sk[3])};
          *reinterpret_cast<u32x2*>(dV + (size_t)key * d + c) = u32x2{pack2(sv[0], sv[1]), pack2(sv[2], sv[3])};
        }
      }
      // Stores share the vector-memory counter with loads.  With stores
      // outstanding the compiler cannot count loads in order and waits for
      // the counter to drain before every later use of a fetched stage;
      // draining it here once per row keeps those waits exact.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (NQR > 0) {
    // nqb is even, so iteration parity is the query block's parity
    auto pair = [&](auto Q0_c) __attribute__((always_inline)) {
      constexpr int Q0 = decltype(Q0_c)::value;
      if constexpr (Q0 < NQR) {
        if (Q0 < nqb) {
          step(I0{}, Q0_c);
          step(I1{}, std::integral_constant<int, Q0 + 1>{});
        }
      }
    };
    for (int b = b0; b < b1; ++b) {
      pair(std::integral_constant<int, 0>{});
      pair(std::integral_constant<int, 2>{});
      pair(std::integral_constant<int, 4>{});
    }
    if (key < N) {
      float* part = a.partial + ((size_t)p * H + h) * N * N;
#pragma unroll
      for (int qblk = 0; qblk < NQR; ++qblk)
        if (qblk < nqb)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int q = qblk * 64 + 16 * (2 * qh + j) + 4 * g + r;
              if (q < N) part[(size_t)q * N + key] = rslab[qblk][j][r];
            }
    }
    return;
  }
  for (int it = 0; it < T; it += 2) {
    step(I0{}, I0{});
    if (it + 1 < T) step(I1{}, I0{});
  }

  if (SLAB && key < N) {
    // this chunk's dBias sums -> partial p (lane (g, n) of a tile holds rows 4g..4g+3)
    float* part = a.partial + ((size_t)p * H + h) * N * N;
    for (int qblk = 0; qblk < nqb; ++qblk)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f32x4 v = slab[((qblk * 4 + 2 * qh + j) * 2 + kt) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = qblk * 64 + 16 * (2 * qh + j) + 4 * g + r;
          if (q < N) part[(size_t)q * N + key] = v[r];
        }
      }
  }
}

// ------------------------------------------------------------------ 2c. dK/dV, 128-query steps
// The register-slab tile (d <= 32, N % 8 == 0) in steps of 128 queries.  A
// workgroup of NW waves owns 32 keys; wave (kt, qg) takes its 16 keys against
// query group qg of every step, JT = 16 / NW of its eight 16-query tiles:
//   NW = 4: two groups of four tiles, N <= 384 (three steps per row);
//   NW = 8: four groups of two tiles, N <= 768 (six steps per row).
// Either way a wave's dBias slab is 12 register tiles (48 VGPRs), so no LDS
// slab limits the workgroups per CU.  Every operand of a step -- the Q and
// dA tiles, the row seeds, each wave's own bias tiles and, at a row's first
// step, the K and V rows -- goes from memory straight into LDS through
// LDS-destination buffer loads issued one step ahead into the other of two
// buffers.  No register holds a staged tile and no LDS store is issued; each
// step ends with one wait for this wave's loads and the barrier that
// publishes them.  At a row's end the query groups' dK and dV are summed in
// group order.
template <int NW>
struct DkdvWSmem {
  static constexpr int JT = 16 / NW;  // 16-query tiles per wave and step
  static constexpr int NB = NW == 8 ? 3 : 2;  // step buffers: loads issued NB - 1 steps ahead
  u16 qa[NB][2 * 128 * 32];            // [buffer][Q tile | dA tile], TileLds<32, 0> rows
  float seed[NB][256];                 // [buffer] -log2(e) LSE of the step's 128 queries, then -D
  u32x4 bias[NB][NW][JT / 2][64];      // [buffer][wave][half u][lane]: the wave's own bias
  u32x4 kv[2][2][2][64];              // [row parity][K | V][key tile][lane]
  f32x4 comb[NW / 2 - 1][2][2][2][64];  // [group - 1][kt][dK | dV][ct][lane]
};

template <int NW>
__device__ __forceinline__ void attn_dkdv_tile_w(int wg, int nwg, DkdvWSmem<NW>& sm, const BwdArgs& a) {
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  using LQ = TileLds<32, 0>;
  constexpr int JT = DkdvWSmem<NW>::JT;
  constexpr int NQB = 12 / JT;    // most 128-query steps per row: 3 or 6
  constexpr int NG = NW / 2;      // query groups
  constexpr int UQ = 8 / NW;      // Q (and dA) loads per wave and step
  constexpr int NB = DkdvWSmem<NW>::NB;
  constexpr int F = 2 * UQ + JT / 2;  // loads every wave issues for every step
  constexpr int kTile = 128 * 32;
  constexpr uint32_t kOob = 0xFFFFFFF0u;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, n = lane & 15;
  const int kt = wave & 1, qg = wave >> 1;
  const int N = a.N, d = a.d, H = a.H;
  const int nkb = (N + 31) / 32;
  const int nqb = (N + 127) / 128;  // 1 .. NQB
  const int L = xcd_remap(wg, nwg);
  const int kblk = L % nkb;
  const int hp = L / nkb;
  const int p = hp % a.P, h = hp / a.P;
  const int kb = kblk * 32;
  const int key = kb + 16 * kt + n;
  const int b0 = p * a.C, b1 = min(a.B, b0 + a.C);
  const int T = (b1 - b0) * nqb;
  const size_t plane = (size_t)N * d;
  const uint32_t plane_bytes = (uint32_t)(plane * 2);
  const bool keep_lane = key < N && (a.mask == nullptr || a.mask[key] != 0);
  const bool wave_masked = __any(!keep_lane);

  // per-lane load offsets.  Q / dA: load i of this wave fills tile units
  // 64 (UQ wave + i) + lane, i.e. row r = 16 (UQ wave + i) + lane / 4 and the
  // 16-byte chunk that the row's swizzle puts in slot lane % 4.
  bool qa_ok[UQ];
  uint32_t qa_off[UQ];
#pragma unroll
  for (int i = 0; i < UQ; ++i) {
    const int r = 16 * (UQ * wave + i) + (lane >> 2);
    const int c = ((lane & 3) ^ LQ::f(r)) & 3;
    qa_ok[i] = 8 * c < d;
    qa_off[i] = (uint32_t)((r * d + 8 * c) * 2);
  }
  // bias: half u holds query rows 16 (JT qg + 2u + g/2) + n of the step, keys
  // k0 .. k0 + 7; the identity product of tile j reads half j / 2, lane
  // groups 2 (j % 2) and 2 (j % 2) + 1
  const int k0 = kb + 16 * kt + 8 * (g & 1);
  const int bq0 = 16 * (JT * qg + (g >> 1)) + n;
  // K / V at a row's start: wave w < 4 loads K (w even) or V (w odd) of key
  // tile w / 2: lane (g, n) key kb + 16 (w / 2) + n, channels 8g .. 8g + 7
  const int kv_key = kb + 16 * ((wave >> 1) & 1) + n;
  const uint32_t kv_off = (8 * g < d) ? (uint32_t)((kv_key * d + 8 * g) * 2) : kOob;
  const i32x4 brs = rsrc_words(static_cast<const u16*>(a.bias) + (size_t)h * N * N, (uint32_t)((size_t)N * N * 2));

  const size_t row_step = (size_t)H * plane;
  const u16* fQ = static_cast<const u16*>(a.q) + ((size_t)b0 * H + h) * plane;
  const u16* fdA = static_cast<const u16*>(a.da) + ((size_t)b0 * H + h) * plane;
  const u16* fKV = static_cast<const u16*>((wave & 1) ? a.v : a.k) + ((size_t)b0 * H + h) * plane;
  const float2* fS = a.seed + ((size_t)b0 * H + h) * N;
  int fb = b0, fq = 0;
  // loads of the step at the fetch position (fb, fq) into buffer buf.  The
  // loads only some waves issue (K/V at a row's start, the seeds) go first
  // and the F that every wave issues last, so that waiting until at most F
  // loads are outstanding completes every older step.
  auto issue = [&](int buf) {
    if (fq == 0 && wave < 4)
      lds_dma16(rsrc_words(fKV, plane_bytes), lds_addr(&sm.kv[(fb - b0) & 1][wave & 1][wave >> 1][0]), kv_off);
    if (wave < 4) {
      // the step's 128 (-log2(e) LSE, -D) pairs split into two planes of
      // 128 floats, so that each seeds an accumulator with one LDS read:
      // wave w < 4 loads floats 64 w .. 64 w + 63 of the two planes
      const int e = 64 * wave + lane;
      lds_dma4(rsrc_words(fS, (uint32_t)N * 8u), lds_addr(sm.seed[buf]) + 256 * wave,
               (uint32_t)((fq * 128 + (e & 127)) * 8 + 4 * (e >> 7)));
    }
    const i32x4 rq = rsrc_words(fQ, plane_bytes), ra = rsrc_words(fdA, plane_bytes);
    const uint32_t qoff = (uint32_t)(fq * 128 * d * 2);
    const uint32_t dq = lds_addr(sm.qa[buf]);
#pragma unroll
    for (int i = 0; i < UQ; ++i) {
      const uint32_t off = qa_ok[i] ? qa_off[i] + qoff : kOob;
      lds_dma16(rq, dq + 1024 * (UQ * wave + i), off);
      lds_dma16(ra, dq + 2 * kTile + 1024 * (UQ * wave + i), off);
    }
#pragma unroll
    for (int u = 0; u < JT / 2; ++u) {
      const int q = fq * 128 + bq0 + 32 * u;
      const uint32_t off = (q < N && k0 < N) ? (uint32_t)(((size_t)q * N + k0) * 2) : kOob;
      lds_dma16(brs, lds_addr(&sm.bias[buf][wave][u][0]), off);
    }
    if (++fq == nqb) {
      fq = 0;
      ++fb;
      fQ += row_step;
      fdA += row_step;
      fKV += row_step;
      fS += (size_t)H * N;
    }
  };

  const bf16x8 id_l2hi[2] = {ident_cols_frag(lane, kLog2eHiBf16, 0), ident_cols_frag(lane, kLog2eHiBf16, 2)};
  const bf16x8 id_l2lo[2] = {ident_cols_frag(lane, kLog2eLoBf16, 0), ident_cols_frag(lane, kLog2eLoBf16, 2)};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const float c1 = a.scale * kLog2e;
  f32x4 rslab[NQB][JT];
#pragma unroll
  for (int i = 0; i < NQB; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j) rslab[i][j] = zero4;
  f32x4 dk[2], dv[2];
  dk[0] = dk[1] = dv[0] = dv[1] = zero4;
  bf16x8 kf, vf;

  // the first NB - 1 steps; then each step issues the loads of the step
  // NB - 1 ahead into the buffer the previous step used (with NB = 3 that
  // is a step whose K/V parity differs from the current row's: eight waves
  // run only with at least four steps per row)
  if (T > 0) issue(0);
  if (NB == 3 && T > 1) {
    issue(1);
    vm_wait<F>();
  } else {
    vm_wait<0>();
  }
  __syncthreads();

  int it = 0, cb = b0;
  auto step = [&](auto QB_c) {
    constexpr int QB = decltype(QB_c)::value;
    const int buf = it % NB;
    const bool last_q = QB == nqb - 1;
    if (it + NB - 1 < T) issue((it + NB - 1) % NB);
    if constexpr (QB == 0) {
      kf = as_bf8(sm.kv[(cb - b0) & 1][0][kt][lane]);
      vf = as_bf8(sm.kv[(cb - b0) & 1][1][kt][lane]);
    }
    const u16* tQ = sm.qa[buf];
    const u16* tA = tQ + kTile;
    f32x4 sacc[JT], dp[JT];
    bf16x8 qfr[JT], afr[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int qt = JT * qg + j;
      const float* sp = sm.seed[buf] + 16 * qt + 4 * g;
      sacc[j] = *reinterpret_cast<const f32x4*>(sp);
      dp[j] = *reinterpret_cast<const f32x4*>(sp + 128);
      qfr[j] = as_bf8(*reinterpret_cast<const u32x4*>(&tQ[LQ::off(16 * qt + n, 8 * g)]));
      afr[j] = as_bf8(*reinterpret_cast<const u32x4*>(&tA[LQ::off(16 * qt + n, 8 * g)]));
    }
    bf16x8 trA[JT / 2][2], trQ[JT / 2][2];
#pragma unroll
    for (int m = 0; m < JT / 2; ++m)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int r0 = 16 * (JT * qg + 2 * m) + 4 * g;
        trA[m][ct] = tr_frag_l<LQ>(tA, r0, r0 + 16, 16 * ct, lane);
        trQ[m][ct] = tr_frag_l<LQ>(tQ, r0, r0 + 16, 16 * ct, lane);
      }
    bf16x8 bb[JT / 2];
#pragma unroll
    for (int u = 0; u < JT / 2; ++u) bb[u] = as_bf8(sm.bias[buf][wave][u][lane]);
#pragma unroll
    for (int j = 0; j < JT; ++j) sacc[j] = mfma32(bb[j >> 1], id_l2hi[j & 1], sacc[j]);
#pragma unroll
    for (int j = 0; j < JT; ++j) sacc[j] = mfma32(bb[j >> 1], id_l2lo[j & 1], sacc[j]);
    f32x4 qk[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      qk[j] = mfma32(qfr[j], kf, zero4);
      dp[j] = mfma32(afr[j], vf, dp[j]);
    }
    // P = exp2(S'), dS = P * (dP - D)
    f32x4 pj[JT], dsj[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pj[j][r] = exp2_fast(fmaf(qk[j][r], c1, sacc[j][r]));
        dsj[j][r] = pj[j][r] * dp[j][r];
      }
    if (wave_masked && !keep_lane) {  // masked keys: P = dS = 0
#pragma unroll
      for (int j = 0; j < JT; ++j) pj[j] = dsj[j] = zero4;
    }
    // P and dS as 16x16x32 operands: k slot (g, v) of product m is query
    // row 16 (JT qg + 2m) + 16 (v / 4) + 4 g + v % 4 of the step
#pragma unroll
    for (int j = 0; j < JT; ++j) rslab[QB][j] += dsj[j];
#pragma unroll
    for (int m = 0; m < JT / 2; ++m) {
      const bf16x8 pb = pack8(pj[2 * m], pj[2 * m + 1]);
      const bf16x8 dsb = pack8(dsj[2 * m], dsj[2 * m + 1]);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        dv[ct] = mfma32(trA[m][ct], pb, dv[ct]);
        dk[ct] = mfma32(trQ[m][ct], dsb, dk[ct]);
      }
    }
    // this wave's loads of the next step have landed (with NB = 3 the F
    // loads of the step after it may still be in flight)
    if (NB == 3 && it + 2 < T) vm_wait<F>();
    else vm_wait<0>();
    __syncthreads();
    if (last_q) {
      // sum the query groups' dK, dV in group order and store row cb; `comb`
      // is written again only a row later, after at least one more barrier
      if (qg > 0) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          sm.comb[qg - 1][kt][0][ct][lane] = dk[ct];
          sm.comb[qg - 1][kt][1][ct][lane] = dv[ct];
        }
      }
      __syncthreads();
      if (qg == 0 && key < N) {
        const size_t bh = (size_t)cb * H + h;
        u16* dK = static_cast<u16*>(a.dk) + bh * plane;
        u16* dV = static_cast<u16*>(a.dv) + bh * plane;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int c = 16 * ct + 4 * g;
          if (c >= d) continue;
          f32x4 sk = dk[ct], sv = dv[ct];
#pragma unroll
          for (int q2 = 0; q2 < NG - 1; ++q2) {
            sk += sm.comb[q2][kt][0][ct][lane];
            sv += sm.comb[q2][kt][1][ct][lane];
          }
          sk *= a.scale;
          *reinterpret_cast<u32x2*>(dK + (size_t)key * d + c) = u32x2{pack2(sk[0], sk[1]), pack2(sk[2], sk[3])};
          *reinterpret_cast<u32x2*>(dV + (size_t)key * d + c) = u32x2{pack2(sv[0], sv[1]), pack2(sv[2], sv[3])};
        }
      }
      dk[0] = dk[1] = dv[0] = dv[1] = zero4;
      ++cb;
    }
    ++it;
  };
  for (int b = b0; b < b1; ++b) {
    step(std::integral_constant<int, 0>{});
    if (nqb > 1) step(std::integral_constant<int, 1>{});
    if (nqb > 2) step(std::integral_constant<int, 2>{});
    if constexpr (NQB > 3) {
      if (nqb > 3) step(std::integral_constant<int, 3>{});
      if (nqb > 4) step(std::integral_constant<int, 4>{});
      if (nqb > 5) step(std::integral_constant<int, 5>{});
    }
  }
  if (key < N) {
    float* part = a.partial + ((size_t)p * H + h) * N * N;
#pragma unroll
    for (int qblk = 0; qblk < NQB; ++qblk)
      if (qblk < nqb)
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = qblk * 128 + 16 * (JT * qg + j) + 4 * g + r;
            if (q < N) part[(size_t)q * N + key] = rslab[qblk][j][r];
          }
  }
}

// The eight-wave form as a launch of its own (one workgroup per CU, two
// waves per SIMD): the dK/dV tiles for 384 < N <= 768 at d <= 32, followed by
// a dQ-only launch.
__global__ void __launch_bounds__(512) attn_bwd_dkdv_w8_kernel(BwdArgs a) {
  __shared__ DkdvWSmem<8> sm;
  attn_dkdv_tile_w<8>(blockIdx.x, gridDim.x, sm, a);
}

// ------------------------------------------------------------------ 2b. dK/dV, eight waves (LDS slab)
// When the dBias slab sits in LDS and leaves room for only one workgroup per
// CU (the launches are then split: dK/dV tiles, then dQ tiles), the dK/dV
// tiles at d > 32 run as eight-wave workgroups: wave (kt, qq) owns 16 keys and one
// 16-query tile (quarter qq) of every 64-query block, so the CU holds two
// waves per SIMD instead of one in the same LDS.  The dV and dK products then
// have the wave's 16 queries on their k axis (16x16x16 products, each on an
// accumulator chain of its own), and at the end of a row the four query
// quarters of dK and dV are summed in quarter order through LDS.  The rest
// is the four-wave tile's: the same staged Q/dA tiles, row seeds and
// bias identity products, and each slab cell (query tile, key tile) owned by
// one wave and updated in program order.
template <int DP>
struct Dkdv8Smem {
  static constexpr int kTile = 64 * TileLds<DP, 0>::kRowElems;
  u16 sQA[2][2 * kTile];                  // [buffer][Q tile | dA tile]
  float sLD[2][2][64];                    // [buffer][-log2(e) LSE | -D]
  f32x4 comb[3][2][2][DP / 16][64];       // [quarter 1..3][kt][dK | dV][ct][lane]
};

template <int DP>
struct Dkdv8Stage {
  u32x4 q, da;                   // this thread's chunk of the staged Q and dA tiles (threads < 8 DP)
  u32x4 k[DP / 32], v[DP / 32];  // this lane's K and V row (with a row's first query block)
  u32x4 bias;                    // lane groups 0-1: keys 16 kt + 8 g .. +7 of query row 16 qq + n
  float2 seed;                   // (-log2(e) LSE, -D) of query `lane` of the block (wave 0)
};

__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
  typedef short s16x4v __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4v, a), __builtin_bit_cast(s16x4v, b), c,
                                                   0, 0, 0);
}

template <int DP, bool ALIGNED>
__global__ void __launch_bounds__(512) attn_bwd_dkdv8_kernel(BwdArgs a) {
  static_assert(DP == 64, "eight-wave dK/dV tiles: the 64-wide template only");
  constexpr int KC = DP / 32, CT = DP / 16;
  constexpr int kTile = Dkdv8Smem<DP>::kTile;
  constexpr uint32_t kOob = 0xFFFFFFF0u;
  using LQ = TileLds<DP, 0>;
  __shared__ Dkdv8Smem<DP> sm;
  extern __shared__ f32x4 dkdv8_slab[];  // [nqb][4 query tiles][2 key tiles][64 lanes]
  f32x4* const slab = dkdv8_slab;
  auto& sQA = sm.sQA;
  auto& sLD = sm.sLD;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, n = lane & 15;
  const int kt = wave & 1, qq = wave >> 1;
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
  const int T = (b1 - b0) * nqb;
  const u16* BiasH = static_cast<const u16*>(a.bias) + (size_t)h * N * N;
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(BiasH, (uint32_t)((size_t)N * N * 2));
  const size_t plane = (size_t)N * d;
  const uint32_t plane_bytes = (uint32_t)(plane * 2);
  const bool keep_lane = key < N && (a.mask == nullptr || a.mask[key] != 0);
  const bool wave_masked = __any(!keep_lane);

  {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int idx = tid; idx < nqb * 8 * 64; idx += 512) slab[idx] = z;
  }

  // staging: 64 DP / 8 sixteen-byte chunks per tile, one per thread below that
  const bool stager = tid < 8 * DP;
  const int kap = tid / (DP / 8), col = 8 * (tid % (DP / 8));
  const uint32_t chunk_off = (uint32_t)((kap * d + col) * 2);
  // bias: lane groups 0-1 hold keys 16 kt + 8 g .. + 7 of query row 16 qq + n;
  // groups 2-3 read nothing (their entries meet zeros of the identity operand)
  const int k0 = kb + 16 * kt + 8 * (g & 1);
  const int bq = 16 * qq + n;
  const uint32_t bias_off = (uint32_t)((bq * N + k0) * 2);
  bool colok[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) colok[kc] = 32 * kc + 8 * g < d;

  Dkdv8Stage<DP> R[2];
  const size_t row_step = (size_t)H * plane;
  const u16* fK = static_cast<const u16*>(a.k) + ((size_t)b0 * H + h) * plane;
  const u16* fV = static_cast<const u16*>(a.v) + ((size_t)b0 * H + h) * plane;
  const u16* fQ = static_cast<const u16*>(a.q) + ((size_t)b0 * H + h) * plane;
  const u16* fdA = static_cast<const u16*>(a.da) + ((size_t)b0 * H + h) * plane;
  const float2* fS = a.seed + ((size_t)b0 * H + h) * N;
  uint32_t rec_plane = plane_bytes, rec_row = (uint32_t)N * 8u;
  int fb = b0, fq = 0;
  auto advance_fetch = [&]() {
    if (++fq == nqb) {
      fq = 0;
      ++fb;
      fQ += row_step;
      fdA += row_step;
      fK += row_step;
      fV += row_step;
      fS += (size_t)H * N;
      if (fb >= b1) rec_plane = rec_row = 0u;
    }
  };
  auto fetch = [&](Dkdv8Stage<DP>& st, int qblk) {
    const uint32_t qoff = (uint32_t)(qblk * 64 * d * 2);
    st.q = buf_load16(make_rsrc(fQ, rec_plane), stager ? chunk_off + qoff : kOob);
    st.da = buf_load16(make_rsrc(fdA, rec_plane), stager ? chunk_off + qoff : kOob);
    if (qblk == 0) {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(fK, rec_plane);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(fV, rec_plane);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint32_t off = (uint32_t)((key * d + 32 * kc + 8 * g) * 2);
        st.k[kc] = buf_load16(rk, off);
        st.v[kc] = buf_load16(rv, off);
      }
    }
    if (wave == 0) st.seed = buf_load_f32x2(make_rsrc(fS, rec_row), (uint32_t)((qblk * 64 + lane) * 8));
    if constexpr (ALIGNED) {
      st.bias = buf_load16(brs, g < 2 ? bias_off + (uint32_t)(qblk * 64 * N * 2) : kOob);
    } else {
      const int qa = qblk * 64 + bq;
      st.bias = (g < 2 && qa < N) ? load_bias8(BiasH + (size_t)qa * N, k0, N, false) : u32x4{0, 0, 0, 0};
    }
  };
  auto commit = [&](const Dkdv8Stage<DP>& st, int buf, int qblk) {
    u16* tQ = sQA[buf];
    if (stager) {
      *reinterpret_cast<u32x4*>(&tQ[LQ::off(kap, col)]) = st.q;
      *reinterpret_cast<u32x4*>(&tQ[kTile + LQ::off(kap, col)]) = st.da;
    }
    if (tid < 64) {
      sLD[buf][0][tid] = qblk * 64 + tid < N ? st.seed.x : kNegInf;
      sLD[buf][1][tid] = st.seed.y;
    }
  };

  const bf16x8 id_l2hi = ident_cols_frag(lane, kLog2eHiBf16, 0);
  const bf16x8 id_l2lo = ident_cols_frag(lane, kLog2eLoBf16, 0);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const u32x4 zero_u4 = {0u, 0u, 0u, 0u};
  bf16x8 kf[KC], vf[KC];
  f32x4 dk[CT], dv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;
  const float c1 = a.scale * kLog2e;
  auto take_kv = [&](const Dkdv8Stage<DP>& st) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      kf[kc] = as_bf8(colok[kc] ? st.k[kc] : zero_u4);
      vf[kc] = as_bf8(colok[kc] ? st.v[kc] : zero_u4);
    }
  };

  int cb = b0, cq = 0;
  if (T > 0) {
    fetch(R[0], fq);
    advance_fetch();
    fetch(R[1], fq);
    advance_fetch();
    commit(R[0], 0, 0);
    take_kv(R[0]);
  }
  __syncthreads();

  // transposed operand reads of the dV and dK products: lane (g, 4e + a)
  // supplies row 16 qq + 4 g + e, columns 16 ct + 4 a .. + 3
  const int tre = (lane & 15) >> 2, tra = lane & 3;
  auto step = [&](auto S_c) {
    constexpr int S = decltype(S_c)::value;
    const int b = cb, qblk = cq;
    const bool last_q = qblk == nqb - 1;
    const u16* tQ = sQA[S];
    const u16* tA = tQ + kTile;
    f32x4 sacc = *reinterpret_cast<const f32x4*>(&sLD[S][0][16 * qq + 4 * g]);
    f32x4 dp = *reinterpret_cast<const f32x4*>(&sLD[S][1][16 * qq + 4 * g]);
    bf16x8 qfr[KC], afr[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qfr[kc] = as_bf8(*reinterpret_cast<const u32x4*>(&tQ[LQ::off(16 * qq + n, 32 * kc + 8 * g)]));
      afr[kc] = as_bf8(*reinterpret_cast<const u32x4*>(&tA[LQ::off(16 * qq + n, 32 * kc + 8 * g)]));
    }
    u32x2 trA[CT], trQ[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      trA[ct] = lds_tr16(tA + LQ::off(16 * qq + 4 * g + tre, 16 * ct + 4 * tra));
      trQ[ct] = lds_tr16(tQ + LQ::off(16 * qq + 4 * g + tre, 16 * ct + 4 * tra));
    }
    f32x4* const st = slab + ((qblk * 4 + qq) * 2 + kt) * 64 + lane;
    const f32x4 slab0 = st[0];
    sacc = mfma32(as_bf8(R[S].bias), id_l2hi, sacc);
    sacc = mfma32(as_bf8(R[S].bias), id_l2lo, sacc);
    fetch(R[S], fq);  // iteration it+2
    advance_fetch();
    f32x4 qk = zero4;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qk = mfma32(qfr[kc], kf[kc], qk);
      dp = mfma32(afr[kc], vf[kc], dp);
    }
    f32x4 pj, dsj;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pj[r] = exp2_fast(fmaf(qk[r], c1, sacc[r]));
      dsj[r] = pj[r] * dp[r];
    }
    if (wave_masked && !keep_lane) pj = dsj = zero4;  // masked keys: P = dS = 0
    st[0] = slab0 + dsj;
    // P and dS as 16x16x16 B operands: k slot (g, v) is query 16 qq + 4 g + v
    const u32x2 pb = {pack2(pj[0], pj[1]), pack2(pj[2], pj[3])};
    const u32x2 dsb = {pack2(dsj[0], dsj[1]), pack2(dsj[2], dsj[3])};
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      dv[ct] = mfma16(trA[ct], pb, dv[ct]);
      dk[ct] = mfma16(trQ[ct], dsb, dk[ct]);
    }
    if (++cq == nqb) {
      cq = 0;
      ++cb;
    }
    commit(R[S ^ 1], S ^ 1, cq);
    if (last_q) take_kv(R[S ^ 1]);
    __syncthreads();

    if (last_q) {
      // the four query quarters of dK and dV of row b, summed in quarter order
      if (qq > 0) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          sm.comb[qq - 1][kt][0][ct][lane] = dk[ct];
          sm.comb[qq - 1][kt][1][ct][lane] = dv[ct];
        }
      }
      __syncthreads();
      if (qq == 0 && key < N) {
        const size_t bh = (size_t)b * H + h;
        u16* dK = static_cast<u16*>(a.dk) + bh * plane;
        u16* dV = static_cast<u16*>(a.dv) + bh * plane;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int c = 16 * ct + 4 * g;
          if (c >= d) continue;
          f32x4 sk = dk[ct], sv = dv[ct];
#pragma unroll
          for (int w = 0; w < 3; ++w) {
            sk += sm.comb[w][kt][0][ct][lane];
            sv += sm.comb[w][kt][1][ct][lane];
          }
          sk *= a.scale;
          *reinterpret_cast<u32x2*>(dK + (size_t)key * d + c) = u32x2{pack2(sk[0], sk[1]), pack2(sk[2], sk[3])};
          *reinterpret_cast<u32x2*>(dV + (size_t)key * d + c) = u32x2{pack2(sv[0], sv[1]), pack2(sv[2], sv[3])};
        }
      }
      // stores share the vector-memory counter with the prefetched loads:
      // drain it once per row so later waits stay exact
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) dk[ct] = dv[ct] = zero4;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  for (int it = 0; it < T; it += 2) {
    step(I0{});
    if (it + 1 < T) step(I1{});
  }

  if (key < N) {
    float* part = a.partial + ((size_t)p * H + h) * N * N;
    for (int qblk = 0; qblk < nqb; ++qblk) {
      const f32x4 v = slab[((qblk * 4 + qq) * 2 + kt) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = qblk * 64 + 16 * qq + 4 * g + r;
        if (q < N) part[(size_t)q * N + key] = v[r];
      }
    }
  }
}

// ------------------------------------------------------------------ 3b. dQ, key-split (small grids)
// For grids that leave most CUs idle (a single batch row and a few heads),
// the dQ tiles split the keys the way the key-split forward does: one
// 16-query tile per workgroup, wave w takes key blocks [w nkb / 4,
// (w + 1) nkb / 4), stages its own K, V and bias blocks into a private LDS
// region with LDS-destination loads (no barrier in the key loop), and the
// four partial dQ tiles are summed in wave order through LDS at the end.  Per
// block the arithmetic is the dQ role's with one query tile.  d <= 32 and
// N % 8 == 0 only.
__device__ __forceinline__ void attn_dq_split_tile(int wg, int nwg, KeySplitLds (&wl)[4], uint32_t* keep,
                                                   const BwdArgs& a, int nqt) {
  using LK = TileLds<32, 1>;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int N = a.N, d = a.d;
  const int L = xcd_remap(wg, nwg);
  const int qt = L % nqt;
  const int bh_lin = L / nqt;
  const int h = bh_lin / a.B, b = bh_lin % a.B;
  const size_t bh = (size_t)b * a.H + h;
  const int q0 = 16 * qt;
  const int nkb = (N + 63) / 64;
  const int blo = wave * nkb / 4, bhi = (wave + 1) * nkb / 4;
  const uint32_t plane_bytes = (uint32_t)((size_t)N * d * 2);
  const i32x4 krs = rsrc_words(static_cast<const u16*>(a.k) + bh * N * d, plane_bytes);
  const i32x4 vrs = rsrc_words(static_cast<const u16*>(a.v) + bh * N * d, plane_bytes);
  const i32x4 brs = rsrc_words(static_cast<const u16*>(a.bias) + (size_t)h * N * N, (uint32_t)((size_t)N * N * 2));
  KeySplitLds& my = wl[wave];

  // staging of key block kb into this wave's region (keys past N are masked below)
  auto stage = [&](int kb) { key_split_stage(my, krs, vrs, brs, q0, N, d, kb, lane); };
  if (blo < bhi) stage(64 * blo);
  for (int k = tid; k < nkb * 64; k += 256)
    reinterpret_cast<uint8_t*>(keep)[k] = (k < N && (a.mask == nullptr || a.mask[k] != 0)) ? 1 : 0;

  // this lane's query row: Q and dA as B operands, (-log2(e) LSE, -D) as seeds
  const int qrow = q0 + ln;
  u32x4 rq = u32x4{0, 0, 0, 0}, rda = u32x4{0, 0, 0, 0};
  if (qrow < N && 8 * g < d) {
    rq = ld16(static_cast<const u16*>(a.q) + bh * N * d + (size_t)qrow * d + 8 * g);
    rda = ld16(static_cast<const u16*>(a.da) + bh * N * d + (size_t)qrow * d + 8 * g);
  }
  const bf16x8 qf = as_bf8(rq), daf = as_bf8(rda);
  float nl = kNegInf, nd = 0.f;  // rows without keys carry a -inf seed: P = 0
  if (qrow < N) {
    const float2 sd = a.seed[bh * N + qrow];
    nl = sd.x;
    nd = sd.y;
  }
  const f32x4 nl4 = {nl, nl, nl, nl}, nd4 = {nd, nd, nd, nd};
  const float c1 = a.scale * kLog2e;
  const bf16x8 id2h_lo = ident_rows_frag(lane, 0, kLog2eHiBf16), id2h_hi = ident_rows_frag(lane, 1, kLog2eHiBf16);
  const bf16x8 id2l_lo = ident_rows_frag(lane, 0, kLog2eLoBf16), id2l_hi = ident_rows_frag(lane, 1, kLog2eLoBf16);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 dq[2] = {zero4, zero4};
  const int krow = 16 * (ln >> 2) + (ln & 3);
  __syncthreads();  // keep bytes

  for (int blk = blo; blk < bhi; ++blk) {
    const int kb = blk * 64;
    vm_wait<0>();  // this block's staging (the wave's only loads in flight)
    bf16x8 kf[4], vf[4], kt[2][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kf[t] = as_bf8(*reinterpret_cast<const u32x4*>(my.k + LK::off(krow + 4 * t, 8 * g)));
      vf[t] = as_bf8(*reinterpret_cast<const u32x4*>(my.v + LK::off(krow + 4 * t, 8 * g)));
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int m = 0; m < 2; ++m) kt[ct][m] = tr_frag_l<LK>(my.k, 16 * g + 8 * m, 16 * g + 8 * m + 4, 16 * ct, lane);
    u32x4 blo4 = my.bias[bias_rows_slot(ln, 2 * g)], bhi4 = my.bias[bias_rows_slot(ln, 2 * g + 1)];
    const u32x4 kw = *reinterpret_cast<const u32x4*>(&keep[(kb >> 2) + 4 * g]);  // keep bytes of keys 16g .. 16g+15
    // every read of the region has returned: the next block may overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (blk + 1 < bhi) stage(kb + 64);

    // masked keys and keys past N: the select only in blocks that hold one
    if (__any((kw[0] & kw[1] & kw[2] & kw[3]) != 0x01010101u)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t m01 = ((kw[e] & 0xFFu) ? 0u : 0xFFFFu) | ((kw[e] & 0xFF00u) ? 0u : 0xFFFF0000u);
        const uint32_t m23 = ((kw[e] & 0xFF0000u) ? 0u : 0xFFFFu) | ((kw[e] & 0xFF000000u) ? 0u : 0xFFFF0000u);
        if (e < 2) {
          blo4[2 * e] = (blo4[2 * e] & ~m01) | (kMaskedBias2 & m01);
          blo4[2 * e + 1] = (blo4[2 * e + 1] & ~m23) | (kMaskedBias2 & m23);
        } else {
          bhi4[2 * (e - 2)] = (bhi4[2 * (e - 2)] & ~m01) | (kMaskedBias2 & m01);
          bhi4[2 * (e - 2) + 1] = (bhi4[2 * (e - 2) + 1] & ~m23) | (kMaskedBias2 & m23);
        }
      }
    }
    f32x4 acc[4];
    acc[0] = mfma32(id2l_lo, as_bf8(blo4), mfma32(id2h_lo, as_bf8(blo4), nl4));
    acc[1] = mfma32(id2l_hi, as_bf8(blo4), mfma32(id2h_hi, as_bf8(blo4), nl4));
    acc[2] = mfma32(id2l_lo, as_bf8(bhi4), mfma32(id2h_lo, as_bf8(bhi4), nl4));
    acc[3] = mfma32(id2l_hi, as_bf8(bhi4), mfma32(id2h_hi, as_bf8(bhi4), nl4));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4 qk = mfma32(kf[t], qf, zero4);
      const f32x4 dp = mfma32(vf[t], daf, nd4);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] = exp2_fast(fmaf(qk[r], c1, acc[t][r])) * dp[r];
    }
    const bf16x8 s0 = pack8(acc[0], acc[1]);
    const bf16x8 s1 = pack8(acc[2], acc[3]);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      dq[ct] = mfma32(kt[ct][0], s0, dq[ct]);
      dq[ct] = mfma32(kt[ct][1], s1, dq[ct]);
    }
  }

  // partial dQ^T (lane (g, ln): channels 16 ct + 4 g + r of query ln) into
  // the wave's own K region, then the sum over the waves in wave order
  float* part = reinterpret_cast<float*>(my.k);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[ln * 32 + 16 * ct + 4 * g + r] = dq[ct][r];
  __syncthreads();
  const int mq = tid >> 4, c = 2 * (tid & 15), row = q0 + mq;
  if (row < N && c < d) {
    float x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* pw = reinterpret_cast<const float*>(wl[w].k) + mq * 32 + c;
      x0 += pw[0];
      x1 += pw[1];
    }
    u16* dQ = static_cast<u16*>(a.dq) + bh * N * d;
    *reinterpret_cast<uint32_t*>(dQ + (size_t)row * d + c) = pack2(x0 * a.scale, x1 * a.scale);
  }
}

// ------------------------------------------------------------------ 3. dQ (bf16)
// Same decomposition as the forward kernel: 4 waves x 16*QT queries of one
// (b, h), 64-key blocks of K and V double-buffered in LDS in row-major form.
// S^T = K Q^T and dP^T = V dA^T read K and V row-wise; dQ^T = K^T dS^T reads
// K through the transpose read.  The wave's Q rows are scaled by
// log2(e)/sqrt(d) once in registers, the bias enters through two identity
// products (log2(e) split into bf16 hi + lo) and the accumulators start at -log2(e)*LSE and -D,
// so P = exp2(S') and dS = P * (dP - D) cost one exponential and one multiply.
// The bias of the next key block is fetched one block ahead; masked keys get
// the most negative bias (exp2 of it is 0) without a branch.
//
// This launch also carries the dK/dV workgroups (SLAB: their dBias slab
// variant): they need the same preprocessed inputs and not dQ, so the first
// ndk_slots workgroups (ndk rounded up to a multiple of 8, so both parts keep
// their XCD mapping) run the long dK/dV tiles and the dQ tiles fill the
// slots they leave free, then the chip.  The two roles share the static LDS;
// the dynamic LDS is the dK/dV slab or the dQ keep bytes.  NQR selects the
// dK/dV tile: 0 the LDS slab (or none), 6 the register slab over up to six
// 64-query steps, 3 the register slab over up to three 128-query steps with
// LDS-destination staging.  DK = false builds the dQ role alone (fewer
// registers) for a launch that carries only dQ tiles; KS = true runs the
// key-split dQ tiles (nqblocks then counts 16-query tiles).
template <int DP, int QT, bool ALIGNED, bool SLAB, int NQR, bool DK = true, bool KS = false>
__global__ void __launch_bounds__(256) attn_bwd_dq_bf16_kernel(BwdArgs a, int nqblocks, int ndk, int ndk_slots) {
  constexpr int KC = DP / 32, CT = DP / 16;
  constexpr int QW = 16 * QT, QBLK = 4 * QW;
  constexpr int NCH = DP / 32;
  using LK = TileLds<DP, 1>;
  struct DqSmem {
    u16 sK[2][64 * LK::kRowElems];
    u16 sV[2][64 * LK::kRowElems];
  };
  static_assert(!KS || DP == 32, "key-split dQ tiles: d <= 32");
  union Smem {
    DqSmem dq;
    DkdvSmem<DP> dk;
    KeySplitLds ks[KS ? 4 : 1];
    std::conditional_t<NQR == 3, DkdvWSmem<4>, char> dkw;
    // NQR == 3 (N <= 384, N % 8 == 0, d <= 32): K and V of the whole (b, h)
    // resident for the dQ tiles
    struct {
      u16 k[(NQR == 3 ? 384 : 1) * 32];
      u16 v[(NQR == 3 ? 384 : 1) * 32];
    } dqr;
  };
  __shared__ Smem sm;
  extern __shared__ f32x4 bwd_dyn_lds[];
  int wg = blockIdx.x, nwg = gridDim.x;
  if constexpr (DK) {
    if (wg < ndk_slots) {
      if constexpr (NQR == 3) {
        static_assert(DP == 32 && ALIGNED && SLAB, "128-query steps: d <= 32, N % 8 == 0, slab");
        if (wg < ndk) attn_dkdv_tile_w<4>(wg, ndk, sm.dkw, a);
      } else {
        if (wg < ndk) attn_dkdv_tile<DP, ALIGNED, SLAB, NQR>(wg, ndk, sm.dk, bwd_dyn_lds, a);
      }
      return;
    }
  }
  wg -= ndk_slots;
  nwg -= ndk_slots;
  if constexpr (KS) {
    attn_dq_split_tile(wg, nwg, sm.ks, reinterpret_cast<uint32_t*>(bwd_dyn_lds), a, nqblocks);
    return;
  }
  auto& sK = sm.dq.sK;
  auto& sV = sm.dq.sV;
  // keep bytes of every key (64 per key block): filled once, so the key
  // loop issues no mask loads
  uint32_t* const keep_lds = reinterpret_cast<uint32_t*>(bwd_dyn_lds);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int N = a.N, d = a.d;
  const int L = xcd_remap(wg, nwg);
  const int qb = L % nqblocks;
  const int bh_lin = L / nqblocks;
  const int h = bh_lin / a.B, b = bh_lin % a.B;
  const size_t bh = (size_t)b * a.H + h;
  const u16* Q = static_cast<const u16*>(a.q) + bh * N * d;
  const u16* K = static_cast<const u16*>(a.k) + bh * N * d;
  const u16* V = static_cast<const u16*>(a.v) + bh * N * d;
  const u16* dA = static_cast<const u16*>(a.da) + bh * N * d;
  const u16* BiasH = static_cast<const u16*>(a.bias) + (size_t)h * N * N;
  const float2* seed = a.seed + bh * N;
  u16* dQ = static_cast<u16*>(a.dq) + bh * N * d;
  const int q0 = qb * QBLK + wave * QW;
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(BiasH, (uint32_t)((size_t)N * N * 2));

  // K and V go through buffer resources spanning their plane: keys past N
  // read as zeros, so every load of a fetch is issued unconditionally and the
  // compiler waits for exactly the block it commits.  Columns d..DP-1 of a
  // chunk hold the next key's leading values; they meet only zero Q / dA
  // columns or land in dQ columns that are never stored.
  const uint32_t kv_bytes = (uint32_t)((size_t)N * d * 2);
  const __amdgpu_buffer_rsrc_t rsK = make_rsrc(K, kv_bytes), rsV = make_rsrc(V, kv_bytes);
  u32x4 rk[NCH], rv[NCH];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int c = tid + 256 * it;
      const int kappa = c / (DP / 8), c8 = c % (DP / 8);
      const uint32_t off = (uint32_t)(((kb + kappa) * d + 8 * c8) * 2);
      rk[it] = buf_load16(rsK, off);
      rv[it] = buf_load16(rsV, off);
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int c = tid + 256 * it;
      const int kappa = c / (DP / 8), c8 = c % (DP / 8);
      *reinterpret_cast<u32x4*>(&sK[buf][LK::off(kappa, 8 * c8)]) = rk[it];
      *reinterpret_cast<u32x4*>(&sV[buf][LK::off(kappa, 8 * c8)]) = rv[it];
    }
  };
  u32x4 bnext[QT][2];
  auto fetch_bias = [&](int kb) {
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      const int qrow = q0 + 16 * s + ln;
      if constexpr (ALIGNED) {  // N % 8 == 0: 16-byte aligned rows; reads past the plane give 0
        const uint32_t boff = (uint32_t)(((size_t)qrow * N + kb + 16 * g) * 2);
        bnext[s][0] = buf_load16(brs, boff);
        bnext[s][1] = buf_load16(brs, boff + 16);
      } else {
        bias_row16(BiasH, qrow, kb + 16 * g, N, bnext[s][0], bnext[s][1]);
      }
    }
  };

  bf16x8 qf[QT][KC], daf[QT][KC];
  f32x4 nl4[QT], nd4[QT];  // -log2(e) LSE and -D of the lane's query, as accumulator seeds
  // S' = c1 * Q K^T + (log2(e) * bias - log2(e) * LSE), c1 = log2(e) * scale:
  // unscaled bf16 operands, the scale applied in fp32 by one FMA
  const float c1 = a.scale * kLog2e;
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    const int qrow = q0 + 16 * s + ln;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int c0 = 32 * kc + 8 * g;
      u32x4 rq = u32x4{0, 0, 0, 0}, rda = u32x4{0, 0, 0, 0};
      if (qrow < N && c0 < d) {
        rq = ld16(Q + (size_t)qrow * d + c0);
        rda = ld16(dA + (size_t)qrow * d + c0);
      }
      qf[s][kc] = as_bf8(rq);
      daf[s][kc] = as_bf8(rda);
    }
    float nl = kNegInf, nd = 0.f;  // rows without keys carry a -inf seed: P = exp2(-inf) = 0
    if (qrow < N) {
      const float2 sd = seed[qrow];
      nl = sd.x;
      nd = sd.y;
    }
    nl4[s] = f32x4{nl, nl, nl, nl};
    nd4[s] = f32x4{nd, nd, nd, nd};
  }

  const bf16x8 id2h_lo = ident_rows_frag(lane, 0, kLog2eHiBf16), id2h_hi = ident_rows_frag(lane, 1, kLog2eHiBf16);
  const bf16x8 id2l_lo = ident_rows_frag(lane, 0, kLog2eLoBf16), id2l_hi = ident_rows_frag(lane, 1, kLog2eLoBf16);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 dq[QT][CT];
#pragma unroll
  for (int s = 0; s < QT; ++s)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) dq[s][ct] = zero4;
  const int krow = 16 * (ln >> 2) + (ln & 3);

  const int nkb = (N + 63) / 64;
  for (int k = tid; k < nkb * 64; k += 256)
    reinterpret_cast<uint8_t*>(keep_lds)[k] = (k < N && (a.mask == nullptr || a.mask[k] != 0)) ? 1 : 0;
  // NQR == 3: K and V of the (b, h) resident.  Every 1 KB unit i (keys
  // 16 i .. 16 i + 15 in the key-tile layout) arrives by one LDS-destination
  // load per tensor, lane l holding the chunk that the row's swizzle puts in
  // slot l % 4; then one barrier, and the key loop runs without barriers.
  constexpr bool kResident = NQR == 3;
  if constexpr (kResident) {
    const i32x4 krs = rsrc_words(K, kv_bytes), vrs = rsrc_words(V, kv_bytes);
    for (int i = wave; i < nkb * 4; i += 4) {
      const int r = 16 * i + (lane >> 2);
      const int c8 = ((lane & 3) ^ LK::f(r)) & 3;
      const uint32_t off = 8 * c8 < d ? (uint32_t)((r * d + 8 * c8) * 2) : 0xFFFFFFF0u;
      lds_dma16(krs, lds_addr(sm.dqr.k) + 1024 * i, off);
      lds_dma16(vrs, lds_addr(sm.dqr.v) + 1024 * i, off);
    }
    fetch_bias(0);
    vm_wait<0>();
  } else {
    fetch(0);
    fetch_bias(0);
    commit(0);
  }
  __syncthreads();
  for (int blk = 0; blk < nkb; ++blk) {
    const int buf = blk & 1;
    const int kb = blk * 64;
    u32x4 bcur[QT][2];
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      bcur[s][0] = bnext[s][0];
      bcur[s][1] = bnext[s][1];
    }
    // the next block's loads (past the last block they read zeros and are
    // never used; issuing them anyway keeps every iteration's loads alike)
    if constexpr (!kResident) fetch(kb + 64);
    fetch_bias(kb + 64);
    // keep these loads here, a whole iteration ahead of their use (the
    // scheduler would otherwise sink them next to the commit)
    __builtin_amdgcn_sched_barrier(0);

    bf16x8 kf[4][KC], vf[4][KC], kt[CT][2];
    const u16* tK = kResident ? sm.dqr.k + kb * 32 : sK[buf];
    const u16* tV = kResident ? sm.dqr.v + kb * 32 : sV[buf];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        kf[t][kc] = as_bf8(*reinterpret_cast<const u32x4*>(tK + LK::off(krow + 4 * t, 32 * kc + 8 * g)));
        vf[t][kc] = as_bf8(*reinterpret_cast<const u32x4*>(tV + LK::off(krow + 4 * t, 32 * kc + 8 * g)));
      }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int m = 0; m < 2; ++m) kt[ct][m] = tr_frag_l<LK>(tK, 16 * g + 8 * m, 16 * g + 8 * m + 4, 16 * ct, lane);

    // keep bytes of keys 16g .. 16g + 15 in one read; masked keys and keys
    // past N get the most negative bias, and only blocks that hold one pay
    // for the select (a uniform branch)
    const u32x4 kw4 = *reinterpret_cast<const u32x4*>(&keep_lds[(kb >> 2) + 4 * g]);
    if (__any((kw4[0] & kw4[1] & kw4[2] & kw4[3]) != 0x01010101u)) {
      u32x4 mlo, mhi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kw = kw4[e];
        const uint32_t m01 = ((kw & 0xFFu) ? 0u : 0xFFFFu) | ((kw & 0xFF00u) ? 0u : 0xFFFF0000u);
        const uint32_t m23 = ((kw & 0xFF0000u) ? 0u : 0xFFFFu) | ((kw & 0xFF000000u) ? 0u : 0xFFFF0000u);
        if (e < 2) { mlo[2 * e] = m01; mlo[2 * e + 1] = m23; }
        else { mhi[2 * (e - 2)] = m01; mhi[2 * (e - 2) + 1] = m23; }
      }
#pragma unroll
      for (int s = 0; s < QT; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bcur[s][0][e] = (bcur[s][0][e] & ~mlo[e]) | (kMaskedBias2 & mlo[e]);
          bcur[s][1][e] = (bcur[s][1][e] & ~mhi[e]) | (kMaskedBias2 & mhi[e]);
        }
    }
    // S'^T and (dP - D)^T of every sub-tile first, then the elementwise work
    // and the dQ products as one block of code
    f32x4 acc[QT][4], qk[QT][4], dp[QT][4];
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      const u32x4 blo = bcur[s][0], bhi = bcur[s][1];
      acc[s][0] = mfma32(id2l_lo, as_bf8(blo), mfma32(id2h_lo, as_bf8(blo), nl4[s]));
      acc[s][1] = mfma32(id2l_hi, as_bf8(blo), mfma32(id2h_hi, as_bf8(blo), nl4[s]));
      acc[s][2] = mfma32(id2l_lo, as_bf8(bhi), mfma32(id2h_lo, as_bf8(bhi), nl4[s]));
      acc[s][3] = mfma32(id2l_hi, as_bf8(bhi), mfma32(id2h_hi, as_bf8(bhi), nl4[s]));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        dp[s][t] = nd4[s];
        qk[s][t] = zero4;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          qk[s][t] = mfma32(kf[t][kc], qf[s][kc], qk[s][t]);
          dp[s][t] = mfma32(vf[t][kc], daf[s][kc], dp[s][t]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < QT; ++s) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][t][r] = exp2_fast(fmaf(qk[s][t][r], c1, acc[s][t][r])) * dp[s][t][r];
      const bf16x8 s0 = pack8(acc[s][0], acc[s][1]);
      const bf16x8 s1 = pack8(acc[s][2], acc[s][3]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        dq[s][ct] = mfma32(kt[ct][0], s0, dq[s][ct]);
        dq[s][ct] = mfma32(kt[ct][1], s1, dq[s][ct]);
      }
    }
    if constexpr (!kResident) {
      commit(buf ^ 1);
      __syncthreads();
    }
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
  extern __shared__ f32x4 slab_lds[];
  float* const slab = reinterpret_cast<float*>(slab_lds);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
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
          // one partial per batch row, or (a.direct, b == 0) dBias itself
          float* part = a.direct ? static_cast<float*>(a.dbias) + (size_t)h * N * N
                                 : a.partial + ((size_t)b * H + h) * N * N;
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

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
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
    // eight partials requested at a time, then added in index order
    int p = 0;
    for (; p + 8 <= P; p += 8) {
      f4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const f4*>(partial + (size_t)(p + k) * count + i4);
#pragma unroll
      for (int k = 0; k < 8; ++k) s += v[k];
    }
    for (; p < P; ++p) s += *reinterpret_cast<const f4*>(partial + (size_t)p * count + i4);
    if constexpr (BF16) {
      *reinterpret_cast<u32x2*>(static_cast<u16*>(out) + i4) = u32x2{pack2(s[0], s[1]), pack2(s[2], s[3])};
    } else {
      *reinterpret_cast<f4*>(static_cast<float*>(out) + i4) = s;
    }
    return;
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

// dynamic LDS of the dK/dV kernels' dBias slab (32 keys x all queries, fp32)
static size_t slab_bytes(int N, bool bf16) {
  const size_t nqb = (size_t)(N + 63) / 64;
  return bf16 ? nqb * 8 * 64 * 16 : nqb * 64 * kSlabStride * 4;
}
constexpr size_t kMaxSlabBytes = 112 * 1024;

// LDS of a four-wave dK/dV workgroup besides its slab (staged tiles, seeds,
// combine area)
static size_t dkdv_tile_bytes(int d, bool bf16) {
  const size_t dp = d <= 32 ? 32 : 64;
  return bf16 ? 2 * 2 * 64 * (dp + 8) * 2 + 1024 + 2 * 2 * (dp / 16) * 64 * 16
              : 2 * 64 * (dp + 1) * 4 + 512 + 2 * 2 * (dp / 16) * 64 * 16;
}

// Resident dK/dV workgroups per CU (160 KiB of LDS; at most 2 by registers in
// the bf16 launch that also carries dQ, 3 for fp32).
static int dkdv_wgs_per_cu(int N, int d, bool bf16, bool slab) {
  size_t lds = dkdv_tile_bytes(d, bf16);
  if (slab) lds += slab_bytes(N, bf16);
  return (int)std::max<size_t>(1, std::min<size_t>(bf16 ? 2 : 3, 160 * 1024 / lds));
}

// Batch rows per chunk.  Cost model in microseconds: the dK/dV launch runs in
// rounds of (256 CUs x resident workgroups); each round lasts C rows x nqb
// query blocks at ~0.4 us per block, and each chunk adds one fp32 [H,N,N]
// partial that is written and read back once at ~4 TB/s.
static void pick_chunks(int B, int H, int N, int wpc, int& P, int& C) {
  const long long per_chunk = (long long)H * ((N + 31) / 32);
  const long long slots = 256LL * wpc;
  const double nqb = (N + 63) / 64;
  const double plane_us = 2.0 * H * (double)N * N * 4 / 4.0e6;
  double best = 1e300;
  P = B;
  C = 1;
  for (int c = B; c >= 1; --c) {
    const int p = (B + c - 1) / c;
    const long long rounds = (per_chunk * p + slots - 1) / slots;
    const double cost = rounds * c * nqb * 0.4 + p * plane_us;
    if (cost < best) {
      best = cost;
      P = p;
      C = c;
    }
  }
}

BwdPlan plan_attn_bwd(int B, int H, int N, int d, bool bf16) {
  BwdPlan pl{};
  const size_t rows = (size_t)B * H * N;
  if (B > 1 && slab_bytes(N, bf16) <= kMaxSlabBytes && dkdv_tile_bytes(d, bf16) + slab_bytes(N, bf16) <= 160 * 1024) {
    pl.slab = 1;  // dBias sums in an LDS slab
    pick_chunks(B, H, N, dkdv_wgs_per_cu(N, d, bf16, true), pl.P, pl.C);
  } else {
    pl.slab = 0;  // one partial per batch row
    pl.C = 1;
    pl.P = B;
  }
  // a single batch row without a slab: its dS rows are dBias itself, stored
  // in the output dtype by the main kernel (no partial, no reduction)
  pl.direct = (!pl.slab && B == 1) ? 1 : 0;
  size_t off = 0;
  pl.off_da = off;
  off = align256(off + rows * d * (bf16 ? 2 : 4));
  pl.off_drow = off;  // fp32: D per row; bf16: (-log2(e) LSE, -D) pairs
  off = align256(off + rows * (bf16 ? 8 : 4));
  pl.off_partial = off;
  if (!pl.direct) off = align256(off + (size_t)pl.P * H * N * N * 4);
  pl.total = off;
  return pl;
}

// lanes per row of the bf16 preprocess: d / 8 rounded up to a power of two (log2)
static int pre_lanes_log2(int d) {
  int lg = 0;
  while ((1 << lg) < d / 8) ++lg;
  return lg;
}

hipError_t launch_attn_bwd_pre_bf16(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.N;
  const int lg = pre_lanes_log2(a.d);
  const int rpw = 256 >> lg;
  hipLaunchKernelGGL(attn_bwd_pre_bf16_kernel, dim3((unsigned)((rows + rpw - 1) / rpw)), dim3(256), 0, stream, a, lg);
  return hipGetLastError();
}

hipError_t launch_partial_sum_bf16(const float* partial, int P, size_t count, void* out, hipStream_t stream) {
  const dim3 grid((unsigned)((count / 4 + 255) / 256 + 1));
  hipLaunchKernelGGL(bias_grad_reduce_kernel<true>, grid, dim3(256), 0, stream, partial, P, count, out);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const BwdArgs& args, bool bf16, hipStream_t stream, KernelTimer* timer) {
  BwdArgs a = args;
  const int dp = a.d <= 32 ? 32 : 64;
  const long long rows = (long long)a.B * a.H * a.N;
  const long long bhs = (long long)a.B * a.H;
  hipError_t e;

  timer_start(timer, stream);
  // 1. preprocess
  {
    if (bf16) {
      const int lg = pre_lanes_log2(a.d);
      const int rpw = 256 >> lg;
      const dim3 grid((unsigned)((rows + rpw - 1) / rpw));
      hipLaunchKernelGGL(attn_bwd_pre_bf16_kernel, grid, dim3(256), 0, stream, a, lg);
    } else {
      const dim3 grid((unsigned)((rows + 255) / 256));
      hipLaunchKernelGGL(attn_bwd_pre_f32_kernel, grid, dim3(256), 0, stream, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timer_mark(timer, stream);
  }
  // 2-3. dK, dV, dBias partials and dQ
  const int nkb = (a.N + 31) / 32;
  const int ndk = a.H * a.P * nkb;
  // bf16, d <= 32, an even number of at most 6 query blocks: the dBias slab
  // sits in registers (no dynamic slab LDS)
  const int nqb64 = (a.N + 63) / 64;
  // the 128-query-step tile: N <= 384, N % 8 == 0, grids that fill the chip
  const bool wide = bf16 && a.slab && dp == 32 && a.N % 8 == 0 && a.N <= 384 && bhs * nqb64 >= 512;
  const bool reg_slab = wide || (bf16 && a.slab && dp == 32 && nqb64 % 2 == 0 && nqb64 <= 6);
  const size_t slab_shmem = a.slab && !reg_slab ? slab_bytes(a.N, bf16) : 0;
  if (bf16) {
    // One launch, the dK/dV tiles first and then the dQ tiles, while the slab
    // still leaves room for two workgroups per CU (the dynamic LDS of a
    // launch is sized for its largest role); beyond that, two launches of the
    // same kernel (dK/dV tiles only, then dQ tiles only with a small LDS).
    const int ndk_slots = (ndk + 7) & ~7;
    const bool qt2 = dp == 32 && bhs * ((a.N + 127) / 128) >= 1024;
    const bool al = (a.N % 8) == 0;
    const size_t keep_bytes = (size_t)((a.N + 63) / 64) * 64;
    const bool fuse = dkdv_wgs_per_cu(a.N, a.d, true, a.slab != 0 && !reg_slab) >= 2;
    // grids that would leave most CUs idle run key-split dQ tiles (one per 16
    // queries) in the fused launch
    const bool ks = fuse && dp == 32 && al && a.N > 64 && a.N <= 16384 && bhs * ((a.N + 63) / 64) < 512;
    const int nqb = ks ? (a.N + 15) / 16 : qt2 ? (a.N + 127) / 128 : (a.N + 63) / 64;
    const void* fn;
#define PBA_BWD_FN(DPV, QTV, ALV, SLV, NQV) \
  reinterpret_cast<const void*>(&attn_bwd_dq_bf16_kernel<DPV, QTV, ALV, SLV, NQV>)
#define PBA_BWD_FN6(DPV, QTV, ALV) \
  reinterpret_cast<const void*>(&attn_bwd_dq_bf16_kernel<DPV, QTV, ALV, false, 0, false>)
#define PBA_BWD_FNKS(SLV, NQV) \
  reinterpret_cast<const void*>(&attn_bwd_dq_bf16_kernel<32, 1, true, SLV, NQV, true, true>)
#define PBA_BWD_PICK(SLV)                                                                          \
  if (dp == 32) {                                                                                  \
    if (qt2) fn = al ? PBA_BWD_FN(32, 2, true, SLV, 0) : PBA_BWD_FN(32, 2, false, SLV, 0);         \
    else fn = al ? PBA_BWD_FN(32, 1, true, SLV, 0) : PBA_BWD_FN(32, 1, false, SLV, 0);             \
  } else {                                                                                         \
    if (qt2) fn = al ? PBA_BWD_FN(64, 2, true, SLV, 0) : PBA_BWD_FN(64, 2, false, SLV, 0);         \
    else fn = al ? PBA_BWD_FN(64, 1, true, SLV, 0) : PBA_BWD_FN(64, 1, false, SLV, 0);             \
  }
    if (ks) {
      fn = reg_slab ? PBA_BWD_FNKS(true, 6) : a.slab ? PBA_BWD_FNKS(true, 0) : PBA_BWD_FNKS(false, 0);
    } else if (wide) {
      fn = qt2 ? PBA_BWD_FN(32, 2, true, true, 3) : PBA_BWD_FN(32, 1, true, true, 3);
    } else if (reg_slab) {
      if (qt2) fn = al ? PBA_BWD_FN(32, 2, true, true, 6) : PBA_BWD_FN(32, 2, false, true, 6);
      else fn = al ? PBA_BWD_FN(32, 1, true, true, 6) : PBA_BWD_FN(32, 1, false, true, 6);
    } else if (a.slab) {
      PBA_BWD_PICK(true)
    } else {
      PBA_BWD_PICK(false)
    }
    // the dQ-only launch of the unfused case takes the dQ role alone
    const void* fn_dq;
    if (dp == 32) {
      if (qt2) fn_dq = al ? PBA_BWD_FN6(32, 2, true) : PBA_BWD_FN6(32, 2, false);
      else fn_dq = al ? PBA_BWD_FN6(32, 1, true) : PBA_BWD_FN6(32, 1, false);
    } else {
      fn_dq = al ? PBA_BWD_FN6(64, 1, true) : PBA_BWD_FN6(64, 1, false);
    }
#undef PBA_BWD_PICK
#undef PBA_BWD_FN
#undef PBA_BWD_FN6
#undef PBA_BWD_FNKS
    const size_t shmem_max = std::max(slab_shmem, keep_bytes);
    // the slab can exceed the default 64 KiB dynamic LDS limit
    if (shmem_max > 64 * 1024 &&
        (e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem_max)) != hipSuccess)
      return e;
    auto launch = [&](const void* f, unsigned grid, int ndk_arg, int slots_arg, size_t shmem) -> hipError_t {
      int nqb_arg = nqb;
      void* kargs[] = {&a, &nqb_arg, &ndk_arg, &slots_arg};
      return hipLaunchKernel(f, dim3(grid), dim3(256), kargs, shmem, stream);
    };
    if (fuse) {
      if ((e = launch(fn, (unsigned)(ndk_slots + bhs * nqb), ndk, ndk_slots, shmem_max)) != hipSuccess) return e;
    } else {
      // the dK/dV launch: at d > 32, eight-wave workgroups (two waves per
      // SIMD) when the LDS slab fits beside their tiles, else the four-wave
      // tile (at d <= 32 the eight-wave form measured slower: each wave's
      // per-block overhead is paid for half the products)
      const size_t lds8 = sizeof(Dkdv8Smem<64>) + slab_shmem;
      // 384 < N <= 768 at d <= 32: eight-wave 128-query steps with the dBias
      // slab in registers (no LDS slab)
      const bool w8 = dp == 32 && al && a.slab && a.N > 384 && a.N <= 768;
      if (w8) {
        void* kargs[] = {&a};
        if ((e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dkdv_w8_kernel), dim3((unsigned)ndk),
                                 dim3(512), kargs, 0, stream)) != hipSuccess)
          return e;
      } else if (dp == 64 && a.slab && !reg_slab && lds8 <= 160 * 1024) {
        const void* f8 = al ? reinterpret_cast<const void*>(&attn_bwd_dkdv8_kernel<64, true>)
                            : reinterpret_cast<const void*>(&attn_bwd_dkdv8_kernel<64, false>);
        if (slab_shmem > 64 * 1024 &&
            (e = hipFuncSetAttribute(f8, hipFuncAttributeMaxDynamicSharedMemorySize, (int)slab_shmem)) != hipSuccess)
          return e;
        void* kargs[] = {&a};
        if ((e = hipLaunchKernel(f8, dim3((unsigned)ndk), dim3(512), kargs, slab_shmem, stream)) != hipSuccess)
          return e;
      } else if ((e = launch(fn, (unsigned)ndk_slots, ndk, ndk_slots, std::max(slab_shmem, (size_t)16))) !=
                 hipSuccess) {
        return e;
      }
      timer_mark(timer, stream);
      if ((e = launch(fn_dq, (unsigned)(bhs * nqb), 0, 0, keep_bytes)) != hipSuccess) return e;
    }
    timer_mark(timer, stream);
  } else {
    {
      const void* fn = dp == 32 ? reinterpret_cast<const void*>(&attn_bwd_dkdv_f32_kernel<32>)
                                : reinterpret_cast<const void*>(&attn_bwd_dkdv_f32_kernel<64>);
      if (slab_shmem > 64 * 1024 &&
          (e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)slab_shmem)) != hipSuccess)
        return e;
      void* kargs[] = {&a};
      if ((e = hipLaunchKernel(fn, dim3((unsigned)ndk), dim3(256), kargs, slab_shmem, stream)) != hipSuccess) return e;
      timer_mark(timer, stream);
    }
    const int nqb = (a.N + 63) / 64;
    const dim3 grid((unsigned)(bhs * nqb));
    if (dp == 32) hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<32>, grid, dim3(256), 0, stream, a, nqb);
    else hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<64>, grid, dim3(256), 0, stream, a, nqb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timer_mark(timer, stream);
  }
  // 4. dBias = sum of partials (already in place when the kernel stored it directly)
  if (a.direct) {
    timer_mark(timer, stream);
  } else {
    const size_t count = (size_t)a.H * a.N * a.N;
    const dim3 grid((unsigned)((count / 4 + 255) / 256 + 1));
    if (bf16) hipLaunchKernelGGL(bias_grad_reduce_kernel<true>, grid, dim3(256), 0, stream, a.partial, a.P, count, a.dbias);
    else hipLaunchKernelGGL(bias_grad_reduce_kernel<false>, grid, dim3(256), 0, stream, a.partial, a.P, count, a.dbias);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timer_mark(timer, stream);
  }
  return hipSuccess;
}

}  // namespace pba

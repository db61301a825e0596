// attn_fwd.hip - forward pair-biased gated attention for gfx950.
//
// Computes, per (b, h):  O = sigmoid(G) * softmax(Q K^T / sqrt(d) + bias[h] + mask) V
// and the natural-log row logsumexp.  The bias is added after the key-query
// product, as the "Model Efficiency" section of the AlphaFold3
// open-source implementation page describes (molayo1419.me, "Show HN:
// AlphaFold3 open-source implementation"); the score tile is never written
// to memory (online softmax over key blocks, the tiling that section credits
// for the memory savings of fused biased-attention kernels).
//
// Work decomposition: one workgroup (4 waves) per (b, h, block of 64*QT
// queries); each wave owns 16*QT queries and walks all keys in blocks of 64
// that the workgroup stages through LDS (double-buffered).  Scores are
// produced transposed, S^T = K Q^T, so each lane owns one query column and
// its softmax statistics stay in-lane; the same layout feeds P^T straight
// into the O^T = V^T P^T product, and the gate epilogue needs no shuffles.
#include "pba_device.h"
#include "pba_kernels.h"

namespace pba {

namespace {

// Key order inside a 64-key block: result row i of score tile t holds key
// 16*(i/4) + 4*t + (i%4), so lane group g sees the 16 contiguous keys
// 16g..16g+15 across its four tiles (one 32-byte bias load per lane).
__device__ __forceinline__ void kperm_slot(int kappa, int& t, int& i) {
  t = (kappa & 15) >> 2;
  i = ((kappa >> 4) << 2) | (kappa & 3);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

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

}  // namespace

// One workgroup = 4 waves = 64*QT queries of one (b, h).  LDS holds the
// current and the next 64-key block of K and V in plain row-major form (row
// stride DP+8 elements); the K operand of S^T = K Q^T is read row-wise and the
// V^T operand of O^T = V^T P^T with the transpose read, so staging is two
// 16-byte copies per thread and no transposition happens in the copy.
template <int DP, int QT, bool ALIGNED>
__global__ void __launch_bounds__(256) attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int KC = DP / 32, CT = DP / 16, RS = DP + 8;
  constexpr int QW = 16 * QT, QBLK = 4 * QW;
  constexpr int NCH = DP / 32;  // 16-byte chunks per thread per tensor per block
  __shared__ __attribute__((aligned(16))) u16 sK[2][64 * RS];
  __shared__ __attribute__((aligned(16))) u16 sV[2][64 * RS];
  __shared__ uint32_t sKeep[2][16];
  __shared__ int sAny[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int N = a.N, d = a.d;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = L % a.nqb;
  const int bh_lin = L / a.nqb;
  const int h = bh_lin / a.B, b = bh_lin % a.B;
  const size_t bh = (size_t)b * a.H + h;
  const u16* Q = static_cast<const u16*>(a.q) + bh * N * d;
  const u16* K = static_cast<const u16*>(a.k) + bh * N * d;
  const u16* V = static_cast<const u16*>(a.v) + bh * N * d;
  const u16* G = static_cast<const u16*>(a.g) + bh * N * d;
  u16* O = static_cast<u16*>(a.out) + bh * N * d;
  float* LSE = a.lse + bh * N;
  const int q0 = qb * QBLK + wave * QW;
  // the head's bias plane; reads past its end return zero
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(static_cast<const u16*>(a.bias) + (size_t)h * N * N,
                                               (uint32_t)((size_t)N * N * 2));

  // ---- staging of one 64-key block: global -> registers -> LDS
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

  // ---- per-wave query fragments (B operand of S^T = K Q^T), pre-scaled by 1/sqrt(d)
  bf16x8 qf[QT][KC];
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    const int qrow = q0 + 16 * s + ln;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int c0 = 32 * kc + 8 * g;
      u32x4 raw = u32x4{0, 0, 0, 0};
      if (qrow < N && c0 < d) raw = ld16(Q + (size_t)qrow * d + c0);
      u32x4 sc;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sc[e] = pack2(bf2f((u16)(raw[e] & 0xFFFFu)) * a.scale, bf2f((u16)(raw[e] >> 16)) * a.scale);
      qf[s][kc] = as_bf8(sc);
    }
  }

  const bf16x8 id_lo = ident_rows_frag(lane, 0), id_hi = ident_rows_frag(lane, 1);
  const bf16x8 ones = ones_frag();
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 oacc[QT][CT];
  f32x4 lacc[QT];
  float mrun[QT];
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    lacc[s] = zero4;
    mrun[s] = kNegInf;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) oacc[s][ct] = zero4;
  }
  // key row of A-operand row i in score tile t: 16*(i/4) + 4t + (i%4), so the
  // 16 keys of lane group g are 16g..16g+15 (one 32-byte bias read per lane)
  const int krow = 16 * (ln >> 2) + (ln & 3);

  const int nkb = (N + 63) / 64;
  fetch(0);
  commit(0);
  __syncthreads();

  for (int blk = 0; blk < nkb; ++blk) {
    const int buf = blk & 1;
    const int kb = blk * 64;
    if (blk + 1 < nkb) fetch(kb + 64);

    // key-block operands shared by the wave's query sub-tiles
    bf16x8 kf[4][KC], vt[CT][2];
    const u16* tK = sK[buf];
    const u16* tV = sV[buf];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kf[t][kc] = as_bf8(*reinterpret_cast<const u32x4*>(tK + (krow + 4 * t) * RS + 32 * kc + 8 * g));
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int m = 0; m < 2; ++m) vt[ct][m] = tr_frag<RS>(tV, 16 * g + 8 * m, 16 * g + 8 * m + 4, 16 * ct, lane);

    // masked keys (and keys past N) get the most negative bias
    const bool masked_blk = sAny[buf] != 0;
    u32x4 mlo = u32x4{0, 0, 0, 0}, mhi = u32x4{0, 0, 0, 0};
    if (masked_blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kw = sKeep[buf][4 * g + e];  // keep bytes of keys 16g+4e .. +3
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
      if constexpr (ALIGNED) {  // N % 8 == 0: 16-byte aligned rows
        const uint32_t boff = (uint32_t)(((size_t)qrow * N + kb + 16 * g) * 2);
        blo = buf_load16(brs, boff);
        bhi = buf_load16(brs, boff + 16);
      } else {
        bias_row16(static_cast<const u16*>(a.bias) + (size_t)h * N * N, qrow, kb + 16 * g, N, blo, bhi);
      }
      if (masked_blk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          blo[e] = (blo[e] & ~mlo[e]) | (kMaskedBias2 & mlo[e]);
          bhi[e] = (bhi[e] & ~mhi[e]) | (kMaskedBias2 & mhi[e]);
        }
      }
      // scores S^T (rows: keys, columns: this wave's queries); the bias enters
      // through the identity product so no VALU work converts it
      f32x4 acc[4];
      acc[0] = mfma32(id_lo, as_bf8(blo), zero4);  // keys 16g + 0..3
      acc[1] = mfma32(id_hi, as_bf8(blo), zero4);  // keys 16g + 4..7
      acc[2] = mfma32(id_lo, as_bf8(bhi), zero4);  // keys 16g + 8..11
      acc[3] = mfma32(id_hi, as_bf8(bhi), zero4);  // keys 16g + 12..15
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) acc[t] = mfma32(kf[t][kc], qf[s][kc], acc[t]);

      float mx = fmaxf(fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])),
                       fmaxf(fmaxf(acc[1][0], acc[1][1]), fmaxf(acc[1][2], acc[1][3])));
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(acc[2][0], acc[2][1]), fmaxf(acc[2][2], acc[2][3])),
                           fmaxf(fmaxf(acc[3][0], acc[3][1]), fmaxf(acc[3][2], acc[3][3]))));
      mx = max_over_groups(mx);
      const float mnew = fmaxf(mrun[s], mx);
      if (__any(mnew > mrun[s])) {
        const float alpha = exp2_fast((mrun[s] - mnew) * kLog2e);  // 0 when mrun is -inf or masked
        if (mnew > mrun[s]) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) oacc[s][ct] *= alpha;
          lacc[s] *= alpha;
          mrun[s] = mnew;
        }
      }
      // a row whose keys so far are all masked keeps P = 0
      const float msc = (mrun[s] < kMaskedThreshold) ? kPosInf : mrun[s] * kLog2e;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = exp2_fast(fmaf(acc[t][r], kLog2e, -msc));
      // P^T as the B operand: k slot (g, v) <-> key 16g + 8m + v
      const bf16x8 p0 = pack8(acc[0], acc[1]);
      const bf16x8 p1 = pack8(acc[2], acc[3]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        oacc[s][ct] = mfma32(vt[ct][0], p0, oacc[s][ct]);
        oacc[s][ct] = mfma32(vt[ct][1], p1, oacc[s][ct]);
      }
      // row sums of the same rounded P, on the matrix core
      lacc[s] = mfma32(ones, p0, lacc[s]);
      lacc[s] = mfma32(ones, p1, lacc[s]);
    }

    if (blk + 1 < nkb) commit(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, gate, store O and LSE
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    const int qrow = q0 + 16 * s + ln;
    if (qrow >= N) continue;
    const float l = lacc[s][0];
    const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = 16 * ct + 4 * g;
      if (c >= d) continue;
      const size_t off = (size_t)qrow * d + c;
      const u32x2 graw = *reinterpret_cast<const u32x2*>(G + off);
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t w = graw[r >> 1];
        const float gv = bf2f((u16)((r & 1) ? (w >> 16) : (w & 0xFFFFu)));
        o[r] = oacc[s][ct][r] * inv * sigmoidf_fast(gv);
      }
      *reinterpret_cast<u32x2*>(O + off) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
    }
    if (g == 0) LSE[qrow] = l > 0.f ? mrun[s] + __builtin_amdgcn_logf(l) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------- fp32 path
// Same decomposition with fp32 matrix-core products (v_mfma_f32_16x16x4_f32),
// used for fp32 inputs where rounding P or Q to bf16 would cost accuracy.
template <int DP>
struct FwdSmemF32 {
  static constexpr int KC4 = DP / 4;
  float k[2][4 * KC4 * 64];     // K fragments [t][kc][lane]
  float v[2][64 * (DP + 1)];    // V natural, padded rows
  uint32_t keep[2][16];
  int any_masked[2];
};

template <int DP>
__global__ void __launch_bounds__(256) attn_fwd_f32_kernel(FwdArgs a) {
  using Sm = FwdSmemF32<DP>;
  constexpr int KC4 = Sm::KC4, CT = DP / 16, VS = DP + 1;
  constexpr int NCH = DP / 16;  // 16-byte chunks (4 floats) per thread per tensor
  __shared__ Sm sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int N = a.N, d = a.d;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = L % a.nqb;
  const int bh_lin = L / a.nqb;
  const int h = bh_lin / a.B, b = bh_lin % a.B;
  const size_t bh = (size_t)b * a.H + h;
  const float* Q = static_cast<const float*>(a.q) + bh * N * d;
  const float* K = static_cast<const float*>(a.k) + bh * N * d;
  const float* V = static_cast<const float*>(a.v) + bh * N * d;
  const float* G = static_cast<const float*>(a.g) + bh * N * d;
  const float* Bias = static_cast<const float*>(a.bias) + (size_t)h * N * N;
  float* O = static_cast<float*>(a.out) + bh * N * d;
  float* LSE = a.lse + bh * N;
  const int q0 = qb * 64 + wave * 16;
  const int qrow = q0 + ln;

  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 rk[NCH], rv[NCH];
  bool rkeep = true;
  auto fetch = [&](int kb) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int c = tid + 256 * it;
      const int kappa = c / (DP / 4), c4 = c % (DP / 4);
      const int key = kb + kappa;
      if (key < N && 4 * c4 < d) {
        rk[it] = *reinterpret_cast<const f4*>(K + (size_t)key * d + 4 * c4);
        rv[it] = *reinterpret_cast<const f4*>(V + (size_t)key * d + 4 * c4);
      } else {
        rk[it] = f4{0, 0, 0, 0};
        rv[it] = f4{0, 0, 0, 0};
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
      const int kappa = c / (DP / 4), c4 = c % (DP / 4);
      int t, i;
      kperm_slot(kappa, t, i);
      // element 4*c4 + e is k index kc = c4 (lane group e) of the 16x16x4 product
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.k[buf][(t * KC4 + c4) * 64 + e * 16 + i] = rk[it][e];
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.v[buf][kappa * VS + 4 * c4 + e] = rv[it][e];
    }
    if (tid < 64) {
      reinterpret_cast<uint8_t*>(&sm.keep[buf][0])[tid] = rkeep ? 1 : 0;
      const unsigned long long bal = __ballot(!rkeep);
      if (tid == 0) sm.any_masked[buf] = bal != 0ull;
    }
  };

  float qf[KC4];
#pragma unroll
  for (int kc = 0; kc < KC4; ++kc) {
    const int c = 4 * kc + g;
    qf[kc] = (qrow < N && c < d) ? Q[(size_t)qrow * d + c] * a.scale : 0.f;
  }

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) oacc[ct] = zero4;
  float lpart = 0.f, mrun = kNegInf;

  const int nkb = (N + 63) / 64;
  fetch(0);
  commit(0);
  __syncthreads();
  for (int blk = 0; blk < nkb; ++blk) {
    const int buf = blk & 1;
    const int kb = blk * 64;
    if (blk + 1 < nkb) fetch(kb + 64);

    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 16 * g + 4 * t + r;
        acc[t][r] = (qrow < N && key < N) ? Bias[(size_t)qrow * N + key] : 0.f;
      }
#pragma unroll
      for (int kc = 0; kc < KC4; ++kc) acc[t] = mfma4f(sm.k[buf][(t * KC4 + kc) * 64 + lane], qf[kc], acc[t]);
    }
    if (sm.any_masked[buf]) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int byte = 16 * g + 4 * t + r;
          const uint32_t w = sm.keep[buf][byte >> 2];
          if (((w >> (8 * (byte & 3))) & 0xFFu) == 0u) acc[t][r] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[t][r]);
    mx = max_over_groups(mx);
    const float mnew = fmaxf(mrun, mx);
    if (__any(mnew > mrun)) {
      const float alpha = (mnew == kNegInf) ? 1.f : exp2_fast((mrun - mnew) * kLog2e);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) oacc[ct] *= alpha;
      lpart *= alpha;
      mrun = mnew;
    }
    const float msc = (mrun == kNegInf) ? 0.f : mrun * kLog2e;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[t][r] = exp2_fast(fmaf(acc[t][r], kLog2e, -msc));
        lpart += acc[t][r];
      }
    // O^T += V^T P^T with one key per lane group and k step
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          oacc[ct] = mfma4f(sm.v[buf][(16 * g + 4 * t + r) * VS + 16 * ct + ln], acc[t][r], oacc[ct]);

    if (blk + 1 < nkb) commit(buf ^ 1);
    __syncthreads();
  }

  float l = lpart + __shfl_xor(lpart, 16);
  l = l + __shfl_xor(l, 32);
  if (qrow < N) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = 16 * ct + 4 * g;
      if (c >= d) continue;
      const size_t off = (size_t)qrow * d + c;
      f4 gv = *reinterpret_cast<const f4*>(G + off);
      f4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = oacc[ct][r] * inv * (1.0f / (1.0f + expf(-gv[r])));
      *reinterpret_cast<f4*>(O + off) = o;
    }
    if (g == 0) LSE[qrow] = l > 0.f ? mrun + logf(l) : kNegInf;
  }
}

// ---------------------------------------------------------------- launch
hipError_t launch_attn_fwd(const FwdArgs& args, bool bf16, hipStream_t stream) {
  FwdArgs a = args;
  const int dp = a.d <= 32 ? 32 : 64;
  const long long bhs = (long long)a.B * a.H;
  if (!bf16) {
    a.nqb = (a.N + 63) / 64;
    const dim3 grid((unsigned)(bhs * a.nqb));
    if (dp == 32) hipLaunchKernelGGL(attn_fwd_f32_kernel<32>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  // two query sub-tiles per wave when that still leaves enough workgroups
  const bool qt2 = dp == 32 && bhs * ((a.N + 127) / 128) >= 1024;
  const bool al = (a.N % 8) == 0;
  a.nqb = qt2 ? (a.N + 127) / 128 : (a.N + 63) / 64;
  const dim3 grid((unsigned)(bhs * a.nqb));
#define PBA_FWD_LAUNCH(DPV, QTV, ALV) \
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<DPV, QTV, ALV>), grid, dim3(256), 0, stream, a)
  if (dp == 32) {
    if (qt2) { if (al) PBA_FWD_LAUNCH(32, 2, true); else PBA_FWD_LAUNCH(32, 2, false); }
    else { if (al) PBA_FWD_LAUNCH(32, 1, true); else PBA_FWD_LAUNCH(32, 1, false); }
  } else {
    if (qt2) { if (al) PBA_FWD_LAUNCH(64, 2, true); else PBA_FWD_LAUNCH(64, 2, false); }
    else { if (al) PBA_FWD_LAUNCH(64, 1, true); else PBA_FWD_LAUNCH(64, 1, false); }
  }
#undef PBA_FWD_LAUNCH
  return hipGetLastError();
}

}  // namespace pba

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
// Work decomposition (three kernels, chosen by the launcher):
//  - streaming: one workgroup (4 waves) per (b, h, block of 64*QT queries);
//    each wave owns 16*QT queries and walks all keys in blocks of 64 that the
//    workgroup stages through LDS (double-buffered);
//  - K/V-resident (N <= 512 on grids that fill the chip): the workgroup
//    stages all of K and V of its (b, h) once, then its waves walk the key
//    blocks without barriers;
//  - key-split (grids too small to fill the chip): one 16-query tile per
//    workgroup, its four waves over quarters of the keys, partial softmax
//    states merged at the end.
// Scores are produced transposed, S^T = K Q^T, so each lane owns one query
// column and its softmax statistics stay in-lane; the same layout feeds P^T
// straight into the O^T = V^T P^T product, and the gate epilogue needs no
// shuffles.
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
    if (tid < 64) reinterpret_cast<uint8_t*>(&sKeep[buf][0])[tid] = rkeep ? 1 : 0;
  };

  // ---- per-wave query fragments (B operand of S^T = K Q^T), unscaled
  bf16x8 qf[QT][KC];
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    const int qrow = q0 + 16 * s + ln;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int c0 = 32 * kc + 8 * g;
      u32x4 raw = u32x4{0, 0, 0, 0};
      if (qrow < N && c0 < d) raw = ld16(Q + (size_t)qrow * d + c0);
      qf[s][kc] = as_bf8(raw);
    }
  }

  // T = Q K^T + bias / scale on the matrix core: the bias enters through two
  // identity products with 1/scale split into bf16 hi + lo, and Q K^T
  // accumulates onto them unscaled, so no score takes a separate scaling
  // step.  The exponentials apply cs = scale * log2(e): P = exp2(cs (T - m)),
  // and the natural-log LSE is scale * m + ln(l).
  const float isc = 1.f / a.scale;
  const uint32_t isc_hi = f2bf(isc), isc_lo = f2bf(isc - bf2f((u16)isc_hi));
  const bf16x8 ih0 = ident_rows_frag(lane, 0, isc_hi), ih1 = ident_rows_frag(lane, 1, isc_hi);
  const bf16x8 il0 = ident_rows_frag(lane, 0, isc_lo), il1 = ident_rows_frag(lane, 1, isc_lo);
  const float cs = a.scale * kLog2e;
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

  // bias fragments of a key block for the wave's query sub-tiles, fetched one
  // block ahead (16 keys 16g..16g+15 of query row q0 + 16s + ln per lane)
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
        bias_row16(static_cast<const u16*>(a.bias) + (size_t)h * N * N, qrow, kb + 16 * g, N, bnext[s][0],
                   bnext[s][1]);
      }
    }
  };

  const int nkb = (N + 63) / 64;
  fetch(0);
  fetch_bias(0);
  commit(0);
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
    if (blk + 1 < nkb) {
      fetch(kb + 64);
      fetch_bias(kb + 64);
    }

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

    // masked keys (and keys past N) get the most negative bias; the select
    // runs on every block (all-zero masks leave the bias unchanged), so the
    // block body has no branch and the sub-tiles' work can interleave
    u32x4 mlo, mhi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t kw = sKeep[buf][4 * g + e];  // keep bytes of keys 16g+4e .. +3
      const uint32_t m01 = ((kw & 0xFFu) ? 0u : 0xFFFFu) | ((kw & 0xFF00u) ? 0u : 0xFFFF0000u);
      const uint32_t m23 = ((kw & 0xFF0000u) ? 0u : 0xFFFFu) | ((kw & 0xFF000000u) ? 0u : 0xFFFF0000u);
      if (e < 2) { mlo[2 * e] = m01; mlo[2 * e + 1] = m23; }
      else { mhi[2 * (e - 2)] = m01; mhi[2 * (e - 2) + 1] = m23; }
    }

    // scores S^T (rows: keys, columns: this wave's queries) for every
    // sub-tile first; the bias enters through the identity product
    f32x4 acc[QT][4];
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      u32x4 blo = bcur[s][0], bhi = bcur[s][1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        blo[e] = (blo[e] & ~mlo[e]) | (kMaskedBias2 & mlo[e]);
        bhi[e] = (bhi[e] & ~mhi[e]) | (kMaskedBias2 & mhi[e]);
      }
      acc[s][0] = mfma32(il0, as_bf8(blo), mfma32(ih0, as_bf8(blo), zero4));  // keys 16g + 0..3
      acc[s][1] = mfma32(il1, as_bf8(blo), mfma32(ih1, as_bf8(blo), zero4));  // keys 16g + 4..7
      acc[s][2] = mfma32(il0, as_bf8(bhi), mfma32(ih0, as_bf8(bhi), zero4));  // keys 16g + 8..11
      acc[s][3] = mfma32(il1, as_bf8(bhi), mfma32(ih1, as_bf8(bhi), zero4));  // keys 16g + 12..15
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) acc[s][t] = mfma32(kf[t][kc], qf[s][kc], acc[s][t]);
    }

    // block maxima of every sub-tile, then one (rarely taken) rescale branch,
    // so that the exp / pack / PV work of all sub-tiles forms one block of
    // code the compiler can interleave (PV products of one sub-tile under the
    // exponentials of the next).
    // Lazy rescaling: the reference maximum moves only when a block's
    // maximum exceeds it by more than 8 in log2 units, so P <= 2^8 between
    // rescales (exact enough in fp32, and in bf16 for the PV product); the
    // LSE uses the same reference.
    float mx[QT];
    bool grow = false;
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      float m = fmaxf(fmaxf(fmaxf(acc[s][0][0], acc[s][0][1]), fmaxf(acc[s][0][2], acc[s][0][3])),
                      fmaxf(fmaxf(acc[s][1][0], acc[s][1][1]), fmaxf(acc[s][1][2], acc[s][1][3])));
      m = fmaxf(m, fmaxf(fmaxf(fmaxf(acc[s][2][0], acc[s][2][1]), fmaxf(acc[s][2][2], acc[s][2][3])),
                         fmaxf(fmaxf(acc[s][3][0], acc[s][3][1]), fmaxf(acc[s][3][2], acc[s][3][3]))));
      mx[s] = max_over_groups(m);
      grow = grow || (mx[s] * cs > mrun[s] * cs + 8.f);
    }
    if (__any(grow)) {
#pragma unroll
      for (int s = 0; s < QT; ++s) {
        if (mx[s] * cs > mrun[s] * cs + 8.f) {
          const float mnew = fmaxf(mrun[s], mx[s]);
          const float alpha = exp2_fast((mrun[s] - mnew) * cs);  // 0 when mrun is -inf or masked
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) oacc[s][ct] *= alpha;
          lacc[s] *= alpha;
          mrun[s] = mnew;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      // a row whose keys so far are all masked keeps P = 0
      const float msc = (mrun[s] < kMaskedThreshold) ? kPosInf : mrun[s] * cs;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][t][r] = exp2_fast(fmaf(acc[s][t][r], cs, -msc));
      // P^T as the B operand: k slot (g, v) <-> key 16g + 8m + v
      const bf16x8 p0 = pack8(acc[s][0], acc[s][1]);
      const bf16x8 p1 = pack8(acc[s][2], acc[s][3]);
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
    if (g == 0) LSE[qrow] = l > 0.f ? mrun[s] * a.scale + __builtin_amdgcn_logf(l) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------- key-split variant
// For grids that leave most of the chip idle (a single batch row and a few
// heads: B H ceil(N / 64) < 512 workgroups of the streaming kernel), more
// waves come from splitting the keys.  A workgroup takes one 16-query tile of
// one (b, h) and its four waves split the key blocks: wave w walks blocks
// [w nkb / 4, (w + 1) nkb / 4).  Each wave stages its own K, V and bias
// blocks into a private LDS region with buffer loads that write LDS directly,
// so the key loop has no barrier: once a block's fragments are in registers
// the next block's loads go into the same region while this block's products
// run.  The four partial softmax states (reference maximum m_w, row sum l_w,
// unnormalised output o_w) are then merged through LDS in wave order,
//   M = max_w m_w,  O = sum_w e^(m_w - M) o_w / sum_w e^(m_w - M) l_w,
// which is the online-softmax recurrence applied across the four key ranges.
// The per-block arithmetic is the streaming kernel's with one query tile.
// d <= 32 and N % 8 == 0 (16-byte bias rows) only.
__global__ void __launch_bounds__(256) attn_fwd_split_kernel(FwdArgs a) {
  using LK = TileLds<32, 1>;
  constexpr uint32_t kOob = 0xFFFFFFF0u;
  __shared__ KeySplitLds wl[4];
  extern __shared__ __attribute__((aligned(16))) uint32_t split_keep[];  // keep bytes of every key block

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int N = a.N, d = a.d;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = L % a.nqb;
  const int bh_lin = L / a.nqb;
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
    reinterpret_cast<uint8_t*>(split_keep)[k] = (k < N && (a.mask == nullptr || a.mask[k] != 0)) ? 1 : 0;

  // this tile's query row as the B operand of S^T = K Q^T (unscaled)
  const u16* Q = static_cast<const u16*>(a.q) + bh * N * d;
  u32x4 rq = u32x4{0, 0, 0, 0};
  if (q0 + ln < N && 8 * g < d) rq = ld16(Q + (size_t)(q0 + ln) * d + 8 * g);
  const bf16x8 qf = as_bf8(rq);
  __syncthreads();  // keep bytes

  // T = Q K^T + bias / scale on the matrix core: the bias enters through two
  // identity products with 1/scale split into bf16 hi + lo, and Q K^T
  // accumulates onto them unscaled, so no score takes a separate scaling
  // step.  The exponentials apply cs = scale * log2(e): P = exp2(cs (T - m)),
  // and the natural-log LSE is scale * m + ln(l).
  const float isc = 1.f / a.scale;
  const uint32_t isc_hi = f2bf(isc), isc_lo = f2bf(isc - bf2f((u16)isc_hi));
  const bf16x8 ih0 = ident_rows_frag(lane, 0, isc_hi), ih1 = ident_rows_frag(lane, 1, isc_hi);
  const bf16x8 il0 = ident_rows_frag(lane, 0, isc_lo), il1 = ident_rows_frag(lane, 1, isc_lo);
  const float cs = a.scale * kLog2e;
  const bf16x8 ones = ones_frag();
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 oacc[2] = {zero4, zero4};
  f32x4 lacc = zero4;
  float mrun = kNegInf;
  const int krow = 16 * (ln >> 2) + (ln & 3);

  for (int blk = blo; blk < bhi; ++blk) {
    const int kb = blk * 64;
    vm_wait<0>();  // this block's staging (the wave's only loads in flight)
    bf16x8 kf[4], vt[2][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) kf[t] = as_bf8(*reinterpret_cast<const u32x4*>(my.k + LK::off(krow + 4 * t, 8 * g)));
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int m = 0; m < 2; ++m) vt[ct][m] = tr_frag_l<LK>(my.v, 16 * g + 8 * m, 16 * g + 8 * m + 4, 16 * ct, lane);
    u32x4 blo4 = my.bias[bias_rows_slot(ln, 2 * g)], bhi4 = my.bias[bias_rows_slot(ln, 2 * g + 1)];
    const u32x4 kw = *reinterpret_cast<const u32x4*>(&split_keep[(kb >> 2) + 4 * g]);  // keep bytes of keys 16g .. 16g+15
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
    acc[0] = mfma32(il0, as_bf8(blo4), mfma32(ih0, as_bf8(blo4), zero4));  // keys 16g + 0..3
    acc[1] = mfma32(il1, as_bf8(blo4), mfma32(ih1, as_bf8(blo4), zero4));  // keys 16g + 4..7
    acc[2] = mfma32(il0, as_bf8(bhi4), mfma32(ih0, as_bf8(bhi4), zero4));  // keys 16g + 8..11
    acc[3] = mfma32(il1, as_bf8(bhi4), mfma32(ih1, as_bf8(bhi4), zero4));  // keys 16g + 12..15
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = mfma32(kf[t], qf, acc[t]);
    float m = fmaxf(fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])),
                    fmaxf(fmaxf(acc[1][0], acc[1][1]), fmaxf(acc[1][2], acc[1][3])));
    m = fmaxf(m, fmaxf(fmaxf(fmaxf(acc[2][0], acc[2][1]), fmaxf(acc[2][2], acc[2][3])),
                       fmaxf(fmaxf(acc[3][0], acc[3][1]), fmaxf(acc[3][2], acc[3][3]))));
    const float mx = max_over_groups(m);
    // lazy rescaling as in the streaming kernel: the reference moves only
    // when a block's maximum passes it by more than 8 in log2 units
    const bool grow = mx * cs > mrun * cs + 8.f;
    if (__any(grow)) {
      if (grow) {
        const float mnew = fmaxf(mrun, mx);
        const float alpha = exp2_fast((mrun - mnew) * cs);  // 0 when mrun is -inf or masked
        oacc[0] *= alpha;
        oacc[1] *= alpha;
        lacc *= alpha;
        mrun = mnew;
      }
    }
    const float msc = (mrun < kMaskedThreshold) ? kPosInf : mrun * cs;  // every key so far masked: P = 0
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] = exp2_fast(fmaf(acc[t][r], cs, -msc));
    const bf16x8 p0 = pack8(acc[0], acc[1]);
    const bf16x8 p1 = pack8(acc[2], acc[3]);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      oacc[ct] = mfma32(vt[ct][0], p0, oacc[ct]);
      oacc[ct] = mfma32(vt[ct][1], p1, oacc[ct]);
    }
    lacc = mfma32(ones, p0, lacc);
    lacc = mfma32(ones, p1, lacc);
  }

  // the merging thread's gate, requested before the barrier: query mq,
  // channels 2 cp and 2 cp + 1
  const int mq = tid >> 4, cp = tid & 15;
  const int qrow = q0 + mq, c = 2 * cp;
  const bool live = qrow < N && c < d;
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(static_cast<const u16*>(a.g) + bh * N * d, plane_bytes);
  const uint32_t gw = __builtin_bit_cast(uint32_t, buf_load_f32(grs, live ? (uint32_t)((qrow * d + c) * 2) : kOob));

  // partial state into the wave's own region: o_w [16 queries][32 channels]
  // over the K tile, (m_w, l_w) per query over the V tile.  Lane (g, ln)
  // holds channels 16 ct + 4 g + r of query ln.
  float* part = reinterpret_cast<float*>(my.k);
  float2* ml = reinterpret_cast<float2*>(my.v);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[ln * 32 + 16 * ct + 4 * g + r] = oacc[ct][r];
  if (g == 0) ml[ln] = float2{mrun, lacc[0]};
  __syncthreads();

  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2 s = reinterpret_cast<const float2*>(wl[w].v)[mq];
    if (s.y > 0.f) M = fmaxf(M, s.x);
  }
  float lsum = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2 s = reinterpret_cast<const float2*>(wl[w].v)[mq];
    if (s.y > 0.f) {
      const float f = exp2_fast((s.x - M) * cs);
      const float* pw = reinterpret_cast<const float*>(wl[w].k) + mq * 32 + c;
      lsum = fmaf(f, s.y, lsum);
      o0 = fmaf(f, pw[0], o0);
      o1 = fmaf(f, pw[1], o1);
    }
  }
  const float inv = lsum > 0.f ? __builtin_amdgcn_rcpf(lsum) : 0.f;
  if (live) {
    u16* O = static_cast<u16*>(a.out) + bh * N * d;
    const float g0 = bf2f((u16)(gw & 0xFFFFu)), g1 = bf2f((u16)(gw >> 16));
    *reinterpret_cast<uint32_t*>(O + (size_t)qrow * d + c) =
        pack2(o0 * inv * sigmoidf_fast(g0), o1 * inv * sigmoidf_fast(g1));
  }
  if (cp == 0 && qrow < N)
    a.lse[bh * N + qrow] = lsum > 0.f ? M * a.scale + __builtin_amdgcn_logf(lsum) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------- K/V-resident variant
// For moderate N the whole K and V of one (b, h) fit in LDS: the workgroup
// (NW waves, 16*QT queries each) stages them once, synchronises once, and
// then every wave walks all key blocks on its own -- no per-block staging,
// waits or barriers.  With four waves two workgroups share a CU, so one's
// staging overlaps the other's products.  Only the wave's bias fragments stream from memory,
// prefetched one block ahead; its Q and gate rows are requested before the
// staging barrier.
//
// Softmax in log2 units with a reference maximum.  The Q K^T product is
// scaled by log2(e)/sqrt(d) in fp32 and the bias is multiplied by log2(e) on
// the matrix core (two identity products, log2(e) split into bf16 hi + lo),
// so scores are S' = log2(e) * L.  The first key block sets each query's reference r to its
// block maximum; every later block starts its accumulators at -r, so
// P = exp2(S') is one exponential per score.  The block's row sums (ones
// product on the matrix core) show whether any P may exceed 2^8 (sum above
// 2^14, or not finite); only then does the block take the slow path: true maximum, new
// reference, rescale of the running sums, P recomputed -- the same lazy
// rescaling the streaming kernel uses.  Rows whose reference is still -inf
// (every key so far masked) also take the slow path.
template <int DP, int QT, bool ALIGNED, int NW>
__global__ void __launch_bounds__(NW * 64) attn_fwd_res_kernel(FwdArgs a) {
  constexpr int kResThreads = NW * 64;
  constexpr int KC = DP / 32, CT = DP / 16;
  // K and V rows in the key-tile layout: 64-byte rows with permuted 16-byte
  // units at d <= 32 (the operand reads and the transposed reads of V each
  // cover every bank), padded 144-byte rows at d <= 64
  using LK = TileLds<DP, 1>;
  constexpr int RS = LK::kRowElems;
  constexpr int QW = 16 * QT, QBLK = NW * QW;
  constexpr int C8 = DP / 8;
  constexpr int RIT = 512 * C8 / kResThreads;  // staging chunks per thread (N up to 512)
  constexpr uint32_t kOob = 0xFFFFFFF0u;
  constexpr float kGrowLimit = 16384.f;  // largest block row sum of P (64 keys x 2^8) kept without rescaling
  extern __shared__ __attribute__((aligned(16))) u16 res_lds[];
  const int N = a.N, d = a.d;
  const int nkb = (N + 63) / 64, NP = nkb * 64;
  u16* const sK = res_lds;               // [NP][RS]
  u16* const sV = sK + NP * RS;          // [NP][RS]
  uint32_t* const sKeep = reinterpret_cast<uint32_t*>(sV + NP * RS);  // keep bytes [NP]

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = L % a.nqb;
  const int bh_lin = L / a.nqb;
  const int h = bh_lin / a.B, b = bh_lin % a.B;
  const size_t bh = (size_t)b * a.H + h;
  const u16* Q = static_cast<const u16*>(a.q) + bh * N * d;
  const u16* G = static_cast<const u16*>(a.g) + bh * N * d;
  u16* O = static_cast<u16*>(a.out) + bh * N * d;
  float* LSE = a.lse + bh * N;
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(static_cast<const u16*>(a.bias) + (size_t)h * N * N,
                                               (uint32_t)((size_t)N * N * 2));
  const int q0 = qb * QBLK + wave * QW;
  const uint32_t pb = (uint32_t)((size_t)N * d * 2);

  // this wave's Q and gate rows (zero past N or d), requested first
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q, pb);
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(G, pb);
  u32x4 qraw[QT][KC];
  u32x2 graw[QT][CT];
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    const int qrow = q0 + 16 * s + ln;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int c0 = 32 * kc + 8 * g;
      qraw[s][kc] = buf_load16(qrs, (qrow < N && c0 < d) ? (uint32_t)((qrow * d + c0) * 2) : kOob);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = 16 * ct + 4 * g;
      graw[s][ct] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                   grs, (qrow < N && c < d) ? (uint32_t)((qrow * d + c) * 2) : kOob, 0, 0));
    }
  }
  {
    // stage K and V of (b, h): buffer loads over the (b, h) plane, zero past N
    // and past d, all issued before the first LDS store
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const u16*>(a.k) + bh * N * d, pb);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const u16*>(a.v) + bh * N * d, pb);
    u32x4 rk[RIT], rv[RIT];
#pragma unroll
    for (int it = 0; it < RIT; ++it) {
      const int c = tid + kResThreads * it;
      const int key = c / C8, c8 = c % C8;
      const uint32_t off = (8 * c8 < d) ? (uint32_t)((key * d + 8 * c8) * 2) : kOob;
      rk[it] = buf_load16(krs, off);
      rv[it] = buf_load16(vrs, off);
    }
#pragma unroll
    for (int it = 0; it < RIT; ++it) {
      const int c = tid + kResThreads * it;
      const int key = c / C8, c8 = c % C8;
      if (key < NP) {
        *reinterpret_cast<u32x4*>(&sK[LK::off(key, 8 * c8)]) = rk[it];
        *reinterpret_cast<u32x4*>(&sV[LK::off(key, 8 * c8)]) = rv[it];
      }
    }
    for (int k = tid; k < NP; k += kResThreads)
      reinterpret_cast<uint8_t*>(sKeep)[k] = (k < N && (a.mask == nullptr || a.mask[k] != 0)) ? 1 : 0;
  }
  __syncthreads();  // the only barrier: from here on every wave runs alone
  if (q0 >= N) return;

  // S' = c1 * Q K^T + log2(e) * bias - ref with c1 = log2(e) / sqrt(d): the
  // product takes the unscaled bf16 operands and is scaled in fp32
  const float c1 = a.scale * kLog2e;
  bf16x8 qf[QT][KC];
#pragma unroll
  for (int s = 0; s < QT; ++s)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qf[s][kc] = as_bf8(qraw[s][kc]);

  const bf16x8 i2h_lo = ident_rows_frag(lane, 0, kLog2eHiBf16), i2h_hi = ident_rows_frag(lane, 1, kLog2eHiBf16);
  const bf16x8 i2l_lo = ident_rows_frag(lane, 0, kLog2eLoBf16), i2l_hi = ident_rows_frag(lane, 1, kLog2eLoBf16);
  const bf16x8 ones = ones_frag();
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 oacc[QT][CT];
  f32x4 lacc[QT];
  float ref[QT];  // reference maximum in log2 units (-inf: none yet)
#pragma unroll
  for (int s = 0; s < QT; ++s) {
    lacc[s] = zero4;
    ref[s] = kNegInf;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) oacc[s][ct] = zero4;
  }
  const int krow = 16 * (ln >> 2) + (ln & 3);

  u32x4 bn[QT][2];
  auto fetch_bias = [&](int kb) {  // kb < NP always (the last block is refetched at the end)
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      const int qrow = q0 + 16 * s + ln;
      if constexpr (ALIGNED) {
        const uint32_t boff = (uint32_t)(((size_t)qrow * N + kb + 16 * g) * 2);
        bn[s][0] = buf_load16(brs, boff);
        bn[s][1] = buf_load16(brs, boff + 16);
      } else {
        bias_row16(static_cast<const u16*>(a.bias) + (size_t)h * N * N, qrow, kb + 16 * g, N, bn[s][0],
                   bn[s][1]);
      }
    }
  };
  fetch_bias(0);

  for (int blk = 0; blk < nkb; ++blk) {
    const int kb = blk * 64;
    u32x4 bcur[QT][2];
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      bcur[s][0] = bn[s][0];
      bcur[s][1] = bn[s][1];
    }
    fetch_bias(blk + 1 < nkb ? kb + 64 : kb);

    bf16x8 kf[4][KC], vt[CT][2];
    const u16* tK = sK + kb * RS;
    const u16* tV = sV + kb * RS;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kf[t][kc] = as_bf8(*reinterpret_cast<const u32x4*>(tK + LK::off(krow + 4 * t, 32 * kc + 8 * g)));
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int m = 0; m < 2; ++m) vt[ct][m] = tr_frag_l<LK>(tV, 16 * g + 8 * m, 16 * g + 8 * m + 4, 16 * ct, lane);

    // masked keys get the most negative bias (x log2(e): -inf); only blocks
    // that contain masked keys pay for the select
    const uint32_t kw0 = sKeep[(kb >> 2) + 4 * g + 0], kw1 = sKeep[(kb >> 2) + 4 * g + 1];
    const uint32_t kw2 = sKeep[(kb >> 2) + 4 * g + 2], kw3 = sKeep[(kb >> 2) + 4 * g + 3];
    if (__any((kw0 & kw1 & kw2 & kw3) != 0x01010101u)) {
      const uint32_t kws[4] = {kw0, kw1, kw2, kw3};
      u32x4 mlo, mhi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kw = kws[e];
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

    // S' (log2 units) minus the reference; rows without a reference start at 0
    f32x4 acc[QT][4];
#pragma unroll
    for (int s = 0; s < QT; ++s) {
      const float seed = ref[s] == kNegInf ? 0.f : -ref[s];
      const f32x4 c4 = {seed, seed, seed, seed};
      const bf16x8 blo = as_bf8(bcur[s][0]), bhi = as_bf8(bcur[s][1]);
      acc[s][0] = mfma32(i2l_lo, blo, mfma32(i2h_lo, blo, c4));  // keys 16g + 0..3
      acc[s][1] = mfma32(i2l_hi, blo, mfma32(i2h_hi, blo, c4));  // keys 16g + 4..7
      acc[s][2] = mfma32(i2l_lo, bhi, mfma32(i2h_lo, bhi, c4));  // keys 16g + 8..11
      acc[s][3] = mfma32(i2l_hi, bhi, mfma32(i2h_hi, bhi, c4));  // keys 16g + 12..15
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 qk = zero4;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) qk = mfma32(kf[t][kc], qf[s][kc], qk);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][t][r] = fmaf(qk[r], c1, acc[s][t][r]);
      }
    }
    // fast path: P = exp2(acc) and the block row sums.  The first block has
    // no reference yet and goes straight to the slow path.
    f32x4 pv[QT][4];
    bf16x8 p0[QT], p1[QT];
    f32x4 bsum[QT];
    bool slow = blk == 0;
    if (blk != 0) {
#pragma unroll
      for (int s = 0; s < QT; ++s) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) pv[s][t][r] = exp2_fast(acc[s][t][r]);
        p0[s] = pack8(pv[s][0], pv[s][1]);
        p1[s] = pack8(pv[s][2], pv[s][3]);
        bsum[s] = mfma32(ones, p1[s], mfma32(ones, p0[s], zero4));
        // not (sum <= limit) also catches NaN and +inf
        slow = slow || ref[s] == kNegInf || !(bsum[s][0] <= kGrowLimit);
      }
    }
    if (__any(slow)) {
      // slow path: true block maxima, reference moves up (lazily, by more
      // than 8), running sums rescaled, P and its row sums recomputed
#pragma unroll
      for (int s = 0; s < QT; ++s) {
        float m = fmaxf(fmaxf(fmaxf(acc[s][0][0], acc[s][0][1]), fmaxf(acc[s][0][2], acc[s][0][3])),
                        fmaxf(fmaxf(acc[s][1][0], acc[s][1][1]), fmaxf(acc[s][1][2], acc[s][1][3])));
        m = fmaxf(m, fmaxf(fmaxf(fmaxf(acc[s][2][0], acc[s][2][1]), fmaxf(acc[s][2][2], acc[s][2][3])),
                           fmaxf(fmaxf(acc[s][3][0], acc[s][3][1]), fmaxf(acc[s][3][2], acc[s][3][3]))));
        m = max_over_groups(m);  // block maximum relative to the seed
        const float seed = ref[s] == kNegInf ? 0.f : ref[s];
        const float bmax = m + seed;  // absolute block maximum (-inf: every key masked so far)
        float shift = 0.f;  // subtracted from acc
        if (bmax > kMaskedThreshold && (ref[s] == kNegInf || bmax > ref[s] + 8.f)) {
          if (ref[s] != kNegInf) {
            const float alpha = exp2_fast(ref[s] - bmax);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) oacc[s][ct] *= alpha;
            lacc[s] *= alpha;
          }
          shift = bmax - seed;
          ref[s] = bmax;
        } else if (ref[s] == kNegInf) {
          shift = kPosInf;  // still no kept key: P = 0
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) pv[s][t][r] = exp2_fast(acc[s][t][r] - shift);
        p0[s] = pack8(pv[s][0], pv[s][1]);
        p1[s] = pack8(pv[s][2], pv[s][3]);
        bsum[s] = mfma32(ones, p1[s], mfma32(ones, p0[s], zero4));
      }
    }
#pragma unroll
    for (int s = 0; s < QT; ++s) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        oacc[s][ct] = mfma32(vt[ct][0], p0[s], oacc[s][ct]);
        oacc[s][ct] = mfma32(vt[ct][1], p1[s], oacc[s][ct]);
      }
      lacc[s] += bsum[s];
    }
  }

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
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t w = graw[s][ct][r >> 1];
        const float gv = bf2f((u16)((r & 1) ? (w >> 16) : (w & 0xFFFFu)));
        o[r] = oacc[s][ct][r] * inv * sigmoidf_fast(gv);
      }
      *reinterpret_cast<u32x2*>(O + (size_t)qrow * d + c) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
    }
    // natural-log LSE from the log2-unit reference
    if (g == 0) LSE[qrow] = l > 0.f ? (ref[s] + __builtin_amdgcn_logf(l)) * kLn2 : kNegInf;
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
  const bool al = (a.N % 8) == 0;
  // K/V-resident kernel when K and V of one (b, h) fit (N <= 512) and the
  // grid still fills the chip
  // (d <= 32: 4 waves x 48 queries; d <= 64: 8 waves x 32 queries)
  {
    const int qt = dp == 32 ? 3 : 2;
    const int nw = dp == 32 ? 4 : 8;
    const int np = (a.N + 63) / 64 * 64;
    const int qblk = nw * 16 * qt;
    const int nqb = (a.N + qblk - 1) / qblk;
    const size_t lds = (size_t)2 * np * (dp == 32 ? 32 : dp + 8) * 2 + np;
    if (a.N <= 512 && bhs * nqb >= 512) {
      a.nqb = nqb;
      const dim3 grid((unsigned)(bhs * nqb));
      const void* fn = dp == 32 ? (al ? reinterpret_cast<const void*>(&attn_fwd_res_kernel<32, 3, true, 4>)
                                      : reinterpret_cast<const void*>(&attn_fwd_res_kernel<32, 3, false, 4>))
                                : (al ? reinterpret_cast<const void*>(&attn_fwd_res_kernel<64, 2, true, 8>)
                                      : reinterpret_cast<const void*>(&attn_fwd_res_kernel<64, 2, false, 8>));
      hipError_t e;
      if (lds > 64 * 1024 &&
          (e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
        return e;
      void* kargs[] = {&a};
      return hipLaunchKernel(fn, grid, dim3(nw * 64), kargs, lds, stream);
    }
  }
  // grids that would leave most CUs idle split the keys over the waves
  if (dp == 32 && al && a.N > 64 && a.N <= 16384 && bhs * ((a.N + 63) / 64) < 512) {
    a.nqb = (a.N + 15) / 16;
    const size_t keep = (size_t)((a.N + 63) / 64) * 64;
    hipLaunchKernelGGL(attn_fwd_split_kernel, dim3((unsigned)(bhs * a.nqb)), dim3(256), keep, stream, a);
    return hipGetLastError();
  }
  // two query sub-tiles per wave when that still leaves enough workgroups
  const bool qt2 = dp == 32 && bhs * ((a.N + 127) / 128) >= 1024;
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

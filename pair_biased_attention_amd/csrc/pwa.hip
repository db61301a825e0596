// pwa.hip - MSA pair-weighted averaging (forward and backward) for gfx950.
//
// The "MSA Pair Averaging Efficiency" section of the AlphaFold3 open-source
// implementation page (molayo1419.me) describes the operation: a weighted
// average over tokens j whose weights come from the pair bias alone,
// w[h,i,j] = softmax_j(b[h,i,j]), replacing MSA row attention; the naive
// form allocates a (*, N_seq, N_res, N_res, heads, c_hidden) intermediate.
// Here nothing of that size exists: per head the average is the GEMM
//   A_h[i, (s,c)] = sum_j w[h,i,j] V[s,j,h,c]     (M = N, K = N, cols = S*d)
// evaluated as O^T = V^T w^T so each lane ends with 4 consecutive channels of
// one (s, i) row for the sigmoid-gate epilogue.
//
// Kernels (all on the caller's stream):
//   pwa_softmax   w and w^T (bf16 workspace) and lse_w
//   pwa_gemm_dl   out = sigmoid(G) * (w V): persistent, operands staged
//                 by direct-to-LDS loads (N % 8 == 0)
//   pwa_gemm<FWD> the same product with register-staged operands (any N),
//                 and dV = w^T dA together with the dw tiles
//   pwa_bwd_pre   dA = dO*sigmoid(G), dG = dO*O*(1-sigmoid(G))
//   pwa_dw        split-K GEMM dw_p[h,i,j] = sum_{s in chunk p, c} dA[s,i,h,c] V[s,j,h,c]
//   pwa_db        dw = sum_p dw_p (index order), db = w*(dw - sum_j w*dw)
#include <atomic>
#include <type_traits>

#include "pba_device.h"
#include "pba_kernels.h"

namespace pba {

namespace {
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u16 lo16(uint32_t w) { return (u16)(w & 0xFFFFu); }
__device__ __forceinline__ u16 hi16(uint32_t w) { return (u16)(w >> 16); }
}  // namespace

// ------------------------------------------------------------------ softmax
// One wave per (h, i) row.
__global__ void __launch_bounds__(256) pwa_softmax_kernel(PwaArgs a, u16* wt) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int N = a.N;
  if (row >= (long long)a.H * N) return;
  const int h = (int)(row / N), i = (int)(row % N);
  const u16* brow = static_cast<const u16*>(a.b) + row * N;
  float mx = kNegInf;
  for (int j = lane; j < N; j += 64) {
    const bool keep = a.mask == nullptr || a.mask[j] != 0;
    if (keep) mx = fmaxf(mx, bf2f(brow[j]));
  }
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float msafe = (mx == kNegInf) ? 0.f : mx;
  float l = 0.f;
  for (int j = lane; j < N; j += 64) {
    const bool keep = a.mask == nullptr || a.mask[j] != 0;
    if (keep) l += expf(bf2f(brow[j]) - msafe);
  }
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  u16* wrow = static_cast<u16*>(a.w) + row * N;
  u16* wcol = wt + (size_t)h * N * N + i;
  for (int j = lane; j < N; j += 64) {
    const bool keep = a.mask == nullptr || a.mask[j] != 0;
    const float w = keep ? expf(bf2f(brow[j]) - msafe) * inv : 0.f;
    const u16 wb = f2bf(w);
    wrow[j] = wb;
    if (wt) wcol[(size_t)j * N] = wb;
  }
  if (lane == 0 && a.lse_w) a.lse_w[row] = l > 0.f ? msafe + logf(l) : kNegInf;
}

// Vectorised variants for N % 8 == 0 and N <= 512 CPL (key mask, if any,
// 8-byte aligned): one wave per (h, i) row as above, but lane chunk
// c = lane + 64 m covers 8 consecutive keys with 16-byte accesses and the
// row stays in registers, so b (and, in the db kernel, the partials) are
// read once.
__device__ __forceinline__ uint32_t keep_bits8(const uint8_t* mask, int c) {
  if (mask == nullptr) return 0xFFu;
  const uint2 m = *reinterpret_cast<const uint2*>(mask + 8 * c);
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bits |= (((m.x >> (8 * e)) & 0xFFu) != 0u ? 1u : 0u) << e;
    bits |= (((m.y >> (8 * e)) & 0xFFu) != 0u ? 1u : 0u) << (4 + e);
  }
  return bits;
}

template <int CPL>
__global__ void __launch_bounds__(256) pwa_softmax_vec_kernel(PwaArgs a) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int N = a.N, nch = N / 8;
  if (row >= (long long)a.H * N) return;
  const u16* brow = static_cast<const u16*>(a.b) + row * N;
  float x[CPL][8];
  float mx = kNegInf;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = lane + 64 * m;
    const bool ok = c < nch;
    const u32x4 raw = ok ? ld16(brow + 8 * c) : u32x4{0, 0, 0, 0};
    const uint32_t keep = ok ? keep_bits8(a.mask, c) : 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t hw = (e & 1) ? (raw[e >> 1] >> 16) : (raw[e >> 1] & 0xFFFFu);
      x[m][e] = ((keep >> e) & 1u) ? bf2f((u16)hw) : kNegInf;
      mx = fmaxf(mx, x[m][e]);
    }
  }
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float msafe = (mx == kNegInf) ? 0.f : mx;
  float l = 0.f;
#pragma unroll
  for (int m = 0; m < CPL; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[m][e] = expf(x[m][e] - msafe);  // masked and absent keys: exp(-inf) = 0
      l += x[m][e];
    }
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  u16* wrow = static_cast<u16*>(a.w) + row * N;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = lane + 64 * m;
    if (c < nch)
      *reinterpret_cast<u32x4*>(wrow + 8 * c) =
          u32x4{pack2(x[m][0] * inv, x[m][1] * inv), pack2(x[m][2] * inv, x[m][3] * inv),
                pack2(x[m][4] * inv, x[m][5] * inv), pack2(x[m][6] * inv, x[m][7] * inv)};
  }
  if (lane == 0 && a.lse_w) a.lse_w[row] = l > 0.f ? msafe + logf(l) : kNegInf;
}

// w^T of every head through 64 x 64 LDS tiles (N % 8 == 0): coalesced
// 16-byte reads of w rows and 16-byte writes of w^T rows.
__global__ void __launch_bounds__(256) pwa_transpose_kernel(const u16* __restrict__ w, u16* __restrict__ wt, int N) {
  __shared__ u16 tile[64][72];
  const int nt = (N + 63) / 64;
  const int t = blockIdx.x;
  const int h = t / (nt * nt), ti = (t / nt) % nt, tj = t % nt;
  const u16* src = w + (size_t)h * N * N;
  u16* dst = wt + (size_t)h * N * N;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = tid + 256 * it;
    const int r = q >> 3, c8 = q & 7;  // row r of the tile, 8 columns from 8 c8
    const int i = ti * 64 + r, j = tj * 64 + 8 * c8;
    const u32x4 v = (i < N && j < N) ? ld16(src + (size_t)i * N + j) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(&tile[r][8 * c8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = tid + 256 * it;
    const int r = q >> 3, c8 = q & 7;  // row r of w^T's tile (column r of w's), 8 entries from 8 c8
    const int j = tj * 64 + r, i = ti * 64 + 8 * c8;
    if (j < N && i < N) {
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)tile[8 * c8 + 2 * e][r] | ((uint32_t)tile[8 * c8 + 2 * e + 1][r] << 16);
      *reinterpret_cast<u32x4*>(dst + (size_t)j * N + i) = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

// ------------------------------------------------------------------ dw split-K GEMM
// dw_p[h][i][j] = sum_{s in chunk p} sum_c dA[s,i,h,c] V[s,j,h,c].  Both operands
// keep their natural layout (channels contiguous = the MFMA k axis).
// Workgroup tile 256 i x 256 j, eight waves of 64 i x 128 j; 64 k values
// (64/DP MSA rows) staged per iteration.
template <int DP>
struct PwaDwSmem {
  static constexpr int SPS = 64 / DP;        // MSA rows per stage (64 k values)
  static constexpr int KS = 2;               // k steps of 32 per stage
  // [buffer][operand]: dA fragments [it][ks][lane], then V fragments
  // [jt][ks][lane]; one buffer spans 64 KB, so every read of a buffer is an
  // immediate offset from one base address
  u32x4 ab[2][2][16 * KS * 64];
};

// One workgroup's tile: wg is its index among the nwg dw workgroups, which
// occupy the first grid slots (the dispatcher sends slot w to XCD w mod 8).
template <int DP>
__device__ __forceinline__ void pwa_dw_tile(int wg, int nwg, PwaDwSmem<DP>& sm, const u16* __restrict__ dA,
                                            const u16* __restrict__ V, float* __restrict__ partial, int S, int N,
                                            int H, int d, int spc, int nt1) {
  using Sm = PwaDwSmem<DP>;
  constexpr int KS = Sm::KS, SPS = Sm::SPS;
  constexpr int C8 = DP / 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int wi = wave & 3, wj = wave >> 2;
  const int L = xcd_remap(wg, nwg);
  // logical order: the nt1 x nt1 tiles fastest, then the head, then the
  // chunk: workgroups reading the same 128-byte lines (neighbouring heads of
  // the same rows) are adjacent and share an XCD's L2
  const int tile = L % (nt1 * nt1);
  const int hp = L / (nt1 * nt1);
  const int h = hp % H, p = hp / H;
  const int it0 = (tile / nt1) * 256, jt0 = (tile % nt1) * 256;
  const int sb = p * spc, se = min(S, sb + spc);
  const size_t srow = (size_t)N * H * d;
  const size_t krow = (size_t)H * d;

  // per stage: SPS MSA rows x 256 tokens x C8 chunks, for each operand.
  // Chunk q of a stage is written to LDS slot q (lane-contiguous 16-byte
  // writes): slot (t, ks, ga, r) holds token 16t + r, MSA row ks / (DP/32)
  // of the stage, channels 8 (4 (ks mod DP/32) + ga) .. +7.  Loads are
  // branch-free buffer loads; elements past the tensors (and stages past
  // the chunk) read as zero.  Both operands stream from HBM, so they are
  // fetched two stages ahead through a ring of two register stages.
  constexpr int NCHUNK = SPS * 256 * C8;    // chunks of 16 B per operand
  constexpr int PER = NCHUNK / 512;         // per thread
  constexpr uint32_t kOob = 0xFFFFFFF0u;
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(dA, (uint32_t)((size_t)S * srow * 2));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V, (uint32_t)((size_t)S * srow * 2));
  u32x4 ra[2][PER], rb[2][PER];
  auto fetch = [&](u32x4 (&da)[PER], u32x4 (&db)[PER], int s_begin) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int q = tid + 512 * it;
      const int r = q & 15, ga = (q >> 4) & 3, ks = (q >> 6) % KS, t = (q >> 6) / KS;
      const int sl = ks / (DP / 32), c8 = 4 * (ks % (DP / 32)) + ga;
      const int s = s_begin + sl, tok = 16 * t + r;
      const int ia = it0 + tok, jb = jt0 + tok;
      const bool cok = s < se && 8 * c8 < d;
      const size_t base = s * srow + (size_t)h * d + 8 * c8;
      da[it] = buf_load16(ars, (cok && ia < N) ? (uint32_t)((base + (size_t)ia * krow) * 2) : kOob);
      db[it] = buf_load16(vrs, (cok && jb < N) ? (uint32_t)((base + (size_t)jb * krow) * 2) : kOob);
    }
  };
  auto commit = [&](const u32x4 (&da)[PER], const u32x4 (&db)[PER], int buf) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int q = tid + 512 * it;
      sm.ab[buf][0][q] = da[it];
      sm.ab[buf][1][q] = db[it];
    }
  };

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[4][8];
#pragma unroll
  for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
    for (int b8 = 0; b8 < 8; ++b8) acc[a4][b8] = zero4;

  const int nst = se > sb ? (se - sb + SPS - 1) / SPS : 0;
  auto stage_s = [&](int st) { return sb + SPS * st; };
  fetch(ra[0], rb[0], stage_s(0));
  fetch(ra[1], rb[1], stage_s(1));
  commit(ra[0], rb[0], 0);
  __syncthreads();
  // stage st (parity S): loads of stage st + 2 into register stage S,
  // products of stage st from LDS buffer S, stage st + 1 into buffer S ^ 1
  auto step = [&](auto S_c, int st) {
    constexpr int buf = decltype(S_c)::value;
    fetch(ra[buf], rb[buf], stage_s(st + 2));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 af[4], bfr[8];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) af[a4] = as_bf8(sm.ab[buf][0][((4 * wi + a4) * KS + ks) * 64 + lane]);
#pragma unroll
      for (int b8 = 0; b8 < 8; ++b8) bfr[b8] = as_bf8(sm.ab[buf][1][((8 * wj + b8) * KS + ks) * 64 + lane]);
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int b8 = 0; b8 < 8; ++b8) acc[a4][b8] = mfma32(af[a4], bfr[b8], acc[a4][b8]);
    }
    commit(ra[buf ^ 1], rb[buf ^ 1], buf ^ 1);
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 2) {
    step(std::integral_constant<int, 0>{}, st);
    if (st + 1 < nst) step(std::integral_constant<int, 1>{}, st + 1);
  }

  // lane (g, n) of tile (a4, b8) holds rows i = 4g..4g+3 of column j = n
  float* part = partial + ((size_t)p * H + h) * N * N;
#pragma unroll
  for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
    for (int b8 = 0; b8 < 8; ++b8) {
      const int j = jt0 + 128 * wj + 16 * b8 + ln;
      if (j >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = it0 + 64 * wi + 16 * a4 + 4 * g + r;
        if (i < N) part[(size_t)i * N + j] = acc[a4][b8][r];
      }
    }
}

// ------------------------------------------------------------------ GEMM with transposed X
// out^T[(s,c)][n] = sum_k X[s,k,h,c] * W[h,n,k]
//   forward:  X = V,  W = w   (n = i, k = j), epilogue * sigmoid(G)
//   dV:       X = dA, W = w^T (n = j, k = i), no epilogue; this launch also
//             carries the dw partials (DW): they read the same dA and do not
//             depend on dV, so the first ndw_slots workgroups (rounded up to
//             a multiple of 8 so both parts keep their XCD mapping) run the
//             long dw tiles and the dV tiles fill the CUs they leave free
// Workgroup tile: 256 columns (s, c) x 256 rows n of one head, K in chunks
// of 64 tokens; eight waves, each 64 columns x 128 rows (4 x 8 accumulator
// tiles).  X is staged row-major ([token][(s,c)], 16-byte writes) and read
// as the A operand through the transpose read; W is staged in operand order.
// Within each 32-token step the k slot (g, v) of both operands is token
// 4g + v (v < 4) or 16 + 4g + v - 4 (v >= 4): one transpose read then covers
// 16 consecutive rows, and with a row stride of 8 (mod 64) dwords those rows
// fall in distinct LDS banks.
// Workgroup order: heads go in pairs (the two 64-byte halves of one
// 128-byte line of X at d = 32); logical order is pair, then column tile,
// then head within the pair, then n tile.  Contiguous logical ranges run on
// one XCD, so each XCD works on one pair at a time: both halves of every X
// line are consumed from its L2, and the pair's two w planes stay resident.
struct PwaDwArgs {
  const u16* V;
  float* partial;
  int P, spc, nt1, ndw, ndw_slots;
};

template <int DP, bool FWD, bool WAL, bool DW>
__global__ void __launch_bounds__(512) pwa_gemm_kernel(const u16* __restrict__ X, const u16* __restrict__ W,
                                                       const u16* __restrict__ G, u16* __restrict__ out,
                                                       int S, int N, int H, int d, int ncolt, int nnt,
                                                       PwaDwArgs dw) {
  constexpr int SPT = 256 / DP;  // MSA rows per column tile
  constexpr int C8 = DP / 8;     // 16-byte chunks per (s, token) row
  constexpr int RSX = 272;       // X tile row stride (elements): 136 dwords = 8 mod 64
  struct Smem {
    u16 sx[2][64 * RSX];       // X tiles [token][(s, c)]
    u32x4 sw[2][16 * 2 * 64];  // W operands [nt][kh][lane]
  };
  static_assert(sizeof(PwaDwSmem<DP>) <= sizeof(Smem), "dw tiles reuse the product's LDS");
  __shared__ Smem sm;
  int wg = blockIdx.x, nwg = gridDim.x;
  if constexpr (DW) {
    if (wg < dw.ndw_slots) {
      if (wg < dw.ndw)
        pwa_dw_tile<DP>(wg, dw.ndw, *reinterpret_cast<PwaDwSmem<DP>*>(&sm), X, dw.V, dw.partial, S, N, H, d, dw.spc,
                        dw.nt1);
      return;
    }
    wg -= dw.ndw_slots;
    nwg -= dw.ndw_slots;
  }
  auto& sx = sm.sx;
  auto& sw = sm.sw;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int wc = wave & 3, wn = wave >> 2;
  const int L = xcd_remap(wg, nwg);
  const int nt_blk = L % nnt;
  const int hp = (L / nnt) & 1;
  const int colt = (L / (2 * nnt)) % ncolt;
  const int h = 2 * (L / (2 * nnt * ncolt)) + hp;
  if (h >= H) return;  // odd H: the last pair has one head (whole workgroup, before any barrier)
  const int s0 = colt * SPT, n0 = nt_blk * 256;
  const u16* Wh = W + (size_t)h * N * N;
  const size_t srow = (size_t)N * H * d;   // stride of s in [S,N,H,d]
  const size_t krow = (size_t)H * d;       // stride of the token index
  // Operand loads are buffer loads with no branch around them (so the
  // compiler can count outstanding loads exactly); an element outside the
  // tensors gets an offset past the resource's end and reads as zero.
  // The host limits these tensors to fewer than 2^32 - 2^7 bytes.
  constexpr uint32_t kOob = 0xFFFFFFF0u;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(X, (uint32_t)((size_t)S * srow * 2));
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(Wh, (uint32_t)((size_t)N * N * 2));

  // X staging: chunk c = tid + 512 it -> token row c / 32, 16-byte column chunk c % 32
  // W staging: pair p = tid + 512 it -> row n, k step kh, chunk pair (m, m+2)
  // X (streamed from HBM) is fetched two K chunks ahead through a ring of two
  // register stages; W (a few MB, resident in L2) one chunk ahead.
  u32x4 rx[2][4], rw[4];
  auto wchunk = [&](int n, int k) -> u32x4 {
    if constexpr (WAL) {  // N % 8 == 0: a chunk is either inside a row or past it
      return buf_load16(wrs, (n < N && k < N) ? (uint32_t)(((size_t)n * N + k) * 2) : kOob);
    }
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = k + 2 * e;
      const uint32_t lo = (n < N && kk < N) ? Wh[(size_t)n * N + kk] : 0u;
      const uint32_t hi = (n < N && kk + 1 < N) ? Wh[(size_t)n * N + kk + 1] : 0u;
      w4[e] = lo | (hi << 16);
    }
    return u32x4{w4[0], w4[1], w4[2], w4[3]};
  };
  // chunks past the last one read as zeros (every fetch is issued)
  auto fetch_x = [&](u32x4 (&dst)[4], int k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + 512 * it;
      const int row = c >> 5, cc = c & 31;
      const int sl = cc / C8, c8 = cc % C8;
      const int s = s0 + sl, k = k0 + row;
      dst[it] = buf_load16(xrs, (s < S && k < N && 8 * c8 < d)
                                    ? (uint32_t)((s * srow + (size_t)k * krow + (size_t)h * d + 8 * c8) * 2)
                                    : kOob);
    }
  };
  auto fetch_w = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int pr = tid + 512 * it;
      const int nn = pr & 15, m = (pr >> 4) & 1, kh = (pr >> 5) & 1, nt = pr >> 6;
      const int n = n0 + 16 * nt + nn, k = k0 + 32 * kh + 8 * m;
      rw[2 * it] = wchunk(n, k);
      rw[2 * it + 1] = wchunk(n, k + 16);
    }
  };
  auto commit = [&](const u32x4 (&src)[4], int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int c = tid + 512 * it;
      *reinterpret_cast<u32x4*>(&sx[buf][(c >> 5) * RSX + 8 * (c & 31)]) = src[it];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int pr = tid + 512 * it;
      const int nn = pr & 15, m = (pr >> 4) & 1, kh = (pr >> 5) & 1, nt = pr >> 6;
      const u32x4 lo = rw[2 * it], hi = rw[2 * it + 1];  // tokens 8m..8m+7 and 16+8m..16+8m+7
      // lane group 2m takes tokens 8m..8m+3 | 16+8m..+3, group 2m+1 the next four of each
      sw[buf][(nt * 2 + kh) * 64 + (2 * m) * 16 + nn] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      sw[buf][(nt * 2 + kh) * 64 + (2 * m + 1) * 16 + nn] = u32x4{lo[2], lo[3], hi[2], hi[3]};
    }
  };

  // A operand (X^T) of column tile ct: lane (g, j) with j = 4e + a reads
  // the 4 columns cb + 8a .. cb + 8a + 3 of token rows r0 + e and r0 + 16 + e,
  // where cb = 64 wc + 32 (ct / 2) + 4 (ct mod 2).  Result lane (g, n) of
  // tiles (2p, 2p + 1) then holds columns 64 wc + 32 p + 8g .. + 7: 8
  // consecutive channels, so the epilogue moves 16 bytes per access.
  auto xt_frag = [&](const u16* tile, int r0, int cb, int ln_) -> bf16x8 {
    const int j = ln_ & 15;
    const int e = j >> 2, a = j & 3;
    const u32x2 lo = lds_tr16(tile + (r0 + e) * RSX + cb + 8 * a);
    const u32x2 hi = lds_tr16(tile + (r0 + 16 + e) * RSX + cb + 8 * a);
    return as_bf8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[4][8];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[ct][nt] = zero4;

  // The nnt workgroups of one column tile (and the two heads of a pair) take
  // the K chunks in the same order, so each X chunk is fetched once from HBM
  // and read by the others from L2 while it is still resident.
  const int nkc = (N + 63) / 64;
  fetch_x(rx[0], 0);
  fetch_w(0);
  fetch_x(rx[1], 64);
  commit(rx[0], 0);
  __syncthreads();
  // step kcix (parity S): X of chunk kcix + 2 into register stage S, W of
  // chunk kcix + 1; products of chunk kcix from LDS buffer S; then chunk
  // kcix + 1 (X from stage S ^ 1) into LDS buffer S ^ 1
  auto step = [&](auto S_c, int kcix) {
    constexpr int buf = decltype(S_c)::value;
    fetch_w(64 * (kcix + 1));
    fetch_x(rx[buf], 64 * (kcix + 2));
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 af[4], bfr[8];
      const int r0 = 32 * kh + 4 * g;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) af[ct] = xt_frag(sx[buf], r0, 64 * wc + 32 * (ct >> 1) + 4 * (ct & 1), lane);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) bfr[nt] = as_bf8(sw[buf][((8 * wn + nt) * 2 + kh) * 64 + lane]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[ct][nt] = mfma32(af[ct], bfr[nt], acc[ct][nt]);
    }
    commit(rx[buf ^ 1], buf ^ 1);
    __syncthreads();
  };
  for (int kcix = 0; kcix < nkc; kcix += 2) {
    step(std::integral_constant<int, 0>{}, kcix);
    if (kcix + 1 < nkc) step(std::integral_constant<int, 1>{}, kcix + 1);
  }

  // epilogue: lane (g, n) of tiles (2p, 2p + 1, nt) holds columns
  // 64 wc + 32 p + 8g .. + 7 of row n: one MSA row's channels 8g'..8g'+7.
  // Tiles fully inside the tensors take a branch-free path that issues the
  // gate loads of a column pair together; ragged tiles check every element.
  auto gate8 = [&](const f32x4& a0, const f32x4& a1, u32x4 gr) -> u32x4 {
    float o[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    if constexpr (FWD) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] *= sigmoidf_fast(bf2f(lo16(gr[e])));
        o[2 * e + 1] *= sigmoidf_fast(bf2f(hi16(gr[e])));
      }
    }
    return u32x4{pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
  };
  const bool full = s0 + SPT <= S && n0 + 256 <= N && d == DP;
  if (full) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int col = 64 * wc + 32 * p + 8 * g;
      const size_t base = (s0 + col / DP) * srow + (size_t)(n0 + 128 * wn + ln) * krow + (size_t)h * d + col % DP;
      u32x4 gr[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        gr[nt] = FWD ? *reinterpret_cast<const u32x4*>(G + base + (size_t)16 * nt * krow) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        *reinterpret_cast<u32x4*>(out + base + (size_t)16 * nt * krow) = gate8(acc[2 * p][nt], acc[2 * p + 1][nt], gr[nt]);
    }
    return;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int col = 64 * wc + 32 * p + 8 * g;
    const int sl = col / DP, c = col % DP;  // d is a multiple of 8: all 8 channels are valid or none
    const int s = s0 + sl;
    if (s >= S || c >= d) continue;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int nrow = n0 + 128 * wn + 16 * nt + ln;
      if (nrow >= N) continue;
      const size_t off = s * srow + (size_t)nrow * krow + (size_t)h * d + c;
      const u32x4 gr = FWD ? *reinterpret_cast<const u32x4*>(G + off) : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(out + off) = gate8(acc[2 * p][nt], acc[2 * p + 1][nt], gr);
    }
  }
}

// ------------------------------------------------------------------ GEMM, direct-to-LDS pipeline
// The forward product of pwa_gemm_kernel (same tile and tile order, N % 8 ==
// 0) with the load path rebuilt around the LDS, run as a persistent kernel:
//  - operands go from memory straight into LDS (buffer loads with an LDS
//    destination): no registers hold staged data and no LDS stores are issued;
//  - a workgroup takes tiles L0, L0 + G, L0 + 2G, ... (G = grid size), and its
//    chunks (64 tokens) form one stream across its tiles.  X chunks rotate
//    through three LDS buffers and W chunks through two: after the barrier
//    that retires chunk q, chunk q + 3 of X (from HBM) and q + 2 of W (from
//    L2) go into the buffers chunk q held, one load after each group of
//    products (a burst of them right after the barrier would fill the
//    address queue and stall every wave's issue);
//  - that barrier sits between the two 32-token halves of chunk q's
//    products: the second half's fragments are read before it and the next
//    chunk's first half during the second half's products, two reads per
//    four products;
//  - a tile's epilogue runs while the next tile's first chunks load, so
//    there is no per-tile prologue;
//  - token row r of an X chunk stores its 16-byte unit u (8 columns) at slot
//    u ^ f(r), f(r) = 4 (r mod 4) + (r / 8 mod 2).  A transposing read gives
//    lane group g token rows 8g .. 8g + 7 (so the k axis of each lane is W's
//    natural 16-byte chunk), and the four address lanes a of a row take
//    units U0 + a with alternating 8-byte halves.  With the permutation each
//    32-lane half of a read covers the 64 banks once.
// Result lane (g, n) of tile 2p + t holds half t ^ (g mod 2) of unit U0 + g;
// the epilogue swaps the two tiles of a pair on odd lane groups, so every
// lane moves the 8 channels of one unit in one 16-byte access.
__device__ __forceinline__ int xunit_swz(int r) { return 4 * (r & 3) + ((r >> 3) & 1); }

// Position of a workgroup in its tile list: tile index ti, chunk k, and the
// tile's coordinates as mixed-radix digits of L (n tile, head in the pair,
// column tile, head pair), stepped by adding the grid size digit by digit.
struct PwaCursor {
  int ti, k, ntb, hp, colt, hpr;
};

template <int DP, bool FWD>
__global__ void __launch_bounds__(512) pwa_gemm_dl_kernel(const u16* __restrict__ X, const u16* __restrict__ W,
                                                          const u16* __restrict__ G, u16* __restrict__ out,
                                                          int S, int N, int H, int d, int ncolt, int nnt) {
  constexpr int SPT = 256 / DP;    // MSA rows per column tile
  constexpr int C8 = DP / 8;       // 16-byte units per (s, token) row
  constexpr int XB = 64 * 32;      // 16-byte units per X buffer (64 tokens x 256 columns)
  constexpr int WB = 16 * 2 * 64;  // per W buffer (256 rows x 64 tokens, operand order)
  constexpr uint32_t kOob = 0xFFFFFFF0u;
  __shared__ u32x4 lds[3 * XB + 2 * WB];
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, ln = lane & 15;
  const int wc = wave & 3, wn = wave >> 2;
  const int pairs = (H + 1) / 2;
  const int ntiles = nnt * 2 * ncolt * pairs;
  const int L0 = xcd_remap(wg, nwg);
  if (L0 >= ntiles) return;  // whole workgroup, before any barrier
  const int ntw = (ntiles - L0 + nwg - 1) / nwg;  // tiles of this workgroup
  const int nkc = (N + 63) / 64;
  const int nq = ntw * nkc;                      // chunks in its stream
  const size_t srow = (size_t)N * H * d;
  const size_t krow = (size_t)H * d;
  const i32x4 xrs = rsrc_words(X, (uint32_t)((size_t)S * srow * 2));
  const i32x4 wrs = rsrc_words(W, (uint32_t)((size_t)H * N * N * 2));

  // grid size as digits of the tile numbering (n tile, head in pair, column tile, pair)
  const int g0 = nwg % nnt, g1 = (nwg / nnt) & 1, g2 = (nwg / (2 * nnt)) % ncolt, g3 = nwg / (2 * nnt * ncolt);
  auto start = [&](PwaCursor& c) {
    c.ti = 0;
    c.k = 0;
    c.ntb = L0 % nnt;
    c.hp = (L0 / nnt) & 1;
    c.colt = (L0 / (2 * nnt)) % ncolt;
    c.hpr = L0 / (2 * nnt * ncolt);
  };
  auto advance = [&](PwaCursor& c) {
    if (++c.k < nkc) return;
    c.k = 0;
    ++c.ti;
    c.ntb += g0;
    int cy = c.ntb >= nnt;
    c.ntb -= cy ? nnt : 0;
    c.hp += g1 + cy;
    cy = c.hp >= 2;
    c.hp -= cy ? 2 : 0;
    c.colt += g2 + cy;
    cy = c.colt >= ncolt;
    c.colt -= cy ? ncolt : 0;
    c.hpr += g3 + cy;
  };

  // Staging: this wave fills four 1 KB blocks of each chunk.  X block b =
  // 4 wave + i holds token rows 2b, 2b + 1 (lane l: row 2b + l / 32, slot
  // l mod 32); W block b holds n tile b / 2, token half b mod 2 in operand
  // order (lane 16 g + n: row n, tokens 8g .. 8g + 7 of the half).  Offsets
  // are recomputed per load rather than kept in registers.
  auto load_x1 = [&](int q, const PwaCursor& c, int i) {  // block i of this wave's share of X chunk q
    const int h = 2 * c.hpr + c.hp, s0 = c.colt * SPT;
    const int r = 2 * (4 * wave + i) + (lane >> 5);
    const int u = (lane & 31) ^ xunit_swz(r);
    const int sl = u / C8, c8 = u % C8;
    const int k = 64 * c.k + r;
    const bool ok = c.ti < ntw && h < H && s0 + sl < S && 8 * c8 < d && k < N;
    const uint32_t off = ok ? (uint32_t)((((size_t)(s0 + sl) * srow + (size_t)k * krow + (size_t)h * d) + 8 * c8) * 2)
                            : kOob;
    lds_dma16(xrs, lds_addr(lds + (q % 3) * XB + (4 * wave + i) * 64), off);
  };
  auto load_w1 = [&](int q, const PwaCursor& c, int i) {  // block i of this wave's share of W chunk q
    const int h = 2 * c.hpr + c.hp, n0 = c.ntb * 256;
    const int b = 4 * wave + i, nr = 16 * (b >> 1) + ln, kk = 32 * (b & 1) + 8 * g;
    const bool ok = c.ti < ntw && h < H && n0 + nr < N && 64 * c.k + kk < N;
    const uint32_t base = (uint32_t)(((size_t)h * N * N + (size_t)n0 * N) * 2);
    const uint32_t off = ok ? base + (uint32_t)((nr * N + kk + 64 * c.k) * 2) : kOob;
    lds_dma16(wrs, lds_addr(lds + 3 * XB + (q & 1) * WB + (4 * wave + i) * 64), off);
  };

  // Fragment reads.  A operand (X^T) of tile 2p + t: lane (g, 4e + a) reads
  // token rows 8g + e and 8g + 4 + e of the half at unit 8 wc + 4p + a, half
  // t ^ (a mod 2); f of those rows is the same (it only sees r mod 4 and r / 8
  // mod 2), so the four reads of a lane share one permuted slot per unit.
  const int e = (lane >> 2) & 3, a = lane & 3;
  const int rr = 8 * g + e;
  const int fsw = xunit_swz(rr);
  uint32_t xro[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int t = 0; t < 2; ++t) xro[p][t] = (uint32_t)((rr * 32 + ((8 * wc + 4 * p + a) ^ fsw)) * 16 + 8 * (t ^ (a & 1)));
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[4][8];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[ct][nt] = zero4;

  // One half-chunk of products (fragments ua, ub) with the 16 reads of the
  // next fragments (chunk q, half kh into va, vb) spread through it, two reads
  // per four products.  Issuing all 16 reads first would leave more LDS
  // operations outstanding than the counter can wait past, so the products
  // would wait for the newest reads behind every other wave's.  Products go
  // n tile by n tile (group j uses W fragment j and all four X fragments) and
  // the X fragments are read first, so each fragment is read several groups
  // before the next half needs it.  issue(j) runs after group j.
  auto half_step = [&](auto read, int q, int kh, bf16x8 (&va)[4], bf16x8 (&vb)[8], const bf16x8 (&ua)[4],
                       const bf16x8 (&ub)[8], auto&& issue) {
    constexpr bool RD = decltype(read)::value;
    const char* xb = reinterpret_cast<const char*>(lds + (q % 3) * XB) + kh * 32 * 512;
    const u32x4* wb = lds + 3 * XB + (q & 1) * WB + kh * 64 + 8 * wn * 128 + lane;
    u32x2 lo[4], hi[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (RD) {
        if (j < 4) {
          const u16* p0 = reinterpret_cast<const u16*>(xb + xro[j >> 1][j & 1]);
          lo[j] = lds_tr16(p0);
          hi[j] = lds_tr16(p0 + 4 * 256);  // token rows + 4
        } else {
          vb[2 * (j - 4)] = as_bf8(wb[(2 * (j - 4)) * 128]);
          vb[2 * (j - 4) + 1] = as_bf8(wb[(2 * (j - 4) + 1) * 128]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct][j] = mfma32(ua[ct], ub[j], acc[ct][j]);
      if constexpr (RD) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                    // four products
      issue(j);
    }
    if constexpr (RD) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) va[ct] = as_bf8(u32x4{lo[ct][0], lo[ct][1], hi[ct][0], hi[ct][1]});
    }
  };
  auto read_frags = [&](int q, int kh, bf16x8 (&af)[4], bf16x8 (&bf)[8]) {
    const char* xb = reinterpret_cast<const char*>(lds + (q % 3) * XB) + kh * 32 * 512;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const u16* p0 = reinterpret_cast<const u16*>(xb + xro[ct >> 1][ct & 1]);
      const u32x2 lo = lds_tr16(p0);
      const u32x2 hi = lds_tr16(p0 + 4 * 256);
      af[ct] = as_bf8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    const u32x4* wb = lds + 3 * XB + (q & 1) * WB;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) bf[nt] = as_bf8(wb[((8 * wn + nt) * 2 + kh) * 64 + lane]);
  };

  // Epilogue of the tile at cursor c: lane (g, n) of tiles 2p and 2p + 1
  // holds the 8 channels of unit U = 8 wc + 4p + g of the column tile in row
  // n: tile 2p + (g mod 2) has channels 0..3, the other tile 4..7.  Gate
  // reads and output writes are buffer accesses with the range check, always
  // 16 of each per lane, so the count of memory operations stays fixed.
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(FWD ? G : out, (uint32_t)((size_t)S * srow * 2));
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(out, (uint32_t)((size_t)S * srow * 2));
  auto epilogue = [&](const PwaCursor& c) {
    // the lane index goes through an empty asm so that the per-lane address
    // terms below are computed here, not hoisted into registers that stay
    // live through the whole product loop
    int el = lane;
    asm volatile("" : "+v"(el));
    const int g = el >> 4, ln = el & 15;
    const bool odd = (g & 1) != 0;
    const int h = 2 * c.hpr + c.hp, s0 = c.colt * SPT, n0 = c.ntb * 256;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int col = 8 * (8 * wc + 4 * p + g);
      const int s = s0 + col / DP, cc = col % DP;  // d % 8 == 0: all 8 channels are valid or none
      const bool ok = h < H && s < S && cc < d;
      const uint32_t base = (uint32_t)((s * srow + (size_t)(n0 + 128 * wn + ln) * krow + (size_t)h * d + cc) * 2);
      auto off = [&](int nt) -> uint32_t {
        return (ok && n0 + 128 * wn + 16 * nt + ln < N) ? base + (uint32_t)(32 * nt * krow) : kOob;
      };
#pragma unroll
      for (int nb = 0; nb < 8; nb += 4) {
      u32x4 gr[4];
#pragma unroll
      for (int nt = nb; nt < nb + 4; ++nt) gr[nt - nb] = FWD ? buf_load16(grs, off(nt)) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int nt = nb; nt < nb + 4; ++nt) {
        const f32x4 lo = odd ? acc[2 * p + 1][nt] : acc[2 * p][nt];
        const f32x4 hi = odd ? acc[2 * p][nt] : acc[2 * p + 1][nt];
        float o[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (FWD) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            o[2 * k] *= sigmoidf_fast(bf2f(lo16(gr[nt - nb][k])));
            o[2 * k + 1] *= sigmoidf_fast(bf2f(hi16(gr[nt - nb][k])));
          }
        }
        const u32x4 v = {pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
        __builtin_amdgcn_raw_buffer_store_b128(v, ors, off(nt), 0, 0);
      }
      }
    }
  };

  // Every wave issues the same loads for every chunk index, past the end of
  // its stream too: there all offsets fail the range check and zeros land in
  // a retired buffer.  So the count of loads after any given one is fixed.
  // Prologue: X chunks 0..2 and W chunks 0..1 in the order X0 W0 X1 W1 X2.
  PwaCursor cx, cw, cc;
  start(cx);
  start(cw);
  start(cc);
#pragma unroll
  for (int q = 0; q < 3; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) load_x1(q, cx, i);
    advance(cx);
    if (q < 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) load_w1(q, cw, i);
      advance(cw);
    }
  }
  vm_wait<12>();
  __syncthreads();
  bf16x8 a0[4], b0[8], a1[4], b1[8];
  read_frags(0, 0, a0, b0);
  // Chunk q: half 0's products with half 1's reads; then, once this wave's
  // loads of chunk q + 1 have landed, the barrier: every wave has finished
  // reading chunk q and chunk q + 1 is complete.  After it half 1's products
  // run with the reads of chunk q + 1's first half (past the end of the
  // stream they read a retired buffer and are not used) and the loads of W
  // chunk q + 2 and X chunk q + 3 into chunk q's buffers.  In issue order
  // the loads after W(q + 1) are X(q + 2) only.  A tile's last chunk reads
  // nothing during its second half; the wave then waits for chunk q + 2 (only
  // X(q + 3) is newer), runs the epilogue and reads the next chunk's first
  // half.  So the fragment registers are free during the epilogue and the
  // next barrier needs no wait past the epilogue's writes.
  using rd_t = std::integral_constant<bool, true>;
  using nord_t = std::integral_constant<bool, false>;
  int q = 0;
  auto chunk = [&](auto read, bool wait) {
    half_step(rd_t{}, q, 1, a1, b1, a0, b0, [](int) {});
    if (wait) vm_wait<4>();
    __syncthreads();
    half_step(read, q + 1, 0, a0, b0, a1, b1, [&](int j) {
      if (j < 4) load_w1(q + 2, cw, j);
      else load_x1(q + 3, cx, j - 4);
    });
    advance(cw);
    advance(cx);
    ++q;
  };
  // Every barrier that publishes a chunk is preceded by this wave's wait for
  // its loads of that chunk, except the first barrier after an epilogue: the
  // wait before the epilogue already covered that chunk.
  for (int ti = 0; ti < ntw; ++ti) {
    for (int k = 0; k + 1 < nkc; ++k) chunk(rd_t{}, k > 0 || ti == 0);
    chunk(nord_t{}, (nkc > 1 || ti == 0) && q + 1 < nq);
    vm_wait<4>();
    epilogue(cc);
    for (int k = 0; k < nkc; ++k) advance(cc);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[ct][nt] = zero4;
    read_frags(q, 0, a0, b0);
  }
  vm_wait<0>();  // the loads past the end of the stream land before the LDS is released
}

// ------------------------------------------------------------------ backward elementwise
__global__ void __launch_bounds__(256) pwa_bwd_pre_kernel(PwaArgs a) {
  const size_t n8 = (size_t)a.S * a.N * a.H * a.d / 8;
  const size_t i8 = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i8 >= n8) return;
  const u16* dO = static_cast<const u16*>(a.dout);
  const u16* O = static_cast<const u16*>(a.out);
  const u16* G = static_cast<const u16*>(a.g);
  // read-once inputs and the write-once dG as streaming (nontemporal)
  // accesses: the dV / dw launch that follows reads dA and V again
  const u32x4 xo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dO + 8 * i8));
  const u32x4 xv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(O + 8 * i8));
  const u32x4 xg = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(G + 8 * i8));
  u32x4 ra, rg;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float f0 = bf2f(lo16(xo[e])), f1 = bf2f(hi16(xo[e]));
    const float o0 = bf2f(lo16(xv[e])), o1 = bf2f(hi16(xv[e]));
    const float s0 = sigmoidf_fast(bf2f(lo16(xg[e]))), s1 = sigmoidf_fast(bf2f(hi16(xg[e])));
    ra[e] = pack2(f0 * s0, f1 * s1);
    rg[e] = pack2(f0 * o0 * (1.f - s0), f1 * o1 * (1.f - s1));
  }
  *reinterpret_cast<u32x4*>(static_cast<u16*>(a.da) + 8 * i8) = ra;
  __builtin_nontemporal_store(rg, reinterpret_cast<u32x4*>(static_cast<u16*>(a.dg) + 8 * i8));
}

// ------------------------------------------------------------------ db
// One wave per (h, i) row: dw = sum_p partial (index order); w recomputed in
// fp32 from b and lse_w; db = w * (dw - sum_j w dw).
__global__ void __launch_bounds__(256) pwa_db_kernel(PwaArgs a) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int N = a.N;
  if (row >= (long long)a.H * N) return;
  const u16* brow = static_cast<const u16*>(a.b) + row * N;
  const float lse = a.lse_w_in[row];
  const size_t plane = (size_t)a.H * N * N;
  float t = 0.f;
  for (int j = lane; j < N; j += 64) {
    const bool keep = (a.mask == nullptr || a.mask[j] != 0) && lse != kNegInf;
    const float w = keep ? expf(bf2f(brow[j]) - lse) : 0.f;
    float dw = 0.f;
    for (int p = 0; p < a.P; ++p) dw += a.partial[p * plane + row * N + j];
    t = fmaf(w, dw, t);
  }
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
  u16* db = static_cast<u16*>(a.db) + row * N;
  for (int j = lane; j < N; j += 64) {
    const bool keep = (a.mask == nullptr || a.mask[j] != 0) && lse != kNegInf;
    const float w = keep ? expf(bf2f(brow[j]) - lse) : 0.f;
    float dw = 0.f;
    for (int p = 0; p < a.P; ++p) dw += a.partial[p * plane + row * N + j];
    db[j] = f2bf(w * (dw - t));
  }
}

template <int CPL>
__global__ void __launch_bounds__(256) pwa_db_vec_kernel(PwaArgs a) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int N = a.N, nch = N / 8;
  if (row >= (long long)a.H * N) return;
  const u16* brow = static_cast<const u16*>(a.b) + row * N;
  const float lse = a.lse_w_in[row];
  const size_t plane = (size_t)a.H * N * N;
  float w[CPL][8], dw[CPL][8];
  float t = 0.f;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = lane + 64 * m;
    const bool ok = c < nch;
    const u32x4 raw = ok ? ld16(brow + 8 * c) : u32x4{0, 0, 0, 0};
    const uint32_t keep = (ok && lse != kNegInf) ? keep_bits8(a.mask, c) : 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t hw = (e & 1) ? (raw[e >> 1] >> 16) : (raw[e >> 1] & 0xFFFFu);
      w[m][e] = ((keep >> e) & 1u) ? expf(bf2f((u16)hw) - lse) : 0.f;
      dw[m][e] = 0.f;
    }
    if (ok) {
      for (int p = 0; p < a.P; ++p) {
        const float* src = a.partial + p * plane + row * N + 8 * c;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src), hi = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dw[m][e] += lo[e];
          dw[m][4 + e] += hi[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) t = fmaf(w[m][e], dw[m][e], t);
  }
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
  u16* db = static_cast<u16*>(a.db) + row * N;
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = lane + 64 * m;
    if (c >= nch) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = w[m][e] * (dw[m][e] - t);
    *reinterpret_cast<u32x4*>(db + 8 * c) =
        u32x4{pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
  }
}

// ------------------------------------------------------------------ plan + launch
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

PwaPlan plan_pwa_bwd(int S, int N, int H, int d, bool /*bf16*/) {
  PwaPlan pl{};
  // dw chunks over S: as many as fit one round of 256 workgroups (one per CU)
  const int nt1 = (N + 255) / 256;
  const long long tiles = (long long)nt1 * nt1 * H;
  int P = (int)std::max<long long>(1, std::min<long long>(S / 2 > 0 ? S / 2 : 1, 256 / tiles));
  pl.P = P;
  size_t off = 0;
  pl.off_w = off;                                         // w and w^T
  off = align256(off + 2 * (size_t)H * N * N * 2);
  pl.off_da = off;
  off = align256(off + (size_t)S * N * H * d * 2);
  pl.off_partial = off;
  off = align256(off + (size_t)P * H * N * N * 4);
  pl.total = off;
  return pl;
}

// One workgroup per CU for the persistent product kernel (the device's CU
// count, read once per device).
static long long pwa_persistent_workgroups() {
  static std::atomic<int> cached[64];  // zero-initialised (static storage); 0 = not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);  // every thread stores the same value
  }
  return n;
}
// The vectorised row kernels need N % 8 == 0, N <= 1024 and an 8-byte
// aligned key mask; other shapes take the element-wise kernels.
static bool pwa_rows_vec(const PwaArgs& a) {
  return a.N % 8 == 0 && a.N <= 1024 && (reinterpret_cast<uintptr_t>(a.mask) & 7) == 0;
}

static hipError_t launch_softmax(const PwaArgs& a, u16* wt, hipStream_t stream) {
  const long long rows = (long long)a.H * a.N;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (!pwa_rows_vec(a)) {
    hipLaunchKernelGGL(pwa_softmax_kernel, grid, dim3(256), 0, stream, a, wt);
    return hipGetLastError();
  }
  if (a.N <= 512) hipLaunchKernelGGL(pwa_softmax_vec_kernel<1>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(pwa_softmax_vec_kernel<2>, grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || wt == nullptr) return e;
  const int nt = (a.N + 63) / 64;
  hipLaunchKernelGGL(pwa_transpose_kernel, dim3((unsigned)(a.H * nt * nt)), dim3(256), 0, stream,
                     static_cast<const u16*>(a.w), wt, a.N);
  return hipGetLastError();
}

template <bool FWD>
static hipError_t launch_gemm(const u16* X, const u16* W, const u16* G, u16* out, const PwaArgs& a,
                              hipStream_t stream) {
  const int dp = a.d <= 32 ? 32 : 64;
  const int spt = 256 / dp;
  const int ncolt = (a.S + spt - 1) / spt;
  const int nnt = (a.N + 255) / 256;
  const int pairs = (a.H + 1) / 2;
  const dim3 grid((unsigned)((long long)ncolt * nnt * 2 * pairs));
  const bool wal = (a.N & 7) == 0;
  // the pipelined kernel is persistent: one workgroup per CU walks its tiles
  const dim3 pgrid((unsigned)std::min<long long>((long long)grid.x, pwa_persistent_workgroups()));
  if (wal) {
    if (dp == 32)
      hipLaunchKernelGGL((pwa_gemm_dl_kernel<32, FWD>), pgrid, dim3(512), 0, stream, X, W, G, out, a.S, a.N, a.H, a.d,
                         ncolt, nnt);
    else
      hipLaunchKernelGGL((pwa_gemm_dl_kernel<64, FWD>), pgrid, dim3(512), 0, stream, X, W, G, out, a.S, a.N, a.H, a.d,
                         ncolt, nnt);
  } else {
    if (dp == 32)
      hipLaunchKernelGGL((pwa_gemm_kernel<32, FWD, false, false>), grid, dim3(512), 0, stream, X, W, G, out, a.S, a.N,
                         a.H, a.d, ncolt, nnt, PwaDwArgs{});
    else
      hipLaunchKernelGGL((pwa_gemm_kernel<64, FWD, false, false>), grid, dim3(512), 0, stream, X, W, G, out, a.S, a.N,
                         a.H, a.d, ncolt, nnt, PwaDwArgs{});
  }
  return hipGetLastError();
}

hipError_t launch_pwa_fwd(const PwaArgs& a, bool /*bf16*/, hipStream_t stream, KernelTimer* timer) {
  timer_start(timer, stream);
  hipError_t e = launch_softmax(a, nullptr, stream);
  if (e != hipSuccess) return e;
  timer_mark(timer, stream);
  e = launch_gemm<true>(static_cast<const u16*>(a.v), static_cast<const u16*>(a.w), static_cast<const u16*>(a.g),
                        static_cast<u16*>(a.o), a, stream);
  if (e != hipSuccess) return e;
  timer_mark(timer, stream);
  return hipSuccess;
}

hipError_t launch_pwa_bwd(const PwaArgs& args, bool /*bf16*/, hipStream_t stream, KernelTimer* timer) {
  timer_start(timer, stream);
  PwaArgs a = args;
  const size_t plane = (size_t)a.H * a.N * a.N;
  u16* w = static_cast<u16*>(a.w);
  u16* wt = w + plane;
  PwaArgs sa = a;
  sa.lse_w = nullptr;  // the backward reuses the caller's lse_w; only w, w^T are rebuilt
  hipError_t e = launch_softmax(sa, wt, stream);
  if (e != hipSuccess) return e;
  timer_mark(timer, stream);
  {
    const size_t n8 = (size_t)a.S * a.N * a.H * a.d / 8;
    hipLaunchKernelGGL(pwa_bwd_pre_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timer_mark(timer, stream);
  }
  {
    // dV = w^T dA and the dw partials in one grid (dw tiles first)
    const int dp = a.d <= 32 ? 32 : 64;
    const int spt = 256 / dp;
    const int ncolt = (a.S + spt - 1) / spt;
    const int nnt = (a.N + 255) / 256;
    const int pairs = (a.H + 1) / 2;
    const long long ngemm = (long long)ncolt * nnt * 2 * pairs;
    PwaDwArgs dw{};
    dw.V = static_cast<const u16*>(a.v);
    dw.partial = a.partial;
    dw.P = a.P;
    dw.nt1 = (a.N + 255) / 256;
    dw.spc = ((a.S + a.P - 1) / a.P + 1) & ~1;  // even number of MSA rows per chunk
    // chunks past the end write zero partials, so every one of the P slots is defined
    dw.ndw = dw.nt1 * dw.nt1 * a.H * a.P;
    dw.ndw_slots = (dw.ndw + 7) & ~7;
    const dim3 grid((unsigned)(dw.ndw_slots + ngemm));
    const bool wal = (a.N & 7) == 0;
    const u16* dA = static_cast<const u16*>(a.da);
    u16* dV = static_cast<u16*>(a.dv);
    // (the register-staged kernel: in this launch, next to the dw tiles, it
    // measured faster than the pipelined one)
#define PBA_PROD_LAUNCH(DPV, WALV)                                                                           \
  hipLaunchKernelGGL((pwa_gemm_kernel<DPV, false, WALV, true>), grid, dim3(512), 0, stream, dA, wt, nullptr, dV, \
                     a.S, a.N, a.H, a.d, ncolt, nnt, dw)
    if (dp == 32) {
      if (wal) PBA_PROD_LAUNCH(32, true); else PBA_PROD_LAUNCH(32, false);
    } else {
      if (wal) PBA_PROD_LAUNCH(64, true); else PBA_PROD_LAUNCH(64, false);
    }
#undef PBA_PROD_LAUNCH
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timer_mark(timer, stream);
  }
  {
    const long long rows = (long long)a.H * a.N;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (!pwa_rows_vec(a)) hipLaunchKernelGGL(pwa_db_kernel, grid, dim3(256), 0, stream, a);
    else if (a.N <= 512) hipLaunchKernelGGL(pwa_db_vec_kernel<1>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(pwa_db_vec_kernel<2>, grid, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timer_mark(timer, stream);
  }
  return hipSuccess;
}

}  // namespace pba

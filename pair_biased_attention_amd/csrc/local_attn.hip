// local_attn.hip - windowed (sequence-local) pair-biased gated attention on
// gfx950, forward and backward.
//
// AlphaFold3 open-source implementation page (molayo1419.me), section "Model
// Efficiency": for the atom attention encoder and decoder the authors tried
// an implementation whose memory grows linearly with the number of atoms,
// next to the plain reuse of the dense pair-biased attention kernel.  Linear
// memory means a fixed window of keys per query and a pair bias that exists
// only inside the windows.  Here query block q (atoms 32q .. 32q+31) attends
// the 128 keys 32q - 48 .. 32q + 79 (slot s = key - 32q + 48); bias and dbias
// are [H, nqb, 32, 128]; everything else (scale, key mask, gate, natural-log
// lse, rows without keys) is as in the dense kernels.
//
// Kernels (d <= 32, bf16):
//  * forward: one wave per (b, h, query block), four consecutive blocks per
//    workgroup sharing one staged V window.  S^T = K Q^T for the whole
//    window (8 key tiles x 2 query tiles), exact softmax in registers (no
//    online rescale: the window fits), O^T = V^T P^T with V read transposed
//    from LDS.  The key order inside the score tiles is permuted
//    so that lane group g owns the 32 contiguous slots 32g .. 32g + 31: its
//    bias comes as four 16-byte loads per query row.
//  * backward, query-stationary: one wave per (h, query block, 16-query tile,
//    batch chunk), two blocks per workgroup sharing a staged K window, walks
//    the chunk's batch rows in order, recomputes P, forms dS and dQ = dS K
//    and accumulates dS in registers: one dbias partial per chunk, summed
//    over chunks in a fixed order afterwards.
//  * backward, key-stationary (in the same launch as the query-stationary
//    role, whose workgroups fill the slots after it): one wave per 16-key tile.  Each key tile lies
//    wholly inside the windows of exactly four query blocks (the windows are
//    16-aligned).  A workgroup walks consecutive groups of four key tiles
//    with a ring of query blocks in LDS; each wave forms S = Q K^T (bias
//    added on the matrix core by identity products), P, dP, dS and
//    accumulates dV = P^T dA and dK = dS^T Q.  No atomics anywhere.
#include <algorithm>

#include "pba.h"
#include "pba_device.h"
#include "pba_kernels.h"

namespace pba {
namespace {

constexpr uint32_t kOob = 0xFFFFFFF0u;
constexpr int kRS = 40;  // LDS row stride (elements) of a staged 32-channel row

// Score tile t (0..7), result row r (0..15) -> window slot: lane group g (rows
// 4g..4g+3) owns slots 32g .. 32g+31, in the order (t, r % 4).
__device__ __forceinline__ int slot_of(int t, int r) { return 32 * (r >> 2) + 4 * t + (r & 3); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Sum over the four lanes of a lane column; every one of them gets the same bits.
__device__ __forceinline__ float sum_over_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  const uint32_t v = __float_as_uint(x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
}

__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

}  // namespace

// ------------------------------------------------------------------ forward
// The four waves of a workgroup take four consecutive query blocks of one
// (b, h) and share one staged V window: keys 128qg - 48 .. 128qg + 175 (224
// rows), wave w's window starting at row 32w.
constexpr int kFwdRows = 224;

__global__ void __launch_bounds__(256) local_fwd_kernel(LocalArgs a) {
  __shared__ __attribute__((aligned(16))) u16 sV[kFwdRows * kRS];
  __shared__ __attribute__((aligned(16))) uint8_t sKeep[kFwdRows + 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const int N = a.N, d = a.d, nqb = a.nqb;
  const int nqg = (nqb + 3) / 4;
  const int bh = blockIdx.x / nqg;
  const int qg = blockIdx.x % nqg;
  const int qb = qg * 4 + wave;
  const int h = bh % a.H;
  const size_t base = (size_t)bh * N * d;
  const uint32_t tb = (uint32_t)N * d * 2u;
  const auto rq = make_rsrc(static_cast<const u16*>(a.q) + base, tb);
  const auto rk = make_rsrc(static_cast<const u16*>(a.k) + base, tb);
  const auto rv = make_rsrc(static_cast<const u16*>(a.v) + base, tb);
  const auto rg = make_rsrc(static_cast<const u16*>(a.g) + base, tb);
  const auto ro = make_rsrc(static_cast<u16*>(a.out) + base, tb);
  const auto rb = make_rsrc(a.bias, (uint32_t)a.H * nqb * kLocalWq * kLocalWk * 2u);
  const int key0 = kLocalWq * qb - kLocalOff;
  const int row0 = 128 * qg - kLocalOff;  // key of staged row 0
  auto key_off = [&](int key, int c) -> uint32_t {
    return (key >= 0 && key < N && c < d) ? (uint32_t)(key * d + c) * 2u : kOob;
  };
  const bool qok = qb < nqb;  // a wave past the last block only helps staging

  // this wave's operands: K of tile t (lane (g, r) holds K[slot_of(t, r)][8g .. 8g+7]),
  // Q^T of query tile qt (lane (g, n) holds Q[32qb + 16qt + n][8g .. 8g+7]),
  // bias of query row 16qt + n, slots 32g + 8c .. +7
  u32x4 ak[8], bq[2], bb[2][4];
#pragma unroll
  for (int t = 0; t < 8; ++t) ak[t] = buf_load16(rk, qok ? key_off(key0 + slot_of(t, n), 8 * g) : kOob);
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) bq[qt] = buf_load16(rq, qok ? key_off(32 * qb + 16 * qt + n, 8 * g) : kOob);
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      bb[qt][c] = buf_load16(
          rb, qok ? (uint32_t)(((h * nqb + qb) * kLocalWq + 16 * qt + n) * kLocalWk + 32 * g + 8 * c) * 2u : kOob);
  // the shared V window and the usable flags of its keys
  u32x4 vv[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it, row = c >> 2, c8 = c & 3;
    vv[it] = buf_load16(rv, row < kFwdRows ? key_off(row0 + row, 8 * c8) : kOob);
  }
  if (tid < kFwdRows) {
    const int key = row0 + tid;
    bool ok = key >= 0 && key < N;
    if (a.mask != nullptr && ok) ok = a.mask[key] != 0;
    sKeep[tid] = ok ? 1 : 0;
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it, row = c >> 2, c8 = c & 3;
    if (row < kFwdRows) *reinterpret_cast<u32x4*>(sV + row * kRS + 8 * c8) = vv[it];
  }
  __syncthreads();
  if (!qok) return;  // after the only barrier
  const u16* const mv = sV + 32 * wave * kRS;
  const uint8_t* const mkeep = sKeep + 32 * wave;
  // byte (4t + j) of this lane group's 32 flags: slot 32g + 4t + j
  const u32x4 kf0 = *reinterpret_cast<const u32x4*>(mkeep + 32 * g);
  const u32x4 kf1 = *reinterpret_cast<const u32x4*>(mkeep + 32 * g + 16);

  const float c1 = a.scale * kLog2e;
  float m[2], l[2];
  f32x4 s[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const f32x4 acc = mfma32(as_bf8(ak[t]), as_bf8(bq[qt]), f32x4{0.f, 0.f, 0.f, 0.f});
      const uint32_t fl = t < 4 ? kf0[t] : kf1[t - 4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = bb[qt][t >> 1][(4 * (t & 1) + j) >> 1];
        const float bv = (j & 1) ? bf_hi(w) : bf_lo(w);
        const float x = ((fl >> (8 * j)) & 0xFFu) ? fmaf(acc[j], c1, bv * kLog2e) : kNegInf;
        s[qt][t][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    m[qt] = max_over_groups(mx);
    const float ms = m[qt] == kNegInf ? 0.f : m[qt];
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[qt][t][j] = exp2_fast(s[qt][t][j] - ms);
        sum += s[qt][t][j];
      }
    l[qt] = sum_over_groups(sum);
  }
  // O^T = V^T P^T: k-step j covers slots 32g + 8j .. +7 (tiles 2j, 2j+1)
  f32x4 o[2][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) o[ct][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const bf16x8 av = tr_frag<kRS>(mv, 32 * g + 8 * j, 32 * g + 8 * j + 4, 16 * ct, lane);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) o[ct][qt] = mfma32(av, pack8(s[qt][2 * j], s[qt][2 * j + 1]), o[ct][qt]);
    }
  }
  // epilogue: lane (g, n) holds channels 16ct + 4g .. +3 of query 32qb + 16qt + n
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int query = 32 * qb + 16 * qt + n;
    const float inv = l[qt] > 0.f ? 1.0f / l[qt] : 0.f;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint32_t off = key_off(query, 16 * ct + 4 * g);
      const u32x2 gw = buf_load8(rg, off);
      const float gv[4] = {bf_lo(gw[0]), bf_hi(gw[0]), bf_lo(gw[1]), bf_hi(gw[1])};
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = sigmoidf_fast(gv[r]) * o[ct][qt][r] * inv;
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])}, ro, off, 0, 0);
    }
    if (g == 0 && query < N)
      a.lse[(size_t)bh * N + query] = m[qt] == kNegInf ? kNegInf : (m[qt] + __log2f(l[qt])) * kLn2;
  }
}

// ------------------------------------------------------------------ backward, dQ and dbias partials
// A workgroup takes query blocks 2p, 2p+1 of one (head, batch chunk); wave w
// owns block 2p + w/2, query tile w%2.  Per batch row the four waves stage
// one shared K window: keys 64p - 48 .. 64p + 111 (160 rows), block 2p + u
// starting at row 32u.
constexpr int kDqRows = 160;

constexpr size_t kDqLds = kDqRows * kRS * 2 + kDqRows;

__device__ __forceinline__ void local_dq_role(const LocalArgs& a, const int blk, char* const lds) {
  u16* const sK = reinterpret_cast<u16*>(lds);
  uint8_t* const sKeep = reinterpret_cast<uint8_t*>(lds + kDqRows * kRS * 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const int N = a.N, d = a.d, nqb = a.nqb, H = a.H;
  const int npair = (nqb + 1) / 2;
  const int p = blk % npair;
  const int h = (blk / npair) % H;
  const int chunk = blk / (npair * H);
  const int qt = wave & 1;
  const int qb = 2 * p + (wave >> 1);
  const bool qok = qb < nqb;  // a wave past the last block only helps staging
  const int b0 = chunk * a.C, b1 = std::min(a.B, b0 + a.C);
  const int row0 = 64 * p - kLocalOff;  // key of staged row 0
  const int key0 = kLocalWq * qb - kLocalOff;
  const int query = 32 * qb + 16 * qt + n;
  const bool qvalid = qok && query < N;
  const uint32_t tb = (uint32_t)N * d * 2u;
  auto key_off = [&](int key, int c) -> uint32_t {
    return (key >= 0 && key < N && c < d) ? (uint32_t)(key * d + c) * 2u : kOob;
  };
  const auto rb = make_rsrc(a.bias, (uint32_t)H * nqb * kLocalWq * kLocalWk * 2u);
  u32x4 bb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    bb[c] = buf_load16(
        rb, qok ? (uint32_t)(((h * nqb + qb) * kLocalWq + 16 * qt + n) * kLocalWk + 32 * g + 8 * c) * 2u : kOob);
  if (tid < kDqRows) {
    const int key = row0 + tid;
    bool ok = key >= 0 && key < N;
    if (a.mask != nullptr && ok) ok = a.mask[key] != 0;
    sKeep[tid] = ok ? 1 : 0;
  }
  __syncthreads();
  const int wr = 32 * (wave >> 1);  // this wave's first window row
  const u32x4 kf0 = *reinterpret_cast<const u32x4*>(&sKeep[wr + 32 * g]);
  const u32x4 kf1 = *reinterpret_cast<const u32x4*>(&sKeep[wr + 32 * g + 16]);
  // log2(e) * bias, -inf where the slot is unusable or the row does not exist
  float b2[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t fl = t < 4 ? kf0[t] : kf1[t - 4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t wv = bb[t >> 1][(4 * (t & 1) + j) >> 1];
      const float bv = (j & 1) ? bf_hi(wv) : bf_lo(wv);
      b2[t][j] = (qvalid && ((fl >> (8 * j)) & 0xFFu)) ? bv * kLog2e : kNegInf;
    }
  }
  const float c1 = a.scale * kLog2e;
  float dacc[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) dacc[t][j] = 0.f;
  const u16* const mk = sK + wr * kRS;

  for (int b = b0; b < b1; ++b) {
    const size_t bh = (size_t)b * H + h;
    const size_t base = bh * N * d;
    const auto rq = make_rsrc(static_cast<const u16*>(a.q) + base, tb);
    const auto rk = make_rsrc(static_cast<const u16*>(a.k) + base, tb);
    const auto rv = make_rsrc(static_cast<const u16*>(a.v) + base, tb);
    const auto rda = make_rsrc(static_cast<const u16*>(a.da) + base, tb);
    const auto rdq = make_rsrc(static_cast<u16*>(a.dq) + base, tb);
    u32x4 kv[3], av[8];
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int c = tid + 256 * it, row = c >> 2, c8 = c & 3;
      kv[it] = buf_load16(rk, row < kDqRows ? key_off(row0 + row, 8 * c8) : kOob);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) av[t] = buf_load16(rv, qok ? key_off(key0 + slot_of(t, n), 8 * g) : kOob);
    const u32x4 bq = buf_load16(rq, qok ? key_off(query, 8 * g) : kOob);
    const u32x4 bda = buf_load16(rda, qok ? key_off(query, 8 * g) : kOob);
    const float2 sd = qvalid ? a.seed[bh * N + query] : make_float2(kNegInf, 0.f);
    // the shared K window: operand rows for S^T and transposed reads for dQ
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int c = tid + 256 * it, row = c >> 2, c8 = c & 3;
      if (row < kDqRows) *reinterpret_cast<u32x4*>(sK + row * kRS + 8 * c8) = kv[it];
    }
    __syncthreads();
    if (qok) {  // wave-uniform
      f32x4 ds[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 akt = *reinterpret_cast<const u32x4*>(mk + slot_of(t, n) * kRS + 8 * g);
        const f32x4 st = mfma32(as_bf8(akt), as_bf8(bq), f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 dp = mfma32(as_bf8(av[t]), as_bf8(bda), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pr = exp2_fast(fmaf(st[j], c1, b2[t][j]) + sd.x);
          ds[t][j] = pr * (dp[j] + sd.y);
          dacc[t][j] += ds[t][j];
        }
      }
      // dQ^T = K^T dS^T over the slots, k-step j = slots 32g + 8j .. +7
      f32x4 dq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 bds = pack8(ds[2 * j], ds[2 * j + 1]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          dq[ct] = mfma32(tr_frag<kRS>(mk, 32 * g + 8 * j, 32 * g + 8 * j + 4, 16 * ct, lane), bds, dq[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const f32x4 y = dq[ct] * a.scale;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])}, rdq,
                                              key_off(query, 16 * ct + 4 * g), 0, 0);
      }
    }
    __syncthreads();  // the window is restaged for the next batch row
  }
  if (!qok) return;
  // partial of this chunk: row 16qt + n, slots 32g + 8c .. +7
  float* const part = a.partial + (((size_t)chunk * H + h) * nqb + qb) * kLocalWq * kLocalWk +
                      (size_t)(16 * qt + n) * kLocalWk + 32 * g;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f32x4 v0, v1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v0[e] = dacc[2 * c][e];
      v1[e] = dacc[2 * c + 1][e];
    }
    *reinterpret_cast<f32x4*>(part + 8 * c) = v0;
    *reinterpret_cast<f32x4*>(part + 8 * c + 4) = v1;
  }
}

// ------------------------------------------------------------------ backward, dK and dV
// Key group kg = key tiles 4kg .. 4kg+3 (64 keys).  Key tile m lies inside the
// windows of query blocks ceil((m-4)/2) .. floor((m+3)/2), so group kg needs
// query blocks 2kg-2 .. 2kg+3.  A workgroup walks a run of consecutive groups
// of one (b, h).  Its LDS holds a ring of 8 query blocks (Q rows, dA rows and
// row seeds; block qb in slot qb mod 8): each step computes one group from the
// six blocks it needs while the two blocks the next group adds, and the next
// group's own K, V and bias operands, are in flight.  The two new blocks then
// go into the two slots that no later group reads.
constexpr int kRing = 8;

constexpr size_t kDkdvLds = 2 * kRing * 32 * kRS * 2 + kRing * 32 * sizeof(float2);

__device__ __forceinline__ void local_dkdv_role(const LocalArgs& a, const int seg, const int blk, char* const lds) {
  u16* const sQ = reinterpret_cast<u16*>(lds);
  u16* const sA = sQ + kRing * 32 * kRS;
  float2* const sSeed = reinterpret_cast<float2*>(sA + kRing * 32 * kRS);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const int N = a.N, d = a.d, nqb = a.nqb, H = a.H;
  const int nkt = (N + 15) / 16;
  const int nkg = (nkt + 3) / 4;
  const int nseg = (nkg + seg - 1) / seg;
  const int bh = blk / nseg;
  const int kg0 = (blk % nseg) * seg;
  const int kg1 = std::min(nkg, kg0 + seg);
  const int h = bh % H;
  const size_t base = (size_t)bh * N * d;
  const uint32_t tb = (uint32_t)N * d * 2u;
  const auto rq = make_rsrc(static_cast<const u16*>(a.q) + base, tb);
  const auto rk = make_rsrc(static_cast<const u16*>(a.k) + base, tb);
  const auto rv = make_rsrc(static_cast<const u16*>(a.v) + base, tb);
  const auto rda = make_rsrc(static_cast<const u16*>(a.da) + base, tb);
  const auto rdk = make_rsrc(static_cast<u16*>(a.dk) + base, tb);
  const auto rdv = make_rsrc(static_cast<u16*>(a.dv) + base, tb);
  const auto rb = make_rsrc(a.bias, (uint32_t)H * nqb * kLocalWq * kLocalWk * 2u);
  auto row_off = [&](int row, int c) -> uint32_t {
    return (row >= 0 && row < N && c < d) ? (uint32_t)(row * d + c) * 2u : kOob;
  };
  const float c1 = a.scale * kLog2e;
  const bf16x8 id_hi = ident_cols_frag(lane, kLog2eHiBf16, 0);
  const bf16x8 id_lo = ident_cols_frag(lane, kLog2eLoBf16, 0);

  // one query block = 32 rows x 4 chunks of Q (waves 0-1) and of dA (waves 2-3):
  // one 16-byte chunk per thread, and the block's 32 seeds
  const int srow = (tid & 127) >> 2, sc8 = tid & 3;
  auto stage_load = [&](int qb, u32x4& r, float2& sd) {
    const int row = 32 * qb + srow;
    r = buf_load16((wave >> 1) ? rda : rq, row_off(row, 8 * sc8));
    const int srow2 = 32 * qb + tid;
    sd = (tid < 32 && srow2 >= 0 && srow2 < N) ? a.seed[(size_t)bh * N + srow2] : make_float2(kNegInf, 0.f);
  };
  auto stage_store = [&](int qb, const u32x4& r, const float2& sd) {
    const int slot = qb & (kRing - 1);
    u16* const dst = (wave >> 1) ? sA : sQ;
    *reinterpret_cast<u32x4*>(dst + (slot * 32 + srow) * kRS + 8 * sc8) = r;
    if (tid < 32) sSeed[slot * 32 + tid] = sd;
  };
  // this wave's operands for key tile m: K^T and V^T rows (lane (g, n) holds key
  // 16m + n, channels 8g .. 8g+7) and the bias tiles of its four query blocks
  // (rows 16qt + i, slots s0 + 8(g & 1) .. +7; lane groups 2-3 repeat them)
  struct Ops {
    u32x4 k, v, b[4][2];
  };
  auto ops_load = [&](int m, Ops& o) {
    const int key = 16 * m + n;
    o.k = buf_load16(rk, row_off(key, 8 * g));
    o.v = buf_load16(rv, row_off(key, 8 * g));
    const int qlo = std::max(0, (m - 3) / 2);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int qb = qlo + u;
      const int s0 = 16 * m - 32 * qb + kLocalOff;
      const bool ok = qb < nqb && s0 >= 0 && s0 + 16 <= kLocalWk;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        o.b[u][qt] = buf_load16(
            rb, ok ? (uint32_t)(((h * nqb + qb) * kLocalWq + 16 * qt + n) * kLocalWk + s0 + 8 * (g & 1)) * 2u : kOob);
    }
  };

  // prologue: the six blocks of the first group, and its operands
  Ops cur;
  ops_load(4 * kg0 + wave, cur);
  {
    u32x4 r[6];
    float2 sd[6];
#pragma unroll
    for (int u = 0; u < 6; ++u) stage_load(2 * kg0 - 2 + u, r[u], sd[u]);
#pragma unroll
    for (int u = 0; u < 6; ++u) stage_store(2 * kg0 - 2 + u, r[u], sd[u]);
  }
  __syncthreads();

  for (int kg = kg0; kg < kg1; ++kg) {
    const bool more = kg + 1 < kg1;
    // next group's two new blocks and operands (past the run: nothing is used)
    u32x4 nr0, nr1;
    float2 nsd0, nsd1;
    Ops nxt;
    stage_load(more ? 2 * kg + 4 : -4, nr0, nsd0);
    stage_load(more ? 2 * kg + 5 : -4, nr1, nsd1);
    ops_load(4 * (kg + 1) + wave, nxt);
    __builtin_amdgcn_sched_barrier(0);

    const int m = 4 * kg + wave;  // this wave's key tile
    if (m < nkt) {                // wave-uniform; the barrier below is reached by every wave
      const int key = 16 * m + n;
      bool kok = key < N;
      if (a.mask != nullptr && kok) kok = a.mask[key] != 0;
      u32x4 bk = cur.k;
#pragma unroll
      for (int e = 0; e < 4; ++e) bk[e] = pack2(bf_lo(bk[e]) * c1, bf_hi(bk[e]) * c1);  // K^T * log2(e)/sqrt(d)
      f32x4 dk[2], dv[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        dk[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        dv[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const int qlo = std::max(0, (m - 3) / 2);
      const int qhi = std::min(nqb - 1, (m + 3) / 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int qb = qlo + u;
        const int s0 = 16 * m - 32 * qb + kLocalOff;  // first slot of this key tile in qb's window
        if (qb > qhi || s0 < 0 || s0 + 16 > kLocalWk) continue;  // wave-uniform
        const int lr = (qb & (kRing - 1)) * 32;                  // ring row of the block's first query
        f32x4 p[2], ds[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const u32x4 aq = *reinterpret_cast<const u32x4*>(sQ + (lr + 16 * qt + n) * kRS + 8 * g);
          const u32x4 ada = *reinterpret_cast<const u32x4*>(sA + (lr + 16 * qt + n) * kRS + 8 * g);
          // S[query][key] in log2 units: (Q K^T) log2(e)/sqrt(d) + log2(e) bias
          f32x4 st = mfma32(as_bf8(aq), as_bf8(bk), f32x4{0.f, 0.f, 0.f, 0.f});
          st = mfma32(as_bf8(cur.b[u][qt]), id_hi, st);
          st = mfma32(as_bf8(cur.b[u][qt]), id_lo, st);
          const f32x4 dp = mfma32(as_bf8(ada), as_bf8(cur.v), f32x4{0.f, 0.f, 0.f, 0.f});
          // lane (g, n) holds queries 16qt + 4g + r of the block
          const f32x4 sA4 = *reinterpret_cast<const f32x4*>(&sSeed[lr + 16 * qt + 4 * g]);
          const f32x4 sB4 = *reinterpret_cast<const f32x4*>(&sSeed[lr + 16 * qt + 4 * g + 2]);
          const float sx[4] = {sA4[0], sA4[2], sB4[0], sB4[2]};
          const float sy[4] = {sA4[1], sA4[3], sB4[1], sB4[3]};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pr = kok ? exp2_fast(st[r] + sx[r]) : 0.f;
            p[qt][r] = pr;
            ds[qt][r] = pr * (dp[r] + sy[r]);
          }
        }
        // dV^T += dA^T P, dK^T += Q^T dS over the block's 32 queries:
        // k slot (g, v) = query 16(v / 4) + 4g + v % 4
        const bf16x8 bp = pack8(p[0], p[1]);
        const bf16x8 bs = pack8(ds[0], ds[1]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          dv[ct] = mfma32(tr_frag<kRS>(sA, lr + 4 * g, lr + 16 + 4 * g, 16 * ct, lane), bp, dv[ct]);
          dk[ct] = mfma32(tr_frag<kRS>(sQ, lr + 4 * g, lr + 16 + 4 * g, 16 * ct, lane), bs, dk[ct]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const uint32_t off = row_off(key, 16 * ct + 4 * g);
        const f32x4 yk = dk[ct] * a.scale;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(yk[0], yk[1]), pack2(yk[2], yk[3])}, rdk, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(dv[ct][0], dv[ct][1]), pack2(dv[ct][2], dv[ct][3])}, rdv,
                                              off, 0, 0);
      }
    }
    // blocks 2kg+4, 2kg+5 go over those of 2kg-4, 2kg-3, which no group from kg on reads
    if (more) {
      stage_store(2 * kg + 4, nr0, nsd0);
      stage_store(2 * kg + 5, nr1, nsd1);
    }
    cur = nxt;
    __syncthreads();
  }
}

// One launch carries both backward roles: the key-stationary runs take the
// first `ndkdv` workgroup slots (they are the longer ones), the
// query-stationary workgroups the rest; the roles share the LDS buffer.
__global__ void __launch_bounds__(256) local_bwd_kernel(LocalArgs a, int seg, int ndkdv) {
  __shared__ __attribute__((aligned(16))) char lds[kDkdvLds > kDqLds ? kDkdvLds : kDqLds];
  if ((int)blockIdx.x < ndkdv)
    local_dkdv_role(a, seg, blockIdx.x, lds);
  else
    local_dq_role(a, blockIdx.x - ndkdv, lds);
}

// ------------------------------------------------------------------ plan + launch
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

LocalPlan plan_local_bwd(int B, int H, int N, int d) {
  LocalPlan pl{};
  const int nqb = (N + kLocalWq - 1) / kLocalWq;
  // enough query-stationary waves to fill the chip (about 16 per CU), at
  // most one chunk per batch row
  const long long per_chunk = (long long)H * nqb * 2;
  int P = (int)std::min<long long>(B, std::max<long long>(1, (4096 + per_chunk - 1) / per_chunk));
  const int C = (B + P - 1) / P;
  P = (B + C - 1) / C;
  pl.P = P;
  pl.C = C;
  size_t off = 0;
  pl.off_da = off;
  off = align256(off + (size_t)B * H * N * d * 2);
  pl.off_seed = off;
  off = align256(off + (size_t)B * H * N * sizeof(float2));
  pl.off_partial = off;
  off = align256(off + (size_t)P * H * nqb * kLocalWq * kLocalWk * 4);
  pl.total = off;
  return pl;
}

hipError_t launch_local_fwd(const LocalArgs& a, hipStream_t stream, KernelTimer* timer) {
  timer_start(timer, stream);
  const unsigned grid = (unsigned)((size_t)a.B * a.H * ((a.nqb + 3) / 4));
  hipLaunchKernelGGL(local_fwd_kernel, dim3(grid), dim3(256), 0, stream, a);
  timer_mark(timer, stream);
  return hipGetLastError();
}

hipError_t launch_local_bwd(const LocalArgs& a, hipStream_t stream, KernelTimer* timer) {
  hipError_t e;
  timer_start(timer, stream);
  // 1. dA, dG and the row seeds: the dense path's preprocess (same layouts)
  {
    BwdArgs pa{};
    pa.g = a.g;
    pa.out = a.out;
    pa.lse = a.lse;
    pa.dout = a.dout;
    pa.dg = a.dg;
    pa.da = a.da;
    pa.seed = a.seed;
    pa.B = a.B;
    pa.H = a.H;
    pa.N = a.N;
    pa.d = a.d;
    if ((e = launch_attn_bwd_pre_bf16(pa, stream)) != hipSuccess) return e;
    timer_mark(timer, stream);
  }
  // 2-3. dK/dV (runs of `seg` key groups per workgroup, about 768 of them:
  // three per CU) and dQ with the dbias partials (one workgroup per batch
  // chunk, head and pair of query blocks), in one launch
  {
    const int nkg = ((a.N + 15) / 16 + 3) / 4;
    const long long bhs = (long long)a.B * a.H;
    const int seg = (int)std::max<long long>(1, (bhs * nkg + 767) / 768);
    const long long ndkdv = bhs * ((nkg + seg - 1) / seg);
    const long long ndq = (long long)a.P * a.H * ((a.nqb + 1) / 2);
    hipLaunchKernelGGL(local_bwd_kernel, dim3((unsigned)(ndkdv + ndq)), dim3(256), 0, stream, a, seg, (int)ndkdv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timer_mark(timer, stream);
  }
  // 4. dbias = sum of the partials in chunk order
  if ((e = launch_partial_sum_bf16(a.partial, a.P, (size_t)a.H * a.nqb * kLocalWq * kLocalWk, a.dbias, stream)) !=
      hipSuccess)
    return e;
  timer_mark(timer, stream);
  return hipSuccess;
}

}  // namespace pba

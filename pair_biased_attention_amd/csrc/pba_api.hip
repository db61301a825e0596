// pba_api.hip - the C ABI declared in include/pba.h: argument validation,
// workspace sizing and dispatch to the gfx950 kernels.  Every check runs on
// the host before anything is enqueued; apart from the *_timed measurement
// entry points (which create HIP events and wait for them), nothing here
// allocates, frees, synchronises or prints.
#include <math.h>

#include <mutex>

#include "pba.h"
#include "pba_kernels.h"

// The workspace of pba_backward_noalloc: one copy per GPU, created with the
// code object on that device.  In host code this name is only a stand-in for
// the symbol; kernels get the device address that hipGetSymbolAddress
// returns for the current device (scratch_for_current_device below).
static __device__ __align__(256) char scratch[PBA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kAbiVersion = 4;
constexpr long long kMaxElems = (1LL << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_dims(long long a, long long b, long long c, int d, int dtype, bool bf16_only) {
  if (dtype != PBA_F32 && dtype != PBA_BF16) return PBA_ERR_UNSUPPORTED;
  if (bf16_only && dtype != PBA_BF16) return PBA_ERR_UNSUPPORTED;
  if (a <= 0 || b <= 0 || c <= 0 || d <= 0) return PBA_ERR_SHAPE;
  if (d % 8 != 0 || d > 64) return PBA_ERR_UNSUPPORTED;
  if (a * b * c * d > kMaxElems) return PBA_ERR_SHAPE;
  return PBA_OK;
}

// attention sizes: tensors [B,H,N,d], bias [H,N,N]
int check_attn_sizes(int B, int H, int N, int d, int dtype) {
  int st = check_dims(B, H, N, d, dtype, false);
  if (st != PBA_OK) return st;
  if ((long long)H * N * N > kMaxElems) return PBA_ERR_SHAPE;
  if ((long long)B * H * ((N + 63) / 64) > 0x7FFFFFFFLL) return PBA_ERR_SHAPE;
  return PBA_OK;
}

// The pair-weighted-average kernels address V, G, out and the [H,N,N]
// planes through 32-bit buffer offsets and use offsets past 2^32 - 16 as
// "outside the tensor": every tensor stays below 2^32 - 128 bytes.
constexpr long long kMaxPwaElems = (1LL << 31) - 64;

int check_pwa_sizes(int S, int N, int H, int d, int dtype) {
  int st = check_dims(S, N, H, d, dtype, true);
  if (st != PBA_OK) return st;
  if ((long long)S * N * H * d > kMaxPwaElems) return PBA_ERR_SHAPE;
  if ((long long)H * N * N > kMaxPwaElems) return PBA_ERR_SHAPE;
  return PBA_OK;
}

// Pair-bias projection: the kernels address z, dz and the [H,N,N] planes
// with 32-bit byte offsets, and a ragged last tile reaches up to 16
// positions past the end.
constexpr long long kMaxProjElems = (1LL << 31) - (1LL << 14);

int check_proj_sizes(int N, int H, int c, int dtype) {
  if (dtype != PBA_BF16) return PBA_ERR_UNSUPPORTED;
  if (N <= 0 || H <= 0 || c <= 0) return PBA_ERR_SHAPE;
  if (H > 16 || (c != 32 && c != 64 && c != 128)) return PBA_ERR_UNSUPPORTED;
  if ((long long)N * N * c > kMaxProjElems || (long long)N * N * H > kMaxProjElems) return PBA_ERR_SHAPE;
  return PBA_OK;
}

// Windowed attention: bf16, d a multiple of 8 up to 32; every (b, h) slice
// is addressed with 32-bit byte offsets.
int check_local_sizes(int B, int H, int N, int d, int dtype) {
  int st = check_dims(B, H, N, d, dtype, true);
  if (st != PBA_OK) return st;
  if (d > 32) return PBA_ERR_UNSUPPORTED;
  const long long nqb = (N + 31) / 32;
  if ((long long)H * nqb * 32 * 128 > kMaxElems / 2) return PBA_ERR_SHAPE;
  return PBA_OK;
}

int all_nonnull(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr) return PBA_ERR_NULL;
  return PBA_OK;
}
int all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned16(p)) return PBA_ERR_ALIGN;
  return PBA_OK;
}

float attn_scale(int d) { return 1.0f / sqrtf((float)d); }

int prep_backward(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                  const void* g, const void* bias, const uint8_t* key_mask, const void* out, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, void* dg, void* dbias, void* workspace,
                  size_t workspace_bytes, pba::BwdArgs& a) {
  int st = check_attn_sizes(B, H, N, d, dtype);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({q, k, v, g, bias, out, lse, dout, dq, dk, dv, dg, dbias})) != PBA_OK) return st;
  if ((st = all_aligned16({q, k, v, g, bias, out, dout, dq, dk, dv, dg, dbias})) != PBA_OK) return st;
  if (!aligned4(lse)) return PBA_ERR_ALIGN;
  const bool bf16 = dtype == PBA_BF16;
  const pba::BwdPlan pl = pba::plan_attn_bwd(B, H, N, d, bf16);
  if (workspace == nullptr || workspace_bytes < pl.total) return PBA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PBA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  a.q = q; a.k = k; a.v = v; a.g = g; a.bias = bias; a.mask = key_mask;
  a.out = out; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbias = dbias;
  a.da = ws + pl.off_da;
  a.drow = bf16 ? nullptr : reinterpret_cast<float*>(ws + pl.off_drow);
  a.seed = bf16 ? reinterpret_cast<float2*>(ws + pl.off_drow) : nullptr;
  a.partial = reinterpret_cast<float*>(ws + pl.off_partial);
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.scale = attn_scale(d);
  a.P = pl.P; a.C = pl.C; a.slab = pl.slab; a.direct = pl.direct;
  return PBA_OK;
}

int prep_proj(int N, int H, int c, int dtype, const void* z, const float* gamma, const float* beta,
              const float* w, float eps, pba::ProjArgs& a) {
  int st = check_proj_sizes(N, H, c, dtype);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({z, gamma, beta, w})) != PBA_OK) return st;
  if ((st = all_aligned16({z, gamma, beta, w})) != PBA_OK) return st;
  if (!(eps > 0.0f) || !isfinite(eps)) return PBA_ERR_SHAPE;
  a.z = z; a.gamma = gamma; a.beta = beta; a.w = w;
  a.N = N; a.H = H; a.c = c; a.eps = eps;
  return PBA_OK;
}

int prep_proj_fwd(int N, int H, int c, int dtype, const void* z, const float* gamma, const float* beta,
                  const float* w, float eps, void* bias, pba::ProjArgs& a) {
  int st = prep_proj(N, H, c, dtype, z, gamma, beta, w, eps, a);
  if (st != PBA_OK) return st;
  if (bias == nullptr) return PBA_ERR_NULL;
  if (!aligned16(bias)) return PBA_ERR_ALIGN;
  a.bias = bias;
  return PBA_OK;
}

int prep_proj_bwd(int N, int H, int c, int dtype, const void* z, const float* gamma, const float* beta,
                  const float* w, float eps, const void* dbias, void* dz, float* dgamma, float* dbeta, float* dw,
                  void* workspace, size_t workspace_bytes, pba::ProjArgs& a) {
  int st = prep_proj(N, H, c, dtype, z, gamma, beta, w, eps, a);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({dbias, dz, dgamma, dbeta, dw})) != PBA_OK) return st;
  if ((st = all_aligned16({dbias, dz, dgamma, dbeta, dw})) != PBA_OK) return st;
  if (workspace == nullptr || workspace_bytes < pba::proj_bwd_workspace_bytes(N, c)) return PBA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PBA_ERR_ALIGN;
  a.dbias = dbias; a.dz = dz; a.dgamma = dgamma; a.dbeta = dbeta; a.dw = dw;
  a.partial = static_cast<float*>(workspace);
  a.nwg = pba::proj_bwd_workgroups(N, c);
  return PBA_OK;
}

int prep_local(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
               const void* g, const void* bias, const uint8_t* key_mask, pba::LocalArgs& a) {
  int st = check_local_sizes(B, H, N, d, dtype);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({q, k, v, g, bias})) != PBA_OK) return st;
  if ((st = all_aligned16({q, k, v, g, bias})) != PBA_OK) return st;
  a.q = q; a.k = k; a.v = v; a.g = g; a.bias = bias; a.mask = key_mask;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.nqb = (N + pba::kLocalWq - 1) / pba::kLocalWq;
  a.scale = attn_scale(d);
  return PBA_OK;
}

int prep_local_fwd(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                   const void* g, const void* bias, const uint8_t* key_mask, void* out, float* lse,
                   pba::LocalArgs& a) {
  int st = prep_local(B, H, N, d, dtype, q, k, v, g, bias, key_mask, a);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({out, lse})) != PBA_OK) return st;
  if (!aligned16(out)) return PBA_ERR_ALIGN;
  if (!aligned4(lse)) return PBA_ERR_ALIGN;
  a.out = out; a.lse = lse;
  return PBA_OK;
}

int prep_local_bwd(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                   const void* g, const void* bias, const uint8_t* key_mask, const void* out, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* dg, void* dbias, void* workspace,
                   size_t workspace_bytes, pba::LocalArgs& a) {
  int st = prep_local(B, H, N, d, dtype, q, k, v, g, bias, key_mask, a);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({out, lse, dout, dq, dk, dv, dg, dbias})) != PBA_OK) return st;
  if ((st = all_aligned16({out, dout, dq, dk, dv, dg, dbias})) != PBA_OK) return st;
  if (!aligned4(lse)) return PBA_ERR_ALIGN;
  const pba::LocalPlan pl = pba::plan_local_bwd(B, H, N, d);
  if (workspace == nullptr || workspace_bytes < pl.total) return PBA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PBA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  a.out = const_cast<void*>(out); a.lse = const_cast<float*>(lse); a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbias = dbias;
  a.da = ws + pl.off_da;
  a.seed = reinterpret_cast<float2*>(ws + pl.off_seed);
  a.partial = reinterpret_cast<float*>(ws + pl.off_partial);
  a.P = pl.P; a.C = pl.C;
  return PBA_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; no allocation.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PBA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PBA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PBA_OK;
}

// Measurement helper: runs `launch` with a kernel timer, waits for the last
// event and reports each kernel's duration in milliseconds.
template <typename F>
int run_timed(F launch, hipStream_t stream, float* kernel_ms, int capacity, int* n_kernels) {
  if (kernel_ms == nullptr || n_kernels == nullptr) return PBA_ERR_NULL;
  pba::KernelTimer t;
  int made = 0;
  int st = PBA_OK;
  for (; made <= pba::KernelTimer::kMax; ++made)
    if (hipEventCreate(&t.ev[made]) != hipSuccess) {
      st = PBA_ERR_HIP;
      break;
    }
  if (st == PBA_OK) {
    const hipError_t e = launch(&t, stream);
    if (e != hipSuccess || !t.ok || hipEventSynchronize(t.ev[t.n]) != hipSuccess) st = PBA_ERR_HIP;
  }
  if (st == PBA_OK) {
    *n_kernels = t.n;
    for (int i = 0; i < t.n && i < capacity; ++i)
      if (hipEventElapsedTime(&kernel_ms[i], t.ev[i], t.ev[i + 1]) != hipSuccess) st = PBA_ERR_HIP;
  }
  for (int i = 0; i < made; ++i) (void)hipEventDestroy(t.ev[i]);
  return st;
}

}  // namespace

extern "C" {

int pba_abi_version(void) { return kAbiVersion; }

const char* pba_status_string(int status) {
  switch (status) {
    case PBA_OK: return "PBA_OK";
    case PBA_ERR_NULL: return "PBA_ERR_NULL: a required pointer is NULL";
    case PBA_ERR_SHAPE: return "PBA_ERR_SHAPE: a size is <= 0 or too large, or eps is not a positive finite value";
    case PBA_ERR_UNSUPPORTED: return "PBA_ERR_UNSUPPORTED: unsupported dtype, head width, head count or channel count";
    case PBA_ERR_ALIGN: return "PBA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case PBA_ERR_WORKSPACE: return "PBA_ERR_WORKSPACE: workspace missing or too small";
    case PBA_ERR_HIP: return "PBA_ERR_HIP: the HIP runtime reported a launch error";
    case PBA_ERR_SCRATCH:
      return "PBA_ERR_SCRATCH: the call needs more workspace than the 128 MiB static scratch area of "
             "pba_backward_noalloc holds";
    default: return "unknown pba status";
  }
}

int pba_forward(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                const void* g, const void* bias, const uint8_t* key_mask, void* out, float* lse,
                void* stream) {
  int st = check_attn_sizes(B, H, N, d, dtype);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({q, k, v, g, bias, out, lse})) != PBA_OK) return st;
  if ((st = all_aligned16({q, k, v, g, bias, out})) != PBA_OK) return st;
  if (!aligned4(lse)) return PBA_ERR_ALIGN;
  pba::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.bias = bias; a.mask = key_mask;
  a.out = out; a.lse = lse;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.scale = attn_scale(d);
  const hipError_t e = pba::launch_attn_fwd(a, dtype == PBA_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

size_t pba_backward_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (check_attn_sizes(B, H, N, d, dtype) != PBA_OK) return 0;
  return pba::plan_attn_bwd(B, H, N, d, dtype == PBA_BF16).total;
}

int pba_backward(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                 const void* g, const void* bias, const uint8_t* key_mask, const void* out,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dg, void* dbias,
                 void* workspace, size_t workspace_bytes, void* stream) {
  pba::BwdArgs a{};
  const int st = prep_backward(B, H, N, d, dtype, q, k, v, g, bias, key_mask, out, lse, dout, dq, dk, dv, dg,
                               dbias, workspace, workspace_bytes, a);
  if (st != PBA_OK) return st;
  const hipError_t e = pba::launch_attn_bwd(a, dtype == PBA_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pba_backward_noalloc(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                         const void* g, const void* bias, const uint8_t* key_mask, const void* out,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dg, void* dbias,
                         void* stream) {
  // every argument check before the first HIP call
  int st = check_attn_sizes(B, H, N, d, dtype);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({q, k, v, g, bias, out, lse, dout, dq, dk, dv, dg, dbias})) != PBA_OK) return st;
  if ((st = all_aligned16({q, k, v, g, bias, out, dout, dq, dk, dv, dg, dbias})) != PBA_OK) return st;
  if (!aligned4(lse)) return PBA_ERR_ALIGN;
  const size_t need = pba::plan_attn_bwd(B, H, N, d, dtype == PBA_BF16).total;
  if (need > PBA_NOALLOC_SCRATCH_BYTES) return PBA_ERR_SCRATCH;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != PBA_OK) return st;
  pba::BwdArgs a{};
  st = prep_backward(B, H, N, d, dtype, q, k, v, g, bias, key_mask, out, lse, dout, dq, dk, dv, dg, dbias, ws,
                     PBA_NOALLOC_SCRATCH_BYTES, a);
  if (st != PBA_OK) return st;
  const hipError_t e = pba::launch_attn_bwd(a, dtype == PBA_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pba_backward_timed(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                       const void* g, const void* bias, const uint8_t* key_mask, const void* out,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dg, void* dbias,
                       void* workspace, size_t workspace_bytes, void* stream, float* kernel_ms, int capacity,
                       int* n_kernels) {
  pba::BwdArgs a{};
  const int st = prep_backward(B, H, N, d, dtype, q, k, v, g, bias, key_mask, out, lse, dout, dq, dk, dv, dg,
                               dbias, workspace, workspace_bytes, a);
  if (st != PBA_OK) return st;
  const bool bf16 = dtype == PBA_BF16;
  return run_timed(
      [&](pba::KernelTimer* t, hipStream_t s) { return pba::launch_attn_bwd(a, bf16, s, t); },
      static_cast<hipStream_t>(stream), kernel_ms, capacity, n_kernels);
}

size_t pair_weighted_avg_workspace_bytes(int S, int N, int H, int d, int dtype) {
  if (check_pwa_sizes(S, N, H, d, dtype) != PBA_OK) return 0;
  return ((size_t)H * N * N * 2 + 255) & ~size_t(255);
}

static int prep_pwa_fwd(int S, int N, int H, int d, int dtype, const void* b, const uint8_t* key_mask,
                        const void* v, const void* g, void* out, float* lse_w, void* workspace,
                        size_t workspace_bytes, pba::PwaArgs& a) {
  int st = check_pwa_sizes(S, N, H, d, dtype);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({b, v, g, out, lse_w})) != PBA_OK) return st;
  if ((st = all_aligned16({b, v, g, out})) != PBA_OK) return st;
  if (!aligned4(lse_w)) return PBA_ERR_ALIGN;
  if (workspace == nullptr || workspace_bytes < pair_weighted_avg_workspace_bytes(S, N, H, d, dtype))
    return PBA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PBA_ERR_ALIGN;
  a.b = b; a.mask = key_mask; a.v = v; a.g = g;
  a.o = out; a.lse_w = lse_w; a.w = workspace;
  a.S = S; a.N = N; a.H = H; a.d = d; a.P = 1;
  return PBA_OK;
}

int pair_weighted_avg(int S, int N, int H, int d, int dtype, const void* b, const uint8_t* key_mask,
                      const void* v, const void* g, void* out, float* lse_w, void* workspace,
                      size_t workspace_bytes, void* stream) {
  pba::PwaArgs a{};
  const int st = prep_pwa_fwd(S, N, H, d, dtype, b, key_mask, v, g, out, lse_w, workspace, workspace_bytes, a);
  if (st != PBA_OK) return st;
  const hipError_t e = pba::launch_pwa_fwd(a, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pair_weighted_avg_timed(int S, int N, int H, int d, int dtype, const void* b, const uint8_t* key_mask,
                            const void* v, const void* g, void* out, float* lse_w, void* workspace,
                            size_t workspace_bytes, void* stream, float* kernel_ms, int capacity, int* n_kernels) {
  pba::PwaArgs a{};
  const int st = prep_pwa_fwd(S, N, H, d, dtype, b, key_mask, v, g, out, lse_w, workspace, workspace_bytes, a);
  if (st != PBA_OK) return st;
  return run_timed([&](pba::KernelTimer* t, hipStream_t s) { return pba::launch_pwa_fwd(a, true, s, t); },
                   static_cast<hipStream_t>(stream), kernel_ms, capacity, n_kernels);
}

size_t pair_weighted_avg_backward_workspace_bytes(int S, int N, int H, int d, int dtype) {
  if (check_pwa_sizes(S, N, H, d, dtype) != PBA_OK) return 0;
  return pba::plan_pwa_bwd(S, N, H, d, true).total;
}

static int prep_pwa_bwd(int S, int N, int H, int d, int dtype, const void* b, const uint8_t* key_mask,
                        const void* v, const void* g, const void* out, const float* lse_w, const void* dout,
                        void* dv, void* dg, void* db, void* workspace, size_t workspace_bytes, pba::PwaArgs& a) {
  int st = check_pwa_sizes(S, N, H, d, dtype);
  if (st != PBA_OK) return st;
  if ((st = all_nonnull({b, v, g, out, lse_w, dout, dv, dg, db})) != PBA_OK) return st;
  if ((st = all_aligned16({b, v, g, out, dout, dv, dg, db})) != PBA_OK) return st;
  if (!aligned4(lse_w)) return PBA_ERR_ALIGN;
  const pba::PwaPlan pl = pba::plan_pwa_bwd(S, N, H, d, true);
  if (workspace == nullptr || workspace_bytes < pl.total) return PBA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PBA_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  a.b = b; a.mask = key_mask; a.v = v; a.g = g; a.out = out; a.lse_w_in = lse_w; a.dout = dout;
  a.dv = dv; a.dg = dg; a.db = db;
  a.w = ws + pl.off_w;
  a.da = ws + pl.off_da;
  a.partial = reinterpret_cast<float*>(ws + pl.off_partial);
  a.S = S; a.N = N; a.H = H; a.d = d; a.P = pl.P;
  return PBA_OK;
}

int pair_weighted_avg_backward(int S, int N, int H, int d, int dtype, const void* b,
                               const uint8_t* key_mask, const void* v, const void* g, const void* out,
                               const float* lse_w, const void* dout, void* dv, void* dg, void* db,
                               void* workspace, size_t workspace_bytes, void* stream) {
  pba::PwaArgs a{};
  const int st = prep_pwa_bwd(S, N, H, d, dtype, b, key_mask, v, g, out, lse_w, dout, dv, dg, db, workspace,
                              workspace_bytes, a);
  if (st != PBA_OK) return st;
  const hipError_t e = pba::launch_pwa_bwd(a, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pair_weighted_avg_backward_timed(int S, int N, int H, int d, int dtype, const void* b,
                                     const uint8_t* key_mask, const void* v, const void* g, const void* out,
                                     const float* lse_w, const void* dout, void* dv, void* dg, void* db,
                                     void* workspace, size_t workspace_bytes, void* stream, float* kernel_ms,
                                     int capacity, int* n_kernels) {
  pba::PwaArgs a{};
  const int st = prep_pwa_bwd(S, N, H, d, dtype, b, key_mask, v, g, out, lse_w, dout, dv, dg, db, workspace,
                              workspace_bytes, a);
  if (st != PBA_OK) return st;
  return run_timed([&](pba::KernelTimer* t, hipStream_t s) { return pba::launch_pwa_bwd(a, true, s, t); },
                   static_cast<hipStream_t>(stream), kernel_ms, capacity, n_kernels);
}

int pba_bias_proj_forward(int N, int H, int c, int dtype, const void* z, const float* gamma, const float* beta,
                          const float* w, float eps, void* bias, void* stream) {
  pba::ProjArgs a{};
  const int st = prep_proj_fwd(N, H, c, dtype, z, gamma, beta, w, eps, bias, a);
  if (st != PBA_OK) return st;
  const hipError_t e = pba::launch_proj_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pba_bias_proj_forward_timed(int N, int H, int c, int dtype, const void* z, const float* gamma,
                                const float* beta, const float* w, float eps, void* bias, void* stream,
                                float* kernel_ms, int capacity, int* n_kernels) {
  pba::ProjArgs a{};
  const int st = prep_proj_fwd(N, H, c, dtype, z, gamma, beta, w, eps, bias, a);
  if (st != PBA_OK) return st;
  return run_timed([&](pba::KernelTimer* t, hipStream_t s) { return pba::launch_proj_fwd(a, s, t); },
                   static_cast<hipStream_t>(stream), kernel_ms, capacity, n_kernels);
}

size_t pba_bias_proj_backward_workspace_bytes(int N, int H, int c, int dtype) {
  if (check_proj_sizes(N, H, c, dtype) != PBA_OK) return 0;
  return pba::proj_bwd_workspace_bytes(N, c);
}

int pba_bias_proj_backward(int N, int H, int c, int dtype, const void* z, const float* gamma, const float* beta,
                           const float* w, float eps, const void* dbias, void* dz, float* dgamma, float* dbeta,
                           float* dw, void* workspace, size_t workspace_bytes, void* stream) {
  pba::ProjArgs a{};
  const int st = prep_proj_bwd(N, H, c, dtype, z, gamma, beta, w, eps, dbias, dz, dgamma, dbeta, dw, workspace,
                               workspace_bytes, a);
  if (st != PBA_OK) return st;
  const hipError_t e = pba::launch_proj_bwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pba_bias_proj_backward_timed(int N, int H, int c, int dtype, const void* z, const float* gamma,
                                 const float* beta, const float* w, float eps, const void* dbias, void* dz,
                                 float* dgamma, float* dbeta, float* dw, void* workspace, size_t workspace_bytes,
                                 void* stream, float* kernel_ms, int capacity, int* n_kernels) {
  pba::ProjArgs a{};
  const int st = prep_proj_bwd(N, H, c, dtype, z, gamma, beta, w, eps, dbias, dz, dgamma, dbeta, dw, workspace,
                               workspace_bytes, a);
  if (st != PBA_OK) return st;
  return run_timed([&](pba::KernelTimer* t, hipStream_t s) { return pba::launch_proj_bwd(a, s, t); },
                   static_cast<hipStream_t>(stream), kernel_ms, capacity, n_kernels);
}

int pba_local_forward(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                      const void* g, const void* bias, const uint8_t* key_mask, void* out, float* lse,
                      void* stream) {
  pba::LocalArgs a{};
  const int st = prep_local_fwd(B, H, N, d, dtype, q, k, v, g, bias, key_mask, out, lse, a);
  if (st != PBA_OK) return st;
  const hipError_t e = pba::launch_local_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pba_local_forward_timed(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                            const void* g, const void* bias, const uint8_t* key_mask, void* out, float* lse,
                            void* stream, float* kernel_ms, int capacity, int* n_kernels) {
  pba::LocalArgs a{};
  const int st = prep_local_fwd(B, H, N, d, dtype, q, k, v, g, bias, key_mask, out, lse, a);
  if (st != PBA_OK) return st;
  return run_timed([&](pba::KernelTimer* t, hipStream_t s) { return pba::launch_local_fwd(a, s, t); },
                   static_cast<hipStream_t>(stream), kernel_ms, capacity, n_kernels);
}

size_t pba_local_backward_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (check_local_sizes(B, H, N, d, dtype) != PBA_OK) return 0;
  return pba::plan_local_bwd(B, H, N, d).total;
}

int pba_local_backward(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                       const void* g, const void* bias, const uint8_t* key_mask, const void* out, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, void* dg, void* dbias, void* workspace,
                       size_t workspace_bytes, void* stream) {
  pba::LocalArgs a{};
  const int st = prep_local_bwd(B, H, N, d, dtype, q, k, v, g, bias, key_mask, out, lse, dout, dq, dk, dv, dg,
                                dbias, workspace, workspace_bytes, a);
  if (st != PBA_OK) return st;
  const hipError_t e = pba::launch_local_bwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pba_local_backward_timed(int B, int H, int N, int d, int dtype, const void* q, const void* k, const void* v,
                             const void* g, const void* bias, const uint8_t* key_mask, const void* out,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dg, void* dbias,
                             void* workspace, size_t workspace_bytes, void* stream, float* kernel_ms, int capacity,
                             int* n_kernels) {
  pba::LocalArgs a{};
  const int st = prep_local_bwd(B, H, N, d, dtype, q, k, v, g, bias, key_mask, out, lse, dout, dq, dk, dv, dg,
                                dbias, workspace, workspace_bytes, a);
  if (st != PBA_OK) return st;
  return run_timed([&](pba::KernelTimer* t, hipStream_t s) { return pba::launch_local_bwd(a, s, t); },
                   static_cast<hipStream_t>(stream), kernel_ms, capacity, n_kernels);
}

}  // extern "C"

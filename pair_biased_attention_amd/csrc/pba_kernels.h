// pba_kernels.h - argument blocks and launchers of the gfx950 kernels
// (host-visible; included by the C-ABI translation unit).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pba {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* bias;
  const uint8_t* mask;
  void* out;
  float* lse;
  int B, H, N, d;
  float scale;
  int nqb;  // query blocks per (b, h), set by the launcher
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* bias;
  const uint8_t* mask;
  const void* out;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* dg;
  void* dbias;
  // workspace views
  void* da;         // dA = dout * sigmoid(G), [B,H,N,d] (bf16 for bf16 inputs, fp32 otherwise)
  float* drow;      // fp32 inputs: D = rowsum(dout * out), [B,H,N]
  float2* seed;     // bf16 inputs: per query row (-log2(e) * LSE, or -inf for a row
                    // without keys; -D), [B,H,N]: the accumulator seeds of S' and dP - D
  float* partial;   // dBias partial sums, [P,H,N,N]
  int B, H, N, d;
  float scale;
  int P;            // number of batch chunks (partials)
  int C;            // batch rows per chunk
  int slab;         // 1: dS sums over the chunk in an LDS slab; 0: one partial per batch row
  int direct;       // 1 (one batch row, no slab): dS is stored into dbias in the output
                    // dtype and no partial or reduction is used
};

struct PwaArgs {
  const void* b;
  const uint8_t* mask;
  const void* v;
  const void* g;
  const void* out;
  const float* lse_w_in;
  const void* dout;
  void* o;          // forward output
  float* lse_w;     // forward lse (written)
  void* dv;
  void* dg;
  void* db;
  void* w;          // workspace: softmax weights, [H,N,N] bf16 or fp32
  void* da;         // workspace: dA [S,N,H,d]
  float* partial;   // workspace: dw partial sums [P,H,N,N]
  int S, N, H, d;
  int P;            // S chunks of the dw reduction
};

// Pair-bias projection bias = Linear(LayerNorm(z)): z, bias, dbias, dz are
// bf16; the LayerNorm and projection parameters and their gradients fp32.
struct ProjArgs {
  const void* z;        // [N, N, c]
  const float* gamma;   // [c]
  const float* beta;    // [c]
  const float* w;       // [H, c]
  void* bias;           // forward output [H, N, N]
  const void* dbias;    // backward input [H, N, N]
  void* dz;             // [N, N, c]
  float* dgamma;        // [c]
  float* dbeta;         // [c]
  float* dw;            // [H, c]
  float* partial;       // workspace: per-workgroup sums, [nwg][16 c + 16]
  int N, H, c;
  float eps;
  int nwg;              // backward workgroups (proj_bwd_workgroups)
};
// Backward: one workgroup per CU at most (its per-workgroup sums are the
// workspace), as many waves as the kernel's registers leave room for.
constexpr int kProjBwdMaxWg = 256;
constexpr int proj_bwd_waves(int c) { return c >= 128 ? 8 : 16; }
int proj_bwd_workgroups(int N, int c);
size_t proj_bwd_workspace_bytes(int N, int c);

// Windowed (sequence-local) attention: query block q (32 queries) attends
// the 128 keys 32q - 48 .. 32q + 79; bias and dbias are [H, nqb, 32, 128].
constexpr int kLocalWq = 32, kLocalWk = 128, kLocalOff = 48;
struct LocalArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* bias;
  const uint8_t* mask;
  void* out;
  float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* dg;
  void* dbias;
  void* da;         // workspace: dA [B,H,N,d] bf16
  float2* seed;     // workspace: (-log2(e) * LSE, -D) per query row [B,H,N]
  float* partial;   // workspace: dbias partial sums [P, H, nqb, 32, 128] fp32
  int B, H, N, d, nqb;
  float scale;
  int P, C;         // backward: batch chunks and batch rows per chunk
};
struct LocalPlan {
  size_t off_da, off_seed, off_partial, total;
  int P, C;
};
LocalPlan plan_local_bwd(int B, int H, int N, int d);

// Workspace plan of the attention backward (byte offsets into one buffer).
struct BwdPlan {
  size_t off_da, off_drow, off_partial, total;
  int P, C, slab, direct;
};
BwdPlan plan_attn_bwd(int B, int H, int N, int d, bool bf16);

struct PwaPlan {
  size_t off_w, off_da, off_partial, total;
  int P;
};
PwaPlan plan_pwa_bwd(int S, int N, int H, int d, bool bf16);

// Optional per-kernel timing for the measurement entry points: a launcher
// given a timer records ev[0] on the stream before its first kernel and
// ev[i] after its i-th kernel.
struct KernelTimer {
  static constexpr int kMax = 8;
  hipEvent_t ev[kMax + 1];
  int n = 0;
  bool ok = true;
};
inline void timer_start(KernelTimer* t, hipStream_t s) {
  if (t && hipEventRecord(t->ev[0], s) != hipSuccess) t->ok = false;
}
inline void timer_mark(KernelTimer* t, hipStream_t s) {
  if (t && t->n < KernelTimer::kMax && hipEventRecord(t->ev[++t->n], s) != hipSuccess) t->ok = false;
}

hipError_t launch_attn_fwd(const FwdArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_attn_bwd(const BwdArgs& a, bool bf16, hipStream_t stream, KernelTimer* timer = nullptr);
hipError_t launch_pwa_fwd(const PwaArgs& a, bool bf16, hipStream_t stream, KernelTimer* timer = nullptr);
hipError_t launch_pwa_bwd(const PwaArgs& a, bool bf16, hipStream_t stream, KernelTimer* timer = nullptr);
hipError_t launch_proj_fwd(const ProjArgs& a, hipStream_t stream, KernelTimer* timer = nullptr);
hipError_t launch_proj_bwd(const ProjArgs& a, hipStream_t stream, KernelTimer* timer = nullptr);
hipError_t launch_local_fwd(const LocalArgs& a, hipStream_t stream, KernelTimer* timer = nullptr);
hipError_t launch_local_bwd(const LocalArgs& a, hipStream_t stream, KernelTimer* timer = nullptr);
hipError_t launch_attn_bwd_pre_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_partial_sum_bf16(const float* partial, int P, size_t count, void* out, hipStream_t stream);

}  // namespace pba

/*
 * pba.h - C ABI of libpba: pair-biased gated attention and MSA pair-weighted
 * averaging on AMD Instinct MI355X (gfx950), forward and backward.
 *
 * What is computed (citations are to the AlphaFold3 open-source
 * implementation page, molayo1419.me "Show HN: AlphaFold3 open-source
 * implementation", mirrored on gittoolsai.com):
 *
 *   Attention, per batch row b and head h (section "Model Efficiency": the
 *   pair bias is projected from the pair representation and added after the
 *   key-query dot product, and it needs a gradient):
 *     L[b,h,i,j] = (Q[b,h,i,:] . K[b,h,j,:]) / sqrt(d) + bias[h,i,j]
 *                  (-inf where key_mask[j] == 0)
 *     P = softmax_j(L),  A = P V,  out = sigmoid(G) * A   (elementwise gate)
 *     lse[b,h,i] = log sum_j exp(L[b,h,i,j])              (natural log)
 *   The backward pass returns dQ, dK, dV, dG and dBias, where dBias is the
 *   gradient of the scaled QK^T product summed over the batch axis: the
 *   forward broadcast of the bias over b becomes a reduction (same section).
 *
 *   Pair-weighted average, per MSA row s and head h (section "MSA Pair
 *   Averaging Efficiency": weights from the pair bias alone, no query-key
 *   term, never materialising the (S, N, N, H, d) intermediate):
 *     w[h,i,j] = softmax_j(b[h,i,j] + mask),  lse_w[h,i] = log sum_j exp(...)
 *     out[s,i,h,:] = sigmoid(G[s,i,h,:]) * sum_j w[h,i,j] V[s,j,h,:]
 *   The backward pass returns dV, dG and db (db is reduced over s).
 *
 *   Pair-bias projection (section "Model Efficiency": the bias each attention
 *   adds is projected from the pair representation z [N, N, c]):
 *     bias[h,i,j] = sum_c w[h,c] * (gamma[c] * LayerNorm(z[i,j,:])[c] + beta[c])
 *   and its backward (dz, dgamma, dbeta, dw given dbias).
 *
 *   Windowed attention (same section, atom attention with memory linear in
 *   the number of atoms): each block of 32 queries attends a window of 128
 *   keys, with a pair bias that exists only inside the windows.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers to contiguous row-major
 *     buffers owned by the caller, 16-byte aligned.  Outputs must not alias
 *     inputs.  The library never allocates, frees or synchronises (except
 *     the *_timed measurement entry points at the end of this header).
 *   - Element type: PBA_F32 (float) or PBA_BF16 (bfloat16 bit patterns,
 *     uint16).  Outputs and gradients use the input type; lse, lse_w and all
 *     workspace partials are float32, and so are the projection's LayerNorm
 *     and weight parameters and their gradients.
 *   - key_mask: [N] uint8 device pointer, 0 = masked key, nonzero = keep;
 *     NULL means every key is kept.  A query with every key masked gets
 *     out = 0, lse = -inf and zero gradients.
 *   - d (head width) must be a multiple of 8 in [8, 64]; sizes must be > 0.
 *   - stream: a hipStream_t (NULL = the default stream).  Work is enqueued
 *     and the call returns; errors in kernels surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated before anything is enqueued; an invalid call
 *     returns a status code and enqueues nothing.  A failed launch returns
 *     PBA_ERR_HIP.  No C++ exception crosses this boundary.
 *   - Results are deterministic: the same inputs give bitwise identical
 *     outputs (no floating-point atomics; fixed-order reductions).
 *   - Calls on different streams that share no output buffers and no
 *     workspace are independent; the library keeps no state.
 */
#ifndef PBA_H
#define PBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PBA_F32 = 0, PBA_BF16 = 1 } pba_dtype;

typedef enum {
  PBA_OK = 0,
  PBA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  PBA_ERR_SHAPE = 2,       /* a size is <= 0 or too large for 32-bit indexing,
                              or a LayerNorm eps that is not finite and > 0   */
  PBA_ERR_UNSUPPORTED = 3, /* unsupported dtype, head width d, head count H
                              or channel count c                              */
  PBA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned               */
  PBA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required         */
  PBA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch     */
  PBA_ERR_SCRATCH = 7      /* pba_backward_noalloc: the call needs more than
                              the static scratch area holds                   */
} pba_status;

/* ABI version; bumped on any change of signature or semantics. */
int pba_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* pba_status_string(int status);

/*
 * Forward attention (AlphaFold3 open-source implementation page, section
 * "Model Efficiency": the pair bias is added after the key-query product).
 *   q, k, v, g : [B, H, N, d]   input type
 *   bias       : [H, N, N]      input type, shared by every b
 *   key_mask   : [N] uint8 or NULL
 *   out        : [B, H, N, d]   input type (written)
 *   lse        : [B, H, N]      float32 (written; needed by pba_backward)
 */
int pba_forward(int B, int H, int N, int d, int dtype,
                const void* q, const void* k, const void* v, const void* g,
                const void* bias, const uint8_t* key_mask,
                void* out, float* lse, void* stream);

/* Bytes of device workspace pba_backward needs for these sizes (0 if invalid). */
size_t pba_backward_workspace_bytes(int B, int H, int N, int d, int dtype);

/*
 * Backward attention (same section: the bias gradient is the gradient of the
 * scaled QK^T product, and the broadcast of the bias over b becomes a
 * reduction).  Inputs as in pba_forward, plus the forward's out and lse and
 * the upstream gradient dout [B, H, N, d].  Writes
 *   dq, dk, dv, dg : [B, H, N, d]  input type
 *   dbias          : [H, N, N]     input type, = sum over b of dS[b]
 * workspace: device buffer of at least pba_backward_workspace_bytes(...)
 * bytes, no initialisation needed; its contents after the call are
 * unspecified.  The P matrix is recomputed from q, k, bias and lse.
 */
int pba_backward(int B, int H, int N, int d, int dtype,
                 const void* q, const void* k, const void* v, const void* g,
                 const void* bias, const uint8_t* key_mask,
                 const void* out, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, void* dg, void* dbias,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace pair_weighted_avg needs (0 if invalid). */
size_t pair_weighted_avg_workspace_bytes(int S, int N, int H, int d, int dtype);

/*
 * Forward pair-weighted average (AlphaFold3 open-source implementation page,
 * section "MSA Pair Averaging Efficiency": weights from the pair bias alone,
 * no query-key term, no scale, without the (S, N, N, H, d) intermediate of the
 * naive form).  bf16 only.
 *   b          : [H, N, N]      input type (pair bias logits)
 *   key_mask   : [N] uint8 or NULL
 *   v, g       : [S, N, H, d]   input type (MSA row, token, head, channel)
 *   out        : [S, N, H, d]   input type (written)
 *   lse_w      : [H, N]         float32 (written; needed by the backward)
 * workspace: at least pair_weighted_avg_workspace_bytes(...) bytes; it holds
 * the [H, N, N] weights between the softmax and the weighted-sum kernels.
 */
int pair_weighted_avg(int S, int N, int H, int d, int dtype,
                      const void* b, const uint8_t* key_mask,
                      const void* v, const void* g,
                      void* out, float* lse_w,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace pair_weighted_avg_backward needs (0 if invalid). */
size_t pair_weighted_avg_backward_workspace_bytes(int S, int N, int H, int d, int dtype);

/*
 * Backward pair-weighted average (bf16 only; same section, with the weights
 * shared by every MSA row, so db is a reduction over s).  Inputs as in
 * pair_weighted_avg, plus the forward's out and lse_w and dout [S, N, H, d].
 * Writes
 *   dv, dg : [S, N, H, d]  input type
 *   db     : [H, N, N]     input type (reduced over the S MSA rows)
 * workspace as for pba_backward.
 */
int pair_weighted_avg_backward(int S, int N, int H, int d, int dtype,
                               const void* b, const uint8_t* key_mask,
                               const void* v, const void* g,
                               const void* out, const float* lse_w, const void* dout,
                               void* dv, void* dg, void* db,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Pair-bias projection bias = Linear(LayerNorm(z)) and its backward (the
 * AlphaFold3 open-source implementation page, section "Model Efficiency":
 * every attention projects its pair bias from the pair representation and
 * that projection needs a gradient; the Protenix page lists LayerNorm among
 * the kernels worth a custom implementation).  Per pair position p = i N + j:
 *   xhat = (z[p,:] - mean) / sqrt(var + eps)   (biased variance over c)
 *   bias[h, p] = sum_c w[h, c] (gamma[c] xhat[c] + beta[c])   (no offset term)
 * Arguments:
 *   z          : [N, N, c]  bf16 (pair representation)
 *   gamma, beta: [c]        float32 (LayerNorm scale and shift)
 *   w          : [H, c]     float32 (projection weight, row h = head h)
 *   eps        : LayerNorm epsilon, finite and > 0
 *   bias       : [H, N, N]  bf16 (written), the layout pba_forward takes
 * Every pointer is 16-byte aligned, as for the other entry points.
 * dtype must be PBA_BF16 (PBA_ERR_UNSUPPORTED otherwise).  Supported sizes:
 * c in {32, 64, 128}, 1 <= H <= 16, N >= 1 and N * N * c below 2^31 - 2^14
 * (PBA_ERR_UNSUPPORTED / PBA_ERR_SHAPE otherwise).  The products run with
 * bf16 operands (xhat and gamma * w) and float32 accumulation.
 */
int pba_bias_proj_forward(int N, int H, int c, int dtype,
                          const void* z, const float* gamma, const float* beta,
                          const float* w, float eps, void* bias, void* stream);

/* Bytes of device workspace pba_bias_proj_backward needs (0 if invalid). */
size_t pba_bias_proj_backward_workspace_bytes(int N, int H, int c, int dtype);

/*
 * Backward of pba_bias_proj_forward given dbias [H, N, N] (bf16, e.g. the
 * dbias of pba_backward).  The LayerNorm statistics are recomputed from z.
 * Writes
 *   dz     : [N, N, c]  bf16
 *   dgamma : [c]        float32   (summed over all N * N positions)
 *   dbeta  : [c]        float32
 *   dw     : [H, c]     float32
 * workspace: at least pba_bias_proj_backward_workspace_bytes(...) bytes
 * (per-workgroup partial sums, no initialisation needed).  The sums over
 * positions are taken in a fixed order, so results are bitwise reproducible.
 */
int pba_bias_proj_backward(int N, int H, int c, int dtype,
                           const void* z, const float* gamma, const float* beta,
                           const float* w, float eps, const void* dbias,
                           void* dz, float* dgamma, float* dbeta, float* dw,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Windowed (sequence-local) pair-biased gated attention, the atom-attention
 * form whose memory grows linearly with the number of atoms (AlphaFold3
 * open-source implementation page, section "Model Efficiency", on the atom
 * attention encoder and decoder).  Query block q = atoms 32q .. 32q+31
 * attends the 128 keys 32q-48 .. 32q+79 (window slot s = key - 32q + 48):
 *   L[b,h,i,s] = Q[b,h,i,:] . K[b,h,32q-48+s,:] / sqrt(d) + bias[h,q,i-32q,s]
 *                (-inf for slots outside [0, N) and for masked keys)
 *   P = softmax_s(L),  out = sigmoid(G) * (P V),  lse = log sum_s exp(L)
 * Arguments as for pba_forward except:
 *   bias   : [H, ceil(N/32), 32, 128] bf16 (head, query block, query in
 *            block, window slot), shared by every b
 * bf16 only; d must be a multiple of 8 up to 32 (PBA_ERR_UNSUPPORTED
 * otherwise).  A query whose window has no usable key gets out = 0,
 * lse = -inf and zero gradients.
 */
int pba_local_forward(int B, int H, int N, int d, int dtype,
                      const void* q, const void* k, const void* v, const void* g,
                      const void* bias, const uint8_t* key_mask,
                      void* out, float* lse, void* stream);

/* Bytes of device workspace pba_local_backward needs (0 if invalid). */
size_t pba_local_backward_workspace_bytes(int B, int H, int N, int d, int dtype);

/*
 * Backward of pba_local_forward.  Inputs as there, plus out, lse and dout
 * [B, H, N, d].  Writes dq, dk, dv, dg [B, H, N, d] and
 *   dbias : [H, ceil(N/32), 32, 128] bf16, summed over b (zero at slots
 *           outside [0, N), at masked keys and at rows past N)
 * workspace: at least pba_local_backward_workspace_bytes(...) bytes (dA, the
 * per-row softmax seeds and per-chunk dbias partials; no initialisation).
 */
int pba_local_backward(int B, int H, int N, int d, int dtype,
                       const void* q, const void* k, const void* v, const void* g,
                       const void* bias, const uint8_t* key_mask,
                       const void* out, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv, void* dg, void* dbias,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement entry points.  Each takes the arguments of the call it names,
 * enqueues exactly the same kernels on `stream`, records a HIP event before
 * the first kernel and after every kernel, waits for the last event and
 * writes each kernel's duration in milliseconds to kernel_ms[0..capacity-1]
 * and the number of kernels to *n_kernels.  Unlike every other entry point
 * they create and destroy HIP events and synchronise; they are meant for
 * benchmarks and profiles, not for production loops.  Kernel order:
 *   pba_backward_timed:                preprocess (dA, dG, row seeds), dK/dV +
 *                                      dBias partials together with dQ (one
 *                                      launch; two, dK/dV then dQ, for PBA_F32
 *                                      and where the dBias slab leaves room
 *                                      for only one workgroup per CU), dBias
 *                                      reduction (an entry of zero duration
 *                                      when B == 1 and no slab is used: the
 *                                      dK/dV tiles then store dBias directly)
 *   pair_weighted_avg_timed:           weight softmax, weighted sum + gate
 *   pair_weighted_avg_backward_timed:  weight softmax (w and w^T), preprocess
 *                                      (dA, dG), dV product together with the
 *                                      dw partials (one launch), db
 *   pba_bias_proj_forward_timed:       LayerNorm + projection (one launch)
 *   pba_bias_proj_backward_timed:      dz with the per-workgroup sums of
 *                                      dbias (x) xhat and dbias, then their
 *                                      reduction into dw, dgamma, dbeta
 *   pba_local_forward_timed:           one launch
 *   pba_local_backward_timed:          preprocess (dA, dG, row seeds), dK/dV
 *                                      together with dQ and the per-chunk
 *                                      dbias partials (one launch), dbias
 *                                      reduction
 * kernel_ms or n_kernels NULL returns PBA_ERR_NULL; a runtime failure returns
 * PBA_ERR_HIP.
 */
int pba_backward_timed(int B, int H, int N, int d, int dtype,
                       const void* q, const void* k, const void* v, const void* g,
                       const void* bias, const uint8_t* key_mask,
                       const void* out, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv, void* dg, void* dbias,
                       void* workspace, size_t workspace_bytes, void* stream,
                       float* kernel_ms, int capacity, int* n_kernels);
int pair_weighted_avg_timed(int S, int N, int H, int d, int dtype,
                            const void* b, const uint8_t* key_mask,
                            const void* v, const void* g,
                            void* out, float* lse_w,
                            void* workspace, size_t workspace_bytes, void* stream,
                            float* kernel_ms, int capacity, int* n_kernels);
int pair_weighted_avg_backward_timed(int S, int N, int H, int d, int dtype,
                                     const void* b, const uint8_t* key_mask,
                                     const void* v, const void* g,
                                     const void* out, const float* lse_w, const void* dout,
                                     void* dv, void* dg, void* db,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     float* kernel_ms, int capacity, int* n_kernels);
int pba_bias_proj_forward_timed(int N, int H, int c, int dtype,
                                const void* z, const float* gamma, const float* beta,
                                const float* w, float eps, void* bias, void* stream,
                                float* kernel_ms, int capacity, int* n_kernels);
int pba_bias_proj_backward_timed(int N, int H, int c, int dtype,
                                 const void* z, const float* gamma, const float* beta,
                                 const float* w, float eps, const void* dbias,
                                 void* dz, float* dgamma, float* dbeta, float* dw,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 float* kernel_ms, int capacity, int* n_kernels);
int pba_local_forward_timed(int B, int H, int N, int d, int dtype,
                            const void* q, const void* k, const void* v, const void* g,
                            const void* bias, const uint8_t* key_mask,
                            void* out, float* lse, void* stream,
                            float* kernel_ms, int capacity, int* n_kernels);
int pba_local_backward_timed(int B, int H, int N, int d, int dtype,
                             const void* q, const void* k, const void* v, const void* g,
                             const void* bias, const uint8_t* key_mask,
                             const void* out, const float* lse, const void* dout,
                             void* dq, void* dk, void* dv, void* dg, void* dbias,
                             void* workspace, size_t workspace_bytes, void* stream,
                             float* kernel_ms, int capacity, int* n_kernels);

/*
 * Backward attention that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code recorded into a HIP graph,
 * tight serving loops, harnesses that forbid allocation.  Arguments, results
 * and kernels are those of pba_backward without the workspace pair.
 *
 * The workspace pba_backward would take lives in one static device array of
 * PBA_NOALLOC_SCRATCH_BYTES bytes (128 MiB), which each GPU the library runs
 * on holds from the library's first use on it until the process ends.  The
 * first call on a device looks that device's copy up once (no allocation);
 * later calls reuse it.  A call for which pba_backward_workspace_bytes(...)
 * exceeds the array returns PBA_ERR_SCRATCH and enqueues nothing (the
 * triangle workload B = N = 384, H = 4, d = 32 needs 63 MiB).  The kernels
 * need no part of the array cleared: every value they read was written by
 * the same call.  All calls on one GPU share the array, so calls that overlap
 * in time on one GPU (two streams, or two host threads) race and give
 * undefined results; calls on different GPUs are independent.
 */
#define PBA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int pba_backward_noalloc(int B, int H, int N, int d, int dtype,
                         const void* q, const void* k, const void* v, const void* g,
                         const void* bias, const uint8_t* key_mask,
                         const void* out, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv, void* dg, void* dbias, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PBA_H */

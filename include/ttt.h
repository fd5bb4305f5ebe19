/*
 * ttt.h -- C ABI of libttt.so, the MI355X (gfx950) TTT (test-time training)
 * sequence layer: the forward of TTT-Linear and TTT-MLP and the backward of
 * TTT-Linear, mini-batch dual form.
 *
 * Pages: [TTT] = news article "大模型最强架构TTT问世！斯坦福UCSD等5年磨一剑，
 * 一夜推翻Transformer" (aharts.cn / itmax.cn).
 *
 * The layer ([TTT] 03 §1, §5, §6, §7, §9).  Per (sequence bi, head h) the
 * hidden state is the weight W of a small model f.  For token t with key,
 * value and query views k_t, v_t, q_t (the caller applies the projections
 * theta_K, theta_V, theta_Q):
 *     W_t = W_{t-1} - eta_t * grad_W |f(k_t; W) - v_t|^2  evaluated at W_{t'}
 *     z_t = f(q_t; W_t)                         (the UPDATED state)
 * where t' is the last token before t's mini-batch of b tokens (mini-batch GD,
 * 03 §6; mini-batch n holds tokens [n*b, (n+1)*b), 0-based).  The library
 * computes this with the dual form of 03 §7, one mini-batch at a time:
 *     E = W K - V,   Z = W Q - 2 E (diag(eta) triu(K^T Q)),
 *     W <- W - 2 E diag(eta) K^T          (K, V, Q: d x b, one column per token)
 * TTT-Linear: f(x) = W x, W square d x d.  TTT-MLP: f(x) = W2 GELU(W1 x),
 * W1 dh x d, W2 d x dh, GELU(x) = x * Phi(x) (exact erf form).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (HIP global memory) allocated by
 *    the caller; the library allocates nothing, keeps no global mutable state,
 *    and is re-entrant.  Nothing is read or written on the host.
 *  - Layouts are row-major and contiguous:
 *      Q, K, V, Z : [B, H, T, d]   (token-major: one row of d per token)
 *      W0, W_final: [B or 1, H, d, d] with z = W q  (row i = output i)
 *  - eta is read as eta[bi*eta_stride_b + h*eta_stride_h + t*eta_stride_t]
 *    (elements, fp32): (0,0,0) = one scalar, (0,1,0) = per head,
 *    (H*T, T, 1) = per token.  Strides must be >= 0.
 *  - The call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Argument errors are detected on the host BEFORE any launch and
 *    nothing is written.  Faults during execution surface at the caller's next
 *    synchronisation.  A call only launches kernels on `stream` (no
 *    allocation, copy, memset or synchronisation), so it can be captured in a
 *    HIP graph and replayed.
 *  - Alignment: Q, K, V, Z, W0, W_final 16-byte aligned; eta 4-byte aligned.
 *  - Outputs (Z, W_final) must not overlap any input, except that W_final may
 *    be exactly W0 when W0 is per sequence (w0_batch_stride == H*d*d): the
 *    in-place state carry used for streaming / resume.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 1

typedef enum {
  TTT_OK = 0,
  TTT_ERR_NULL = 1,        /* a required pointer (or desc) is NULL               */
  TTT_ERR_SHAPE = 2,       /* negative size, b < 1, T % b != 0, size overflow    */
  TTT_ERR_DTYPE = 3,       /* dtype code is not a ttt_dtype                      */
  TTT_ERR_UNSUPPORTED = 4, /* valid request, but no kernel built for it          */
  TTT_ERR_ALIAS = 5,       /* an output overlaps an input in a forbidden way     */
  TTT_ERR_ALIGN = 6,       /* a pointer is not aligned as required               */
  TTT_ERR_HIP = 7,         /* the HIP runtime rejected the launch                */
  TTT_ERR_STRIDE = 8,      /* negative eta stride, or w0 stride not 0 / H*d*d    */
  TTT_ERR_FLAGS = 9,       /* unknown bit set in flags                           */
  TTT_ERR_POS = 10,        /* negative decode position                           */
  TTT_ERR_WORKSPACE = 11,  /* workspace missing, misaligned or too small         */
  TTT_ERR_SCRATCH = 12     /* the call needs more than TTT_NOALLOC_SCRATCH_BYTES  */
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* flags */
#define TTT_FLAG_GENERIC 1u /* force the portable fp32 kernel (testing / cross-check)          */
#define TTT_FLAG_PRIMAL 2u  /* compute token by token (primal form, [TTT] 03 §7's naive form):  */
                            /* the same result, no dual form; d in {16, 32, 64}, any b          */
/* Row blocks of the matrix-core forward (d = 64, b = 16, bf16 inputs).  Rows of
 * W evolve independently ([TTT] 03 §9: row i of the next state and of Z needs
 * only row i of W and column i of V), so one (sequence, head) can be spread
 * over 1, 2 or 4 workgroups of 64, 32 or 16 rows (4, 2 or 1 waves).  The
 * default is one workgroup: its waves already run their rows in parallel, one
 * per SIMD, so more workgroups add no parallelism and the per-step latency
 * stays that of one wave (measured on MI355X: 64 sequences x 32,768 tokens
 * 0.916 -> 0.892 ms with 4 blocks; no gain or a loss on the other shapes).
 * A flag sets the count (results are identical: each row goes through the
 * same arithmetic); at most one may be set, not with TTT_FLAG_GENERIC or
 * TTT_FLAG_PRIMAL (TTT_ERR_FLAGS), and a shape the matrix-core kernel does
 * not support then returns TTT_ERR_UNSUPPORTED.                              */
#define TTT_FLAG_ROWS1 4u
#define TTT_FLAG_ROWS2 8u
#define TTT_FLAG_ROWS4 16u

/* TTT-Linear problem description. */
typedef struct {
  int32_t B, H, T, d, b;    /* batch, heads, tokens, head dim, mini-batch size      */
  int32_t in_dtype;         /* ttt_dtype of Q, K, V                                  */
  int32_t out_dtype;        /* ttt_dtype of Z (W_final is always fp32)               */
  uint32_t flags;           /* TTT_FLAG_*                                            */
  int64_t w0_batch_stride;  /* elements between sequences' W0: 0 (shared, [H,d,d])   */
                            /* or H*d*d (per sequence, [B,H,d,d])                     */
  int64_t eta_stride_b, eta_stride_h, eta_stride_t; /* elements, see above          */
} ttt_linear_desc;

/*
 * TTT-Linear forward ([TTT] 03 §7 dual form, 03 §9 f(x) = W x).
 *   Q, K, V : [B,H,T,d] of in_dtype       W0 : fp32, see w0_batch_stride
 *   eta     : fp32, strided as above      Z  : [B,H,T,d] of out_dtype
 *   W_final : [B,H,d,d] fp32, the state after the last token.
 * Supported: d in {16, 32, 64}, fp32 or bf16 inputs, b <= 64 (b <= 32 for
 * d = 64); d = 64, b = 16, bf16 inputs run the MFMA kernel; with
 * TTT_FLAG_PRIMAL any b >= 1.  B*H == 0 or T == 0 is valid (T == 0 copies W0
 * to W_final; Q/K/V/Z may then be NULL).
 */
ttt_status ttt_linear_fwd(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                          const float* W0, const float* eta, void* Z, float* W_final, void* stream);

/*
 * TTT-Linear forward with the sequence split into nchunks chunks processed in
 * parallel: the same result as ttt_linear_fwd (to rounding), for shapes with
 * few (sequence, head) chains and long sequences.  Each mini-batch maps the
 * state affinely (W -> W P_n + R_n, P_n = I - 2 K diag(eta) K^T,
 * R_n = 2 V diag(eta) K^T; [TTT] 03 §7), so a chunk maps it as W -> W P + R.
 * With nb = T / 16 mini-batches, chunk 0 holds about 1.1 / (nchunks - 1 + 1.1)
 * of them (half for nchunks = 2) and the other chunks share the rest evenly.
 * The library
 * (1) runs chunk 0 from W0 and, in the same launch, composes the maps of
 * chunks 1 .. nchunks-2 (the last chunk needs none), (2) scans them to get the
 * start state of every later chunk, (3) runs chunks 1 .. nchunks-1 in
 * parallel from their start states.  Requires the MFMA path (d = 64, b = 16,
 * bf16 inputs; flags 0 or one TTT_FLAG_ROWS*, which applies to pass (3)) and
 * 1 <= nchunks <= T / 16 (else TTT_ERR_SHAPE).  workspace: device memory of at
 * least ttt_linear_chunked_workspace_bytes(desc, nchunks) bytes, 16-byte
 * aligned, overlapping no argument; contents on return are unspecified.
 * nchunks = 1 is ttt_linear_fwd (the workspace may then be NULL).
 */
ttt_status ttt_linear_fwd_chunked(const ttt_linear_desc* desc, int32_t nchunks, const void* Q, const void* K,
                                  const void* V, const float* W0, const float* eta, void* Z, float* W_final,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes ttt_linear_fwd_chunked needs (0 for nchunks = 1; -1 if desc is NULL or nchunks < 1). */
int64_t ttt_linear_chunked_workspace_bytes(const ttt_linear_desc* desc, int32_t nchunks);

/*
 * ttt_linear_fwd_chunked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The chunk maps and start states go to a
 * static device array of TTT_NOALLOC_SCRATCH_BYTES inside the library: one
 * copy per GPU, taken when the library's code is first loaded on that GPU and
 * held until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); on its first call on a GPU it looks
 * up that GPU's copy (hipGetSymbolAddress, the GPU that owns `stream`).
 * Arguments, results and errors as ttt_linear_fwd_chunked, except:
 *   - a call whose ttt_linear_chunked_workspace_bytes exceeds
 *     TTT_NOALLOC_SCRATCH_BYTES returns TTT_ERR_SCRATCH before any launch;
 *   - every call on one GPU shares that GPU's scratch, so calls that may run
 *     at the same time on one GPU (different streams, or graphs replayed
 *     concurrently) race and give wrong results: order them on one stream.
 * A failed symbol lookup returns TTT_ERR_HIP.  This entry point keeps global
 * state (the scratch and the per-GPU addresses), unlike the others.
 */
#define TTT_NOALLOC_SCRATCH_BYTES (32ll * 1024 * 1024)
ttt_status ttt_linear_fwd_chunked_noalloc(const ttt_linear_desc* desc, int32_t nchunks, const void* Q,
                                          const void* K, const void* V, const float* W0, const float* eta,
                                          void* Z, float* W_final, void* stream);

/*
 * TTT-Linear with layer norm and residual inside f ([TTT] 03 §9: the layer's
 * f carries a layer norm and a residual connection around W x, for stability):
 *     f(x) = x + LN(W x),  LN(y) = gamma * (y - mean(y)) / sqrt(var(y) + eps) + beta
 * over the d outputs (var = mean of squared deviations), gamma and beta fp32
 * [H, d] per head.  The gradient of |f(k) - v|^2 stays rank one per token,
 * delta k^T with delta the loss gradient back-propagated through LN to W k, so
 * the dual form carries over: Y = W Q - Delta (diag(eta) triu(K^T Q)),
 * Z = Q + LN(Y), W <- W - Delta diag(eta) K^T.  Other arguments, layouts and
 * errors as for ttt_linear_fwd (Z fp32 or bf16).  Supported: flags = 0, the
 * dual form, at d = 64, b = 16, bf16 inputs; flags = TTT_FLAG_PRIMAL, token by
 * token ([TTT] 03 §7), at d in {16, 32, 64}, any b, fp32 or bf16 inputs;
 * anything else TTT_ERR_UNSUPPORTED.  In addition eps must be finite and >= 0
 * (TTT_ERR_SHAPE), gamma and beta non-NULL (TTT_ERR_NULL), 4-byte aligned
 * (TTT_ERR_ALIGN) and not overlapping Z or W_final (TTT_ERR_ALIAS).
 */
ttt_status ttt_linear_ln_fwd(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                             const float* W0, const float* gamma, const float* beta, float eps, const float* eta,
                             void* Z, float* W_final, void* stream);

/* Name of the kernel ttt_linear_ln_fwd would launch for desc, or NULL if unsupported. */
const char* ttt_linear_ln_kernel_name(const ttt_linear_desc* desc);

/*
 * TTT-Linear with layer norm, forward for training: ttt_linear_ln_fwd, and also
 *   G_saved : [B,H,T,d] fp32, g_t = -eta_t delta_t, the update factor of
 *             token t exactly as the forward applied it to the state
 *             (W <- W + sum_t g_t k_t^T over each mini-batch), with delta_t
 *             the gradient of |f(k_t) - v_t|^2 with respect to y_t = W k_t at
 *             the mini-batch-start W.  With it and W_final, ttt_linear_ln_bwd
 *             undoes the forward's own steps.  Must overlap no other argument
 *             (TTT_ERR_ALIAS); 16-byte aligned (TTT_ERR_ALIGN); non-NULL when
 *             B*H*T > 0 (TTT_ERR_NULL).
 * Same support and other errors as ttt_linear_ln_fwd with flags = 0 (any
 * other flags: TTT_ERR_UNSUPPORTED); Z and W_final are bit-identical to those
 * of ttt_linear_ln_fwd.
 */
ttt_status ttt_linear_ln_fwd_save(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                  const float* W0, const float* gamma, const float* beta, float eps,
                                  const float* eta, void* Z, float* W_final, float* G_saved, void* stream);

/*
 * TTT-Linear with layer norm, backward ([TTT] 03 §4: the layer is trained end
 * to end; 03 §9: f(x) = x + LN(W x)).  With L any scalar whose gradients with
 * respect to Z and W_final are dZ and dW_final, it returns the gradients of L
 * with respect to every input of ttt_linear_ln_fwd:
 *   in : Q, K, V      [B,H,T,d] bf16 (as given to the forward)
 *        eta          strided as for the forward
 *        gamma, beta  [H,d] fp32, eps (as given to the forward)
 *        W_final      [B,H,d,d] fp32 from ttt_linear_ln_fwd_save
 *        G_saved      [B,H,T,d] fp32 from ttt_linear_ln_fwd_save
 *        dZ           [B,H,T,d] out_dtype
 *        dW_final     [B,H,d,d] fp32, or NULL for zero
 *   out: dQ, dK, dV   [B,H,T,d] out_dtype
 *        deta         [B,H,T] fp32 per token (sum it where tokens share an eta)
 *        dW0          [B,H,d,d] fp32 per sequence (sum over B for a shared W0)
 *        dgamma, dbeta [B,H,d] fp32 per sequence (sum over B for the [H,d] parameters)
 * The mini-batch-start states are rebuilt backward from W_final and G_saved
 * (W = W' - sum_t g_t k_t^T); everything else the backward needs (delta,
 * both layer norms and their statistics) is recomputed from the inputs.
 * Outputs overlap no input and no other output (TTT_ERR_ALIAS).
 * Supported: d = 64, b = 16, bf16 inputs; flags 0 (the matrix-core kernel
 * ttt_linear_ln_bwd_d64b16) or TTT_FLAG_GENERIC (the fp32 kernel
 * ttt_linear_ln_bwd_fp32, the cross-check); anything else TTT_ERR_UNSUPPORTED.
 * eps must be finite and >= 0 (TTT_ERR_SHAPE); other errors as for
 * ttt_linear_bwd.
 */
ttt_status ttt_linear_ln_bwd(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                             const float* eta, const float* gamma, const float* beta, float eps,
                             const float* W_final, const float* G_saved, const void* dZ, const float* dW_final,
                             void* dQ, void* dK, void* dV, float* deta, float* dW0, float* dgamma, float* dbeta,
                             void* stream);

/* Runs every host-side check of ttt_linear_ln_bwd and launches nothing. */
ttt_status ttt_linear_ln_bwd_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                      const float* eta, const float* gamma, const float* beta, float eps,
                                      const float* W_final, const float* G_saved, const void* dZ,
                                      const float* dW_final, const void* dQ, const void* dK, const void* dV,
                                      const float* deta, const float* dW0, const float* dgamma,
                                      const float* dbeta);

/* Name of the kernel ttt_linear_ln_bwd would launch for desc, or NULL if unsupported. */
const char* ttt_linear_ln_bwd_kernel_name(const ttt_linear_desc* desc);

/*
 * TTT-Linear decode ([TTT] 04 §3: generation is sequential and uses the primal
 * form).  Continues B*H sequences by desc->T new tokens (often 1), all at
 * absolute positions pos, pos+1, ..., carrying the state in place:
 *   W  : [B,H,d,d] fp32, the state after the pos tokens seen so far (read, then
 *        overwritten with the state after the new tokens)
 *   Wb : [B,H,d,d] fp32, the state at the start of the current mini-batch (read
 *        and overwritten likewise).  A token at position p with p % b == 0
 *        starts a mini-batch: Wb <- W before its gradient is taken.
 *   Q, K, V, Z : [B,H,T,d]; eta strides index the new tokens (t = 0..T-1).
 * desc->w0_batch_stride and desc->flags must be 0; T need not be a multiple of
 * b.  Decoding T tokens from pos = 0 with W = Wb = W0 gives the same Z and W as
 * ttt_linear_fwd (to rounding).  Supported: d in {16, 32, 64}, fp32/bf16 inputs.
 */
ttt_status ttt_linear_decode(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                             const float* eta, void* Z, float* W, float* Wb, int64_t pos, void* stream);

/*
 * TTT-Linear decode with layer norm and residual inside f ([TTT] 03 §9 and 04
 * §3: generation with the layer's own f(x) = x + LN(W x)).  Per new token t at
 * position p, with Wb the mini-batch-start state:
 *   y = Wb k_t;  delta = the gradient of |k_t + LN(y) - v_t|^2 with respect to y;
 *   W <- W - eta_t delta k_t^T;  z_t = q_t + LN(W q_t)
 * (LN, gamma, beta [H, d] fp32 and eps as for ttt_linear_ln_fwd).  Arguments,
 * state carry, support and errors as ttt_linear_decode, plus the layer-norm
 * checks of ttt_linear_ln_fwd (eps: TTT_ERR_SHAPE; gamma, beta: TTT_ERR_NULL,
 * TTT_ERR_ALIGN, and TTT_ERR_ALIAS when they overlap Z, W or Wb).  Decoding T
 * tokens from pos = 0 with W = Wb = W0 gives the Z and W of ttt_linear_ln_fwd
 * (to rounding).
 */
ttt_status ttt_linear_ln_decode(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                const float* eta, const float* gamma, const float* beta, float eps, void* Z,
                                float* W, float* Wb, int64_t pos, void* stream);

/* Runs every host-side check of ttt_linear_ln_decode and launches nothing. */
ttt_status ttt_linear_ln_decode_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                         const float* eta, const float* gamma, const float* beta, float eps,
                                         const void* Z, const float* W, const float* Wb, int64_t pos);

/*
 * TTT-Linear forward for training: ttt_linear_fwd, and also
 *   E_saved : [B,H,T,d] fp32, e_t = W k_t - v_t with W the state at the start
 *             of t's mini-batch (the reconstruction error the gradient step
 *             uses), which is all ttt_linear_bwd needs besides the inputs and
 *             W_final.  Must overlap no other argument.
 * Same support as ttt_linear_fwd; TTT_FLAG_PRIMAL is rejected (TTT_ERR_FLAGS).
 */
ttt_status ttt_linear_fwd_save(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                               const float* W0, const float* eta, void* Z, float* W_final, float* E_saved,
                               void* stream);

/*
 * TTT-Linear backward ([TTT] 03 §4: the layer is trained end to end, so the
 * gradient flows through the inner gradient steps; 03 §7: the dual form is
 * used for the backward as well).  With L any scalar whose gradients with
 * respect to Z and W_final are dZ and dW_final, it returns the gradients of L
 * with respect to every input of the forward:
 *   in : Q, K     [B,H,T,d] in_dtype (as given to the forward; V is not needed)
 *        eta      strided as for the forward
 *        W_final  [B,H,d,d] fp32 from ttt_linear_fwd_save
 *        E_saved  [B,H,T,d] fp32 from ttt_linear_fwd_save
 *        dZ       [B,H,T,d] out_dtype
 *        dW_final [B,H,d,d] fp32, or NULL for zero
 *   out: dQ, dK, dV [B,H,T,d] out_dtype
 *        deta     [B,H,T] fp32, the gradient for every token's step size (sum
 *                 it over the tokens / sequences that share an eta)
 *        dW0      [B,H,d,d] fp32, per sequence (sum over B for a shared W0)
 * The mini-batch-start states are rebuilt backward from W_final and E_saved
 * (W = W' + 2 E diag(eta) K^T), so nothing else is kept from the forward.
 * Outputs overlap no input and no other output.  flags: 0 or
 * TTT_FLAG_GENERIC; w0_batch_stride is ignored (dW0 is always per sequence).
 * Supported: d = 64, b = 16, bf16 Q/K on the MFMA kernel; the portable fp32
 * kernel for d = 16 (b <= 64), d = 32 (b <= 32), d = 64 (b <= 16).
 */
ttt_status ttt_linear_bwd(const ttt_linear_desc* desc, const void* Q, const void* K, const float* eta,
                          const float* W_final, const float* E_saved, const void* dZ, const float* dW_final,
                          void* dQ, void* dK, void* dV, float* deta, float* dW0, void* stream);

/* Runs every host-side check of ttt_linear_bwd and launches nothing. */
ttt_status ttt_linear_bwd_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const float* eta,
                                   const float* W_final, const float* E_saved, const void* dZ,
                                   const float* dW_final, const void* dQ, const void* dK, const void* dV,
                                   const float* deta, const float* dW0);

/* Name of the kernel ttt_linear_bwd would launch for desc, or NULL if unsupported. */
const char* ttt_linear_bwd_kernel_name(const ttt_linear_desc* desc);

/* Runs every host-side check of ttt_linear_fwd and launches nothing. */
ttt_status ttt_linear_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                               const float* W0, const float* eta, const void* Z, const float* W_final);

/* Runs every host-side check of ttt_linear_decode and launches nothing. */
ttt_status ttt_linear_decode_validate(const ttt_linear_desc* desc, const void* Q, const void* K, const void* V,
                                      const float* eta, const void* Z, const float* W, const float* Wb,
                                      int64_t pos);

/* Name of the kernel ttt_linear_fwd would launch for desc, or NULL if unsupported. */
const char* ttt_linear_kernel_name(const ttt_linear_desc* desc);

/* TTT-MLP problem description ([TTT] 03 §9: two layers, GELU). */
typedef struct {
  int32_t B, H, T, d, dh, b; /* dh = hidden width (4*d on the pages)                */
  int32_t in_dtype, out_dtype;
  uint32_t flags;
  int32_t reserved;          /* must be 0                                            */
  int64_t w_batch_stride;    /* 0 (W1, W2 shared over the batch) or per sequence:   */
                             /* H*dh*d (the same element count for W1 and W2)        */
  int64_t eta_stride_b, eta_stride_h, eta_stride_t;
} ttt_mlp_desc;

/*
 * TTT-MLP forward.  Q, K, V, Z as for TTT-Linear.
 *   W1_0 : [B or 1, H, dh, d] fp32     W2_0 : [B or 1, H, d, dh] fp32
 *   W1_final : [B,H,dh,d] fp32         W2_final : [B,H,d,dh] fp32
 * flags: 0 (the dual form) or TTT_FLAG_PRIMAL (token by token, [TTT] 03 §7's
 * naive form, on ttt_mlp_primal_d64h256: d = 64, dh = 256, any b >= 1, fp32
 * or bf16 inputs and Z; T % b == 0 still required); other bits TTT_ERR_FLAGS.
 * Supported without the flag: d = 64, dh = 256, b = 16, bf16 inputs, fp32 Z
 * (anything else: TTT_ERR_UNSUPPORTED).
 */
ttt_status ttt_mlp_fwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                       const float* W1_0, const float* W2_0, const float* eta, void* Z,
                       float* W1_final, float* W2_final, void* stream);

/*
 * TTT-MLP decode ([TTT] 04 §3: generation is sequential and uses the primal
 * form; Fig 15 compares TTT-MLP generation with TTT-Linear).  Continues B*H
 * sequences by desc->T new tokens (often 1) at absolute positions pos, pos+1,
 * ..., carrying the state in place:
 *   W1, W2   : [B,H,dh,d] and [B,H,d,dh] fp32, the state after the pos tokens
 *              seen so far (read, then overwritten with the state after the
 *              new tokens)
 *   W1b, W2b : the same shapes, the state at the start of the current
 *              mini-batch (read and overwritten likewise).  A token at
 *              position p with p % b == 0 starts a mini-batch: W1b, W2b <- W1, W2
 *              before its gradient is taken.
 *   Q, K, V, Z : [B,H,T,d]; eta strides index the new tokens (t = 0..T-1).
 * Per token: h = W1b k, e = 2 (W2b GELU(h) - v), W2 -= eta e GELU(h)^T,
 * W1 -= eta ((W2b^T e) * GELU'(h)) k^T, z = W2 GELU(W1 q).
 * desc->w_batch_stride, desc->flags and desc->reserved must be 0; T need not
 * be a multiple of b; pos < 0 is TTT_ERR_POS.  Decoding T tokens from pos = 0
 * with W = Wb = W0 gives the same Z and state as ttt_mlp_fwd (to rounding).
 * The five outputs (Z and the four states) overlap no input and each other
 * (TTT_ERR_ALIAS).  Supported: d = 64, dh = 256, any b >= 1, fp32/bf16 inputs
 * and Z.
 */
ttt_status ttt_mlp_decode(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V, const float* eta,
                          void* Z, float* W1, float* W2, float* W1b, float* W2b, int64_t pos, void* stream);

/* Runs every host-side check of ttt_mlp_decode and launches nothing. */
ttt_status ttt_mlp_decode_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                   const float* eta, const void* Z, const float* W1, const float* W2,
                                   const float* W1b, const float* W2b, int64_t pos);

ttt_status ttt_mlp_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                            const float* W1_0, const float* W2_0, const float* eta, const void* Z,
                            const float* W1_final, const float* W2_final);

const char* ttt_mlp_kernel_name(const ttt_mlp_desc* desc);

/*
 * TTT-MLP with layer norm and residual inside f ([TTT] 03 §9, as for
 * ttt_linear_ln_fwd): f(x) = x + LN(W2 GELU(W1 x)), LN over
 * the d outputs with per-head gamma, beta ([H, d] fp32) and eps as for
 * ttt_linear_ln_fwd.  The gradient of |f(k) - v|^2 with respect to the
 * pre-norm output is Delta = J_LN^T (2 (f(k) - v) * gamma), and the dual form
 * carries over with Delta in place of 2 (W2 GELU(W1 k) - v):
 * Z = Q + LN(W2 A_Q - Delta (diag(eta) triu(A_K^T A_Q))), both layers updated
 * from Delta as in ttt_mlp_fwd.  Other arguments, support and errors as for
 * ttt_mlp_fwd (flags 0: the dual form; TTT_FLAG_PRIMAL: token by token, in
 * fp32 throughout); in addition eps must be finite and >= 0 (TTT_ERR_SHAPE),
 * gamma and beta non-NULL (TTT_ERR_NULL), 4-byte aligned (TTT_ERR_ALIGN) and
 * not overlapping Z or the final states (TTT_ERR_ALIAS).
 * Accuracy limit: it depends on gamma and beta.  With gamma = 1, beta = 0
 * the recurrence is well conditioned at the full workload length (std 0.02
 * weights, T = 2048: the dual form's Z within 2.4e-5 of an fp64 reference,
 * the primal form's within 3.4e-6).  With random gamma, beta (e.g.
 * 1 + 0.2 N(0,1), 0.1 N(0,1)) some sequences are chaotic: a 1e-7 relative
 * change of K moves the exact Z by up to 8e-4 at T = 512, and the dual
 * form's Z is then up to 6.5e-3 off on a few of 512 sequences (fp32
 * arithmetic, as in the primal form: up to 2.5e-4).
 */
ttt_status ttt_mlp_ln_fwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                          const float* W1_0, const float* W2_0, const float* gamma, const float* beta,
                          float eps, const float* eta, void* Z, float* W1_final, float* W2_final,
                          void* stream);

/*
 * TTT-MLP backward ([TTT] 03 §4: the layer is trained end to end; 03 §9:
 * f(x) = W2 GELU(W1 x)).  With L any scalar whose gradients with respect to Z,
 * W1_final and W2_final (of ttt_mlp_fwd on the same inputs) are dZ, dW1_final
 * and dW2_final, it returns the gradients of L with respect to every input:
 *   in : Q, K, V [B,H,T,d] in_dtype; W1_0, W2_0 and eta as for ttt_mlp_fwd
 *        (w_batch_stride 0 or H*d*dh); dZ [B,H,T,d] fp32;
 *        dW1_final [B,H,dh,d], dW2_final [B,H,d,dh] fp32, each NULL for zero
 *   out: dQ, dK, dV [B,H,T,d] fp32; deta [B,H,T] fp32 per token (sum it where
 *        tokens share an eta); dW1_0 [B,H,dh,d], dW2_0 [B,H,d,dh] fp32 per
 *        sequence (sum over B for a shared initial state)
 *   workspace: device memory of at least ttt_mlp_bwd_workspace_bytes(desc)
 *        bytes, 16-byte aligned: the state at every mini-batch start, written
 *        by a forward pass inside the call; contents on return unspecified.
 * Two forms, by desc:
 *   - the dual form (03 §7: every mini-batch as b x d x dh matrix products,
 *     on the matrix cores with fp32 operands split into bf16 hi + lo): b = 16,
 *     T a multiple of 16, bf16 inputs, flags 0, and Q, K, V, dZ, dQ, dK, dV
 *     16-byte aligned.  Two launches: the forward kernel writing the
 *     mini-batch-start states, then the mini-batches last to first.
 *   - otherwise, or with flags = TTT_FLAG_PRIMAL, the token loop (the primal
 *     form) differentiated in reverse in fp32; T need not be a multiple of b.
 * One workgroup per (sequence, head) in either.  Outputs and the workspace
 * overlap no input and no other output (TTT_ERR_ALIAS).  flags 0 or
 * TTT_FLAG_PRIMAL (TTT_ERR_FLAGS).  Supported: d = 64, dh = 256,
 * 1 <= b <= 16, out_dtype TTT_F32 (dZ and the gradients fp32); anything else
 * TTT_ERR_UNSUPPORTED.  dQ, dK, W1_0, W2_0, the gradient states and the
 * workspace 16-byte aligned (TTT_ERR_ALIGN / _WORKSPACE).
 */
ttt_status ttt_mlp_bwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V, const float* W1_0,
                       const float* W2_0, const float* eta, const float* dZ, const float* dW1_final,
                       const float* dW2_final, void* workspace, int64_t workspace_bytes, float* dQ, float* dK,
                       float* dV, float* deta, float* dW1_0, float* dW2_0, void* stream);

/* Runs every host-side check of ttt_mlp_bwd and launches nothing. */
ttt_status ttt_mlp_bwd_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                const float* W1_0, const float* W2_0, const float* eta, const float* dZ,
                                const float* dW1_final, const float* dW2_final, const void* workspace,
                                int64_t workspace_bytes, const float* dQ, const float* dK, const float* dV,
                                const float* deta, const float* dW1_0, const float* dW2_0);

/* Bytes of workspace ttt_mlp_bwd needs for desc (B*H*ceil(T/b)*2*d*dh*4), or -1 for an invalid desc. */
int64_t ttt_mlp_bwd_workspace_bytes(const ttt_mlp_desc* desc);

/* Name of the kernel ttt_mlp_bwd would launch for desc (ttt_mlp_bwd_d64h256b16:
 * the dual form, given 16-byte aligned tensors; ttt_mlp_bwd_d64h256: the primal
 * form), or NULL if unsupported. */
const char* ttt_mlp_bwd_kernel_name(const ttt_mlp_desc* desc);

/*
 * Backward of ttt_mlp_ln_fwd ([TTT] 03 §4: the layer is trained end to end;
 * 03 §9: f(x) = x + LN(W2 GELU(W1 x)), the layer norm over the d outputs with
 * per-head gamma, beta and eps).  As ttt_mlp_bwd, with gamma, beta [H, d] fp32
 * and eps the forward's, and two more outputs: dgamma, dbeta [B, H, d] fp32
 * per sequence (sum over B for the shared per-head parameters).
 * The loss gradient pulled back through the layer norm, Delta, takes the place
 * of 2 (W2 GELU(W1 k) - v); the backward differentiates Delta itself through
 * the layer norm (its statistics included), and z = q + LN(...) adds dZ to dQ.
 * Computed in the primal form (the token loop in reverse, fp32, one workgroup
 * per (sequence, head); the same workspace and support as ttt_mlp_bwd's primal
 * form: any b <= 16, ragged T, fp32 or bf16 inputs; flags 0 or
 * TTT_FLAG_PRIMAL).  In addition eps must be finite and >= 0 (TTT_ERR_SHAPE),
 * gamma, beta, dgamma, dbeta non-NULL when B*H > 0 (TTT_ERR_NULL), 4-byte
 * aligned (TTT_ERR_ALIGN), and dgamma, dbeta overlap no input and no other
 * output, nor gamma, beta any output (TTT_ERR_ALIAS).
 * Accuracy: as the forward's, it depends on gamma and beta (see
 * ttt_mlp_ln_fwd): well conditioned with gamma = 1, beta = 0.
 */
ttt_status ttt_mlp_ln_bwd(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                          const float* W1_0, const float* W2_0, const float* gamma, const float* beta, float eps,
                          const float* eta, const float* dZ, const float* dW1_final, const float* dW2_final,
                          void* workspace, int64_t workspace_bytes, float* dQ, float* dK, float* dV, float* deta,
                          float* dW1_0, float* dW2_0, float* dgamma, float* dbeta, void* stream);

/* Runs every host-side check of ttt_mlp_ln_bwd and launches nothing. */
ttt_status ttt_mlp_ln_bwd_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                   const float* W1_0, const float* W2_0, const float* gamma, const float* beta,
                                   float eps, const float* eta, const float* dZ, const float* dW1_final,
                                   const float* dW2_final, const void* workspace, int64_t workspace_bytes,
                                   const float* dQ, const float* dK, const float* dV, const float* deta,
                                   const float* dW1_0, const float* dW2_0, const float* dgamma, const float* dbeta);

/* Name of the kernel ttt_mlp_ln_bwd would launch for desc, or NULL if unsupported. */
const char* ttt_mlp_ln_bwd_kernel_name(const ttt_mlp_desc* desc);

/* Name of the kernel ttt_mlp_ln_fwd would launch for desc, or NULL if unsupported. */
const char* ttt_mlp_ln_kernel_name(const ttt_mlp_desc* desc);

/*
 * TTT-MLP decode with layer norm and residual inside f ([TTT] 03 §9 and 04
 * §3: generation with the layer's own f(x) = x + LN(W2 GELU(W1 x))).  Per new
 * token, with W1b, W2b the mini-batch-start state: y = W2b GELU(W1b k);
 * Delta = the gradient of |k + LN(y) - v|^2 with respect to y; both layers
 * stepped from Delta as in ttt_mlp_decode; z = q + LN(W2 GELU(W1 q)) with the
 * updated state (LN, gamma, beta [H, d] fp32 and eps as for ttt_mlp_ln_fwd).
 * Arguments, state carry, support and errors as ttt_mlp_decode, plus the
 * layer-norm checks of ttt_mlp_ln_fwd (eps: TTT_ERR_SHAPE; gamma, beta:
 * TTT_ERR_NULL, TTT_ERR_ALIGN, and TTT_ERR_ALIAS when they overlap Z or a
 * state).  Decoding T tokens from pos = 0 with W1 = W1b = W1_0, W2 = W2b = W2_0
 * gives the Z and states of ttt_mlp_ln_fwd (to rounding).
 */
ttt_status ttt_mlp_ln_decode(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                             const float* eta, const float* gamma, const float* beta, float eps, void* Z, float* W1,
                             float* W2, float* W1b, float* W2b, int64_t pos, void* stream);

/* Runs every host-side check of ttt_mlp_ln_decode and launches nothing. */
ttt_status ttt_mlp_ln_decode_validate(const ttt_mlp_desc* desc, const void* Q, const void* K, const void* V,
                                      const float* eta, const float* gamma, const float* beta, float eps,
                                      const void* Z, const float* W1, const float* W2, const float* W1b,
                                      const float* W2b, int64_t pos);

/* Human-readable text of a status code (never NULL). */
const char* ttt_status_str(int status);

/* TTT_ABI_VERSION of the built library. */
int ttt_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H_ */

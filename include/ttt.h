/*
 * ttt.h -- C ABI of libttt.so: the chunkwise TTT fast-weight layer and the
 * In-Place TTT W_down chunk update, on AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (cited by page and section):
 *   [MTTT]  "Modular TTT: Rethinking Test-Time Training as Composable Modules",
 *           summary page (paper.rainbus.top): "Prerequisites" (fast weights,
 *           train/query view, chunkwise recurrence, eta_t = 2*Sigmoid(beta_t + b),
 *           scalar and vector decay) and "Method step details" (Algorithm 1's
 *           three passes; chunked dual form O = Q W_start - Tril(Q K_hat^T) dV_hat,
 *           W_end = W_start - K_hat^T dV_hat with K_hat = eta (.) K; chunk 256).
 *   [INPL]  "In-Place Test-Time Training", summary page (shdxiang...pages.dev),
 *           "Core method and technical details": O_[i] = Z_[i] W_down^(i)T, then
 *           W_down^(i+1) = W_down^(i) + eta * V_hat_[i]^T Z_[i].
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates device memory; scratch comes from the caller's workspace.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *     void*; NULL means the default stream).  Outputs are valid after the
 *     caller synchronises that stream.
 *   - Arguments are validated on the host, before any HIP call; a failed check
 *     returns a negative ttt_status and launches nothing.  ttt_last_error()
 *     then describes the failure (thread-local string, valid until the next
 *     call on the same thread).  A launch failure returns TTT_ERR_HIP.  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Tensors are dense and row-major with the shapes given below; the layer's
 *     per-(batch, head) sequences are [B, H, T, d].  Every tensor other than
 *     beta, gamma, dbeta and dgamma, and the workspace and saved context, must
 *     start on a 16-byte boundary (rows are moved in 16-byte pieces); a
 *     misaligned pointer is rejected with TTT_ERR_INVALID_ARG.
 *   - Results are deterministic: no floating-point atomics are used.
 */
#ifndef TTT_H
#define TTT_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define TTT_API __attribute__((visibility("default")))
#else
#define TTT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTT_OK = 0,
  TTT_ERR_INVALID_ARG = -1, /* bad pointer, enum, or size                       */
  TTT_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. d_k > 256)       */
  TTT_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than required  */
  TTT_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed       */
} ttt_status;

/* Element type of q, k, v, o, d_o, dq, dk, dv.  beta, gamma, log_decay, the
 * state W and its gradients are always float32. */
typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* Inner (self-supervised) loss per token, summed over tokens and features:
 * MSE = 1/2 ||f(kW) - v||^2, IP = -<f(kW), v>, L1 = sum |f(kW) - v| (signal
 * sign(f(kW) - v), 0 at a tie; no gradient reaches v through it), RMSE =
 * ||f(kW) - v|| / sqrt(dv) per token (signal e / (sqrt(dv) ||e||); decay NONE or
 * SCALAR).  [MTTT "Experimental results": the loss ablation] */
typedef enum { TTT_LOSS_MSE = 0, TTT_LOSS_IP = 1, TTT_LOSS_L1 = 2, TTT_LOSS_RMSE = 3 } ttt_loss;

/* Single nonlinearity after the fast Linear: v_hat = f(kW), o = f(y).
 * SiLU(z) = z sigmoid(z); GELU(z) = z Phi(z), the exact form with the normal
 * distribution function.  [MTTT "Experimental results": SiLU or GELU]
 * NORM is the Norm primitive in that place: the per-token normalisation
 * N(z) = (z - mean(z)) / sqrt(var(z) + 1e-5) over the dv features (no affine),
 * with its analytic backward [MTTT "Technical novelty"]; decay NONE or SCALAR
 * only, and not in the two-layer net. */
typedef enum { TTT_ACT_NONE = 0, TTT_ACT_SILU = 1, TTT_ACT_GELU = 2, TTT_ACT_NORM = 3 } ttt_act;

/* Decay of the fast weight [MTTT "Prerequisites", weight decay]:
 *   SCALAR: W_{i+1} = gamma_h W_i - K^T diag(eta) G, gamma applied once per chunk;
 *   VECTOR: per token and feature, S_t = diag(a_t) S_{t-1} - eta_t k_t^T g_t,
 *           a_t = exp(log_decay_t); queries read S_t (decayed inside the chunk). */
typedef enum { TTT_DECAY_NONE = 0, TTT_DECAY_SCALAR = 1, TTT_DECAY_VECTOR = 2 } ttt_decay;

/* Problem description of the chunkwise TTT layer.  Supported: 1 <= dk, dv <= 256,
 * 1 <= C <= 256, any T >= 0 (the last chunk may be short), B*H >= 0. */
typedef struct {
  int32_t B, H;   /* batch and heads: B*H independent (b, h) chains            */
  int32_t T;      /* tokens per chain (T % C may be non-zero: short last chunk) */
  int32_t dk, dv; /* key / value width; W is dk x dv per chain                 */
  int32_t C;      /* chunk length (mini-batch of one gradient step), >= 1      */
  int32_t dtype;  /* ttt_dtype                                                  */
  int32_t loss;   /* ttt_loss                                                   */
  int32_t act;    /* ttt_act                                                    */
  int32_t decay;  /* ttt_decay                                                  */
  float lr_bias;  /* b in eta_t = 2 * Sigmoid(beta_t + b)                       */
} ttt_desc;

/* Entry ids for ttt_workspace_size. */
#define TTT_ENTRY_FWD 0
#define TTT_ENTRY_BWD 1

/*
 * ttt_workspace_size -- bytes of device workspace that ttt_chunk_fwd (entry 0)
 * or ttt_chunk_bwd (entry 1) needs for `desc`.  Writes *bytes (0 is possible)
 * and returns TTT_OK, or a negative status for an invalid desc.
 */
TTT_API int ttt_workspace_size(const ttt_desc* desc, int entry, size_t* bytes);

/*
 * ttt_saved_size -- bytes of the optional saved context for `desc` (see the
 * `saved` argument of ttt_chunk_fwd / ttt_chunk_bwd).  0 means the kernels
 * that run `desc` keep none (the arguments are then ignored).  Writes *bytes
 * and returns TTT_OK, or a negative status for an invalid desc.
 */
TTT_API int ttt_saved_size(const ttt_desc* desc, size_t* bytes);

/*
 * ttt_chunk_fwd -- forward of the chunkwise TTT layer  [MTTT Algorithm 1 and
 * its chunked dual form].  For each chain, starting from W_0 = w0 (or 0), for
 * each chunk i of C tokens:
 *   eta = 2 Sigmoid(beta + b); Z = K W_i; G = dL/dZ (loss and act');
 *   O = f(Q~ W_i - Tril(Q~ K~^T) diag(eta) G)      (query view, diagonal included);
 *   W_{i+1} = diag(lambda) W_i - K_bar^T diag(eta) G  (state transition).
 * For NONE/SCALAR decay Q~ = Q, K~ = K_bar = K and lambda = 1 (NONE) or gamma_h
 * (SCALAR).  For
 * VECTOR decay with L = in-chunk inclusive cumsum of log_decay: query t reads key
 * s <= t through e^(L_t - L_s) per feature (Tril(Q~ K~^T) with Q~ = Q (.) e^L,
 * K~ = K (.) e^-L written out), K_bar = K (.) e^(L_last - L), lambda = e^(L_last).
 *
 *   q, k      [B,H,T,dk] dtype          v        [B,H,T,dv] dtype
 *   beta      [B,H,T] f32               gamma    [H] f32 (SCALAR only, else NULL)
 *   log_decay [B,H,T,dk] f32, <= 0 (VECTOR only, else NULL)
 *   w0        [B,H,dk,dv] f32 or NULL (zero initial state)
 *   o         [B,H,T,dv] dtype (written)
 *   w_final   [B,H,dk,dv] f32 or NULL (written: W after the last chunk)
 *   w_ckpt    [B,H,ceil(T/C),dk,dv] f32 or NULL (written: w_ckpt[..,i,..] = W_i,
 *             the state at the start of chunk i; ttt_chunk_bwd needs it)
 *   saved     device buffer of ttt_saved_size(desc) bytes, or NULL.  When given
 *             (and that size is non-zero) the forward also writes intermediates
 *             that ttt_chunk_bwd would otherwise recompute per chunk: the
 *             decay-scaled keys and queries (VECTOR), eta (.) G, and with an act
 *             f'(Y) and Z -- in an opaque layout.
 *   ws, ws_bytes  workspace of at least ttt_workspace_size(desc, TTT_ENTRY_FWD)
 *   VECTOR decay on the bf16 matrix-core kernels splits the decay at 32-token
 *   tiles: every factor between tiles is <= 1, and inside a tile the operands
 *   grow by at most half that tile's own decay, so results stay finite and
 *   within the bf16 tolerance for any decay whose per-feature total over every
 *   32-token tile stays above about e^-150 (a mean per-token a above ~0.01);
 *   beyond that the in-tile operands overflow fp32.  The fp32 path evaluates
 *   e^(L_t - L_s) pairwise and has no such limit.
 */
TTT_API int ttt_chunk_fwd(const ttt_desc* desc, const void* q, const void* k, const void* v,
                  const float* beta, const float* gamma, const float* log_decay,
                  const float* w0, void* o, float* w_final, float* w_ckpt, void* saved,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * ttt_chunk_bwd -- analytic outer backward of ttt_chunk_fwd for the outer loss
 * <d_o, O> + <d_wfinal, W_T>: the reverse chunk sweep carries dW_{i+1} and
 * differentiates each forward step (the hand-written Linear backward that the
 * Modular TTT page credits with its speed-up, "Technical novelty").
 *
 *   q, k, v, beta, gamma, log_decay, w0   as passed to ttt_chunk_fwd
 *   w_ckpt    [B,H,ceil(T/C),dk,dv] f32: the checkpoints ttt_chunk_fwd wrote
 *   saved     NULL (recompute), or the saved context that ttt_chunk_fwd filled
 *             for the same desc and inputs; it is read, not checked
 *   d_o       [B,H,T,dv] dtype          d_wfinal [B,H,dk,dv] f32 or NULL (zero)
 *   dq, dk    [B,H,T,dk] dtype          dv       [B,H,T,dv] dtype
 *   dbeta     [B,H,T] f32
 *   dgamma    [B,H] f32 (SCALAR only, else may be NULL); per chain -- a gamma
 *             shared over the batch has gradient sum_b dgamma[b,h]
 *   dlog_decay [B,H,T,dk] f32 (VECTOR only, else may be NULL)
 *   dw0       [B,H,dk,dv] f32 or NULL
 *   ws, ws_bytes  workspace of at least ttt_workspace_size(desc, TTT_ENTRY_BWD)
 * No gradient is returned for the scalar b (it equals sum(dbeta)).
 */
TTT_API int ttt_chunk_bwd(const ttt_desc* desc, const void* q, const void* k, const void* v,
                  const float* beta, const float* gamma, const float* log_decay,
                  const float* w0, const float* w_ckpt, const void* saved, const void* d_o,
                  const float* d_wfinal, void* dq, void* dk, void* dv, float* dbeta,
                  float* dgamma, float* dlog_decay, float* dw0, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * inplace_ttt_workspace_size -- bytes of the optional workspace of
 * inplace_ttt_fwd for these sizes (0 when the apply step would not use one).
 * Writes *bytes and returns TTT_OK, or TTT_ERR_INVALID_ARG for negative sizes.
 */
TTT_API int inplace_ttt_workspace_size(int B, int T, int d_model, int d_ff, int C, size_t* bytes);

/*
 * inplace_ttt_fwd -- In-Place TTT apply-then-update of the MLP's W_down
 * [INPL "Core method and technical details"].  For each sequence b and each
 * chunk i of C tokens, in order:
 *   O_[i] = Z_[i] W_down^T                     (apply, with the current W_down)
 *   W_down += eta * V_hat_[i]^T Z_[i]          (update, fp32 state)
 *   z     [B,T,d_ff] bf16     (Z = phi(H W_gate^T) (.) (H W_up^T), formed by the caller)
 *   vhat  [B,T,d_model] bf16  (the update target V_hat)
 *   w_down [B,d_model,d_ff] f32, read and updated in place
 *   o     [B,T,d_model] bf16 (written)
 *   ws, ws_bytes  optional device workspace (NULL / 0 allowed): with at least
 *             inplace_ttt_workspace_size bytes the apply step splits its d_ff
 *             contraction over more workgroups and sums fp32 partials there;
 *             without it the apply runs unsplit (same results up to fp32
 *             summation order).
 * The apply step rounds W_down to bf16 as its matrix-core operand; products
 * accumulate in fp32.  T % C may be non-zero.  d_model and d_ff must be
 * multiples of 8 (16-byte rows); pointers 16-byte aligned.
 */
TTT_API int inplace_ttt_fwd(int B, int T, int d_model, int d_ff, int C, float eta, const void* z,
                    const void* vhat, float* w_down, void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * inplace_ttt_guarded_workspace_size -- bytes of the workspace of
 * inplace_ttt_fwd_guarded for these sizes: a small area for the clip norm (one
 * float per 128 x 128 tile of W_down, and the scale) followed by the optional
 * split-K area of inplace_ttt_workspace_size.  Writes *bytes and returns TTT_OK,
 * or TTT_ERR_INVALID_ARG for negative sizes.
 */
TTT_API int inplace_ttt_guarded_workspace_size(int B, int T, int d_model, int d_ff, int C, size_t* bytes);

/*
 * inplace_ttt_fwd_guarded -- inplace_ttt_fwd with the two long-context
 * safeguards of [INPL "Practical advice", the stability item]: a threshold on
 * the Frobenius norm of each update, and a reset of the fast weight at
 * document boundaries.  For each sequence b, each document in it, and each
 * chunk i of C tokens counted from the document's first token:
 *   O_[i] = Z_[i] W_down^T
 *   dW    = eta * V_hat_[i]^T Z_[i];   dW *= min(1, clip_tau / ||dW||_F)
 *   W_down += dW
 * and at the first token of every document but the sequence's first, W_down
 * restarts from w_init (the pretrained weight).
 *   clip_tau    > 0 and finite: clip at this norm (the page uses 1e-5);
 *               0 or +inf: no clipping; negative or NaN: TTT_ERR_INVALID_ARG
 *   doc_starts  HOST array of n_docs int64 positions p = b * T + t, strictly
 *               increasing, each with 0 < t < T: a document begins at token t
 *               of sequence b (every sequence begins one at t = 0).  NULL when
 *               n_docs == 0.
 *   w_init      [B,d_model,d_ff] f32, read only; required when n_docs > 0
 *   w_down      [B,d_model,d_ff] f32: the state at t = 0 on entry, the state
 *               after each sequence's last chunk on return
 *   z, vhat, o  as in inplace_ttt_fwd
 *   ws, ws_bytes  device workspace of at least the clip area of
 *               inplace_ttt_guarded_workspace_size (required when clipping;
 *               the rest of that size enables the split apply)
 * With clip_tau = 0 and n_docs = 0 the results equal inplace_ttt_fwd's.  The
 * norm is formed from the same fp32 products as the update (an extra GEMM of
 * the update's shape per chunk when clipping) and summed in fp64.
 */
TTT_API int inplace_ttt_fwd_guarded(int B, int T, int d_model, int d_ff, int C, float eta, float clip_tau,
                                    const int64_t* doc_starts, int n_docs, const void* z, const void* vhat,
                                    const float* w_init, float* w_down, void* o, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * inplace_ttt_bwd_workspace_size -- bytes of the (required) workspace of
 * inplace_ttt_bwd: the rewound state of one sequence (d_model * d_ff fp32) and
 * fp32 partial sums.  Writes *bytes; TTT_OK or TTT_ERR_INVALID_ARG.
 */
TTT_API int inplace_ttt_bwd_workspace_size(int B, int T, int d_model, int d_ff, int C, size_t* bytes);

/*
 * inplace_ttt_bwd -- reverse-mode derivative of inplace_ttt_fwd, for training
 * the model the fast weight sits in (the W_down backward; [INPL "Core method and
 * technical details"] fixes the forward it differentiates).  Given
 *   d_o       [B,T,d_model] bf16   dL/dO
 *   d_wfinal  [B,d_model,d_ff] f32 dL/dW_final, or NULL for zero
 *   w_final   [B,d_model,d_ff] f32 the state inplace_ttt_fwd left (read only;
 *             the states of earlier chunks are recovered from it chunk by chunk)
 *   z, vhat, eta, C as given to the forward
 * it writes
 *   dz        [B,T,d_ff] bf16      dL/dZ = dO_i W_i + eta V_hat_i dW_{i+1}
 *   dvhat     [B,T,d_model] bf16   dL/dV_hat = eta Z_i dW_{i+1}^T
 *   dw0       [B,d_model,d_ff] f32 dL/dW_0 (dW_i = dW_{i+1} + dO_i^T Z_i down to i = 0)
 * Operands are rounded to bf16 for the matrix cores (W_i and dW_{i+1} too),
 * products accumulate in fp32; the states and dW stay fp32.  Clipping and
 * document resets (inplace_ttt_fwd_guarded) are differentiated by
 * inplace_ttt_bwd_guarded.  ws:
 * at least inplace_ttt_bwd_workspace_size bytes (TTT_ERR_WORKSPACE otherwise);
 * pointers 16-byte aligned.
 */
TTT_API int inplace_ttt_bwd(int B, int T, int d_model, int d_ff, int C, float eta, const void* z, const void* vhat,
                            const float* w_final, const void* d_o, const float* d_wfinal, void* dz, void* dvhat,
                            float* dw0, void* ws, size_t ws_bytes, void* stream);

/*
 * inplace_ttt_bwd_guarded_workspace_size -- bytes of the (required) workspace
 * of inplace_ttt_bwd_guarded: the state and its bf16 copies, the partial
 * products of dZ and dV_hat, the chunk's Gram matrix and a few scalars.
 * Writes *bytes; TTT_OK, TTT_ERR_INVALID_ARG, or TTT_ERR_UNSUPPORTED where
 * min(T, C) > 8192 or the sizes leave the tile path's offset range.
 */
TTT_API int inplace_ttt_bwd_guarded_workspace_size(int B, int T, int d_model, int d_ff, int C, size_t* bytes);

/*
 * inplace_ttt_bwd_guarded -- reverse-mode derivative of inplace_ttt_fwd_guarded
 * (the update clipping and document resets of [INPL "Practical advice", the
 * stability item]), for training with the safeguards on.  Per chunk, with
 * D = eta V_hat_i^T Z_i, n = ||D||_F, s = min(1, clip_tau / n) and
 * A = dL/dW_{i+1}, the adjoint of D is
 *   G = s A - (s <D, A> / n^2) D        (G = A where the update is not clipped)
 * and dZ_i = dO_i W_i + eta V_hat_i G, dV_hat_i = eta Z_i G^T, A += dO_i^T Z_i.
 * A document's final state is discarded at the next document's start, so the
 * adjoint restarts from zero there; at a document's first token it is the
 * derivative with respect to that document's starting state.
 *   clip_tau, doc_starts, n_docs, z, vhat, eta, C  as given to the forward
 *   w0        [B,d_model,d_ff] f32 the state at t = 0 (w_down on entry to the
 *             forward); read only; required when n_docs > 0 (the documents
 *             before the last are replayed from their starting states), else
 *             unused and may be NULL
 *   w_init    [B,d_model,d_ff] f32 as given to the forward; required when n_docs > 0
 *   w_final   [B,d_model,d_ff] f32 the state the forward left (read only)
 *   d_o       [B,T,d_model] bf16   dL/dO
 *   d_wfinal  [B,d_model,d_ff] f32 dL/dW_final, or NULL for zero
 * writes
 *   dz        [B,T,d_ff] bf16      dL/dZ
 *   dvhat     [B,T,d_model] bf16   dL/dV_hat
 *   dw0       [B,d_model,d_ff] f32 dL/dw0 (the first document's starting state)
 *   dw_init   [B,d_model,d_ff] f32 dL/dw_init summed over each sequence's
 *             documents after the first (zero where there are none), or NULL
 *             to skip it
 * The clip decisions recompute the forward's norms from the same products.
 * Operands are rounded to bf16 for the matrix cores, the products accumulate
 * in fp32 and the norms and <D, A> sum in fp64.  With clip_tau = 0 and
 * n_docs = 0 the results equal inplace_ttt_bwd's.  ws: at least
 * inplace_ttt_bwd_guarded_workspace_size bytes (TTT_ERR_WORKSPACE otherwise);
 * pointers 16-byte aligned; TTT_ERR_UNSUPPORTED as for the workspace size.
 */
TTT_API int inplace_ttt_bwd_guarded(int B, int T, int d_model, int d_ff, int C, float eta, float clip_tau,
                                    const int64_t* doc_starts, int n_docs, const void* z, const void* vhat,
                                    const float* w0, const float* w_init, const float* w_final, const void* d_o,
                                    const float* d_wfinal, void* dz, void* dvhat, float* dw0, float* dw_init, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * Two-layer fast net (TTT-MLP): Linear(W1: dk -> dh), the act f, Linear(W2:
 * dh -> dv), no biases -- the deeper fast net of [MTTT "Experimental results"],
 * whose per-chunk computation [MTTT "Method step details", Algorithm 1] composes
 * from the rules of its primitives.  Supported: 1 <= dk, dv <= 256,
 * 1 <= dh <= 1024, 1 <= C <= 256, any T >= 0; decay NONE or SCALAR (a vector
 * decay is not defined for two layers).
 */
typedef struct {
  int32_t B, H, T;
  int32_t dk, dh, dv; /* W1 is dk x dh, W2 is dh x dv per chain            */
  int32_t C;
  int32_t dtype;      /* ttt_dtype of q, k, v, o                          */
  int32_t loss;       /* ttt_loss                                         */
  int32_t act;        /* ttt_act: f between the two Linears               */
  int32_t decay;      /* TTT_DECAY_NONE or TTT_DECAY_SCALAR               */
  float lr_bias;      /* b in eta_t = 2 * Sigmoid(beta_t + b)             */
} ttt_mlp_desc;

/*
 * ttt_mlp_workspace_size -- bytes of the (required) workspace of
 * ttt_mlp_chunk_fwd: per chain, two copies of each weight and the chunk's
 * fp32 intermediates.  Writes *bytes; TTT_OK or a negative status.
 */
TTT_API int ttt_mlp_workspace_size(const ttt_mlp_desc* desc, size_t* bytes);

/*
 * ttt_mlp_chunk_fwd -- forward of the two-layer fast net.  For each chain and
 * each chunk of C tokens, with W1, W2 at the chunk start and
 * eta = 2 Sigmoid(beta + b):
 *   train view:  Z1 = K W1, A = f(Z1), V_hat = A W2;
 *   its signals: G2 = V_hat - V (MSE), -V (IP) or sign(V_hat - V) (L1),
 *                G1 = (G2 W2^T) (.) f'(Z1);
 *   query view:  A_q = f(Q W1 - Tril(Q K^T) diag(eta) G1),
 *                O = A_q W2 - Tril(A_q A^T) diag(eta) G2   (diagonal included);
 *   state:       W1 <- g W1 - K^T diag(eta) G1,  W2 <- g W2 - A^T diag(eta) G2,
 *                g = gamma_h (SCALAR) or 1.
 *   q, k [B,H,T,dk] dtype;  v, o [B,H,T,dv] dtype;  beta [B,H,T] f32;
 *   gamma [H] f32 (SCALAR only);  w1_0 [B,H,dk,dh], w2_0 [B,H,dh,dv] f32 or
 *   NULL (zero);  w1_final, w2_final (same shapes) f32 or NULL (written).
 *   w1_ckpt [B,H,ceil(T/C),dk,dh], w2_ckpt [B,H,ceil(T/C),dh,dv] f32 or NULL
 *   (written: the weights at the start of each chunk; ttt_mlp_chunk_bwd needs them)
 *   saved     device buffer of ttt_mlp_saved_size bytes, or NULL.  When given,
 *             the forward also keeps every chunk's train- and query-view
 *             intermediates (opaque layout) so that ttt_mlp_chunk_bwd does not
 *             recompute them.
 *   ws, ws_bytes  workspace of at least ttt_mlp_workspace_size bytes
 * Arithmetic is fp32 throughout (bf16 inputs are widened, o is rounded once).
 */
TTT_API int ttt_mlp_chunk_fwd(const ttt_mlp_desc* desc, const void* q, const void* k, const void* v,
                              const float* beta, const float* gamma, const float* w1_0, const float* w2_0,
                              void* o, float* w1_final, float* w2_final, float* w1_ckpt, float* w2_ckpt,
                              void* saved, void* ws, size_t ws_bytes, void* stream);

/*
 * ttt_mlp_saved_size -- bytes of the optional saved context of
 * ttt_mlp_chunk_fwd / ttt_mlp_chunk_bwd: per chain and chunk, four C x dh and two
 * C x dv fp32 intermediates, two more C x dh (P, X1) and the two C x C score
 * matrices, and C floats per chunk of the RMSE row scales 1 / (sqrt(dv) ||e||).
 * Writes *bytes; TTT_OK or a negative status.
 */
TTT_API int ttt_mlp_saved_size(const ttt_mlp_desc* desc, size_t* bytes);

/*
 * ttt_mlp_bwd_workspace_size -- bytes of the (required) workspace of
 * ttt_mlp_chunk_bwd: per chain, the carried weight gradients and the chunk's
 * fp32 forward and backward intermediates.  Writes *bytes; TTT_OK or a
 * negative status.
 */
TTT_API int ttt_mlp_bwd_workspace_size(const ttt_mlp_desc* desc, size_t* bytes);

/*
 * ttt_mlp_chunk_bwd -- analytic outer backward of ttt_mlp_chunk_fwd for the
 * outer loss <d_o, O> + <d_w1final, W1_T> + <d_w2final, W2_T>: chunks in
 * reverse, each recomputed from its checkpoints and its steps differentiated
 * in reverse order (the composed three passes of [MTTT Algorithm 1] run
 * backwards).
 *   q, k, v, beta, gamma   as passed to ttt_mlp_chunk_fwd
 *   w1_ckpt, w2_ckpt       the checkpoints ttt_mlp_chunk_fwd wrote
 *   saved     NULL (recompute each chunk's forward), or the saved context that
 *             ttt_mlp_chunk_fwd filled for the same desc and inputs (read, not checked)
 *   d_o [B,H,T,dv] dtype;  d_w1final [B,H,dk,dh], d_w2final [B,H,dh,dv] f32 or NULL
 *   dq, dk [B,H,T,dk] dtype;  dv [B,H,T,dv] dtype;  dbeta [B,H,T] f32
 *   dgamma [B,H] f32 (SCALAR only; per chain);  dw1_0, dw2_0 f32 or NULL
 *   ws, ws_bytes  workspace of at least ttt_mlp_bwd_workspace_size bytes
 * fp32 arithmetic throughout.  No gradient is returned for b (sum(dbeta)).
 */
TTT_API int ttt_mlp_chunk_bwd(const ttt_mlp_desc* desc, const void* q, const void* k, const void* v,
                              const float* beta, const float* gamma, const float* w1_ckpt, const float* w2_ckpt,
                              const void* saved, const void* d_o, const float* d_w1final, const float* d_w2final,
                              void* dq, void* dk,
                              void* dv, float* dbeta, float* dgamma, float* dw1_0, float* dw2_0, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * ttt_chunk_bwd_noalloc -- ttt_chunk_bwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments (less
 * ws and ws_bytes), semantics and results as ttt_chunk_bwd: the same kernels
 * run.  The scratch comes from a fixed device array inside the library of
 * ttt_noalloc_scratch_bytes() bytes (64 MiB) per GPU, held until the process
 * ends.  A problem whose ttt_workspace_size(desc, TTT_ENTRY_BWD) exceeds that is
 * rejected with TTT_ERR_WORKSPACE before any launch.  The call allocates
 * nothing.  Every call on one GPU shares that GPU's array: calls that may run
 * at the same time on one GPU (unordered streams) race; calls ordered on one
 * stream do not.
 */
TTT_API int ttt_chunk_bwd_noalloc(const ttt_desc* desc, const void* q, const void* k, const void* v,
                                  const float* beta, const float* gamma, const float* log_decay, const float* w0,
                                  const float* w_ckpt, const void* saved, const void* d_o, const float* d_wfinal,
                                  void* dq, void* dk, void* dv, float* dbeta, float* dgamma, float* dlog_decay,
                                  float* dw0, void* stream);

/* Bytes of the fixed scratch array behind ttt_chunk_bwd_noalloc (per GPU). */
TTT_API size_t ttt_noalloc_scratch_bytes(void);

/* Message for the last non-OK return on this thread ("" if none). */
TTT_API const char* ttt_last_error(void);

/* Library version string, e.g. "libttt 0.1 gfx950". */
TTT_API const char* ttt_version(void);

/*
 * Per-kernel timing (measurement support, not part of the layer's math).
 * While timing is on, every kernel launched by the entry points above is
 * bracketed by two HIP events recorded on the launch stream, so the time
 * between them is that kernel's duration on the device.
 *
 * ttt_timing_enable(1) clears the record and turns timing on; (0) turns it
 * off and keeps the record.  Events come from a pool the library creates on
 * first use and keeps until the process ends.
 * ttt_timing_read(kernel, &total_ms, &launches) waits for the recorded
 * events of that kernel (a host synchronisation on them) and returns the
 * summed duration and the number of launches since the last enable.
 * kernel is a ttt_kernel value.  Either output pointer may be NULL.
 * Not thread-safe with concurrent launches from other threads.
 */
typedef enum {
  TTT_KERNEL_FWD = 0,            /* matrix-core forward */
  TTT_KERNEL_BWD_SEQ = 1,        /* matrix-core backward, reverse sweep */
  TTT_KERNEL_BWD_CROSS = 2,      /* matrix-core backward, cross-column terms */
  TTT_KERNEL_DGAMMA = 3,         /* per-chain sum of the scalar-decay gradient */
  TTT_KERNEL_GENERIC_FWD = 4,    /* VALU forward */
  TTT_KERNEL_GENERIC_BWD = 5,    /* VALU backward */
  TTT_KERNEL_DECAY_CUMSUM = 6,   /* in-chunk cumulative sum of log a (VALU path) */
  TTT_KERNEL_INPLACE_APPLY = 7,  /* In-Place apply GEMM */
  TTT_KERNEL_INPLACE_UPDATE = 8, /* In-Place update GEMM */
  TTT_KERNEL_DECAY_PREP = 9,     /* vector decay: Q~, K~, lambda per chunk (matrix-core path) */
  TTT_KERNEL_INPLACE_NORM = 10,  /* In-Place update norm GEMM and clip scale */
  TTT_KERNEL_LIN_STATE = 11,     /* chunk-parallel forward (IP loss, no act): per-chunk K^T G */
  TTT_KERNEL_LIN_SCAN = 12,      /* chunk-parallel forward: state recurrence over chunks */
  TTT_KERNEL_LIN_OUT = 13,       /* chunk-parallel forward: query view per chunk */
  TTT_KERNEL_INPLACE_BWD_W = 14, /* In-Place backward: state rewound by one chunk */
  TTT_KERNEL_INPLACE_BWD_DZ = 15,/* In-Place backward: dZ (two-term GEMM and its sum) */
  TTT_KERNEL_INPLACE_BWD_DV = 16,/* In-Place backward: dV_hat */
  TTT_KERNEL_INPLACE_BWD_DW = 17,/* In-Place backward: dW chain */
  TTT_KERNEL_MLP_FWD = 18,       /* two-layer fast net forward */
  TTT_KERNEL_MLP_BWD = 19,       /* two-layer fast net backward, reverse sweep */
  TTT_KERNEL_NORM_FWD = 20,      /* Linear -> Norm forward */
  TTT_KERNEL_NORM_BWD = 21,      /* Linear -> Norm backward, reverse sweep */
  TTT_KERNEL_NORM_QUERY = 22,    /* row-path forward: query view of every chunk */
  TTT_KERNEL_NORM_BWD_PRE = 23,  /* row-path backward: chunk-parallel terms free of the carried dW */
  TTT_KERNEL_MLP_QUERY = 24,     /* two-layer fast net forward: query view of every chunk */
  TTT_KERNEL_MLP_BWD_PRE = 25,   /* two-layer fast net backward: chunk-parallel terms free of the carried dW */
  TTT_KERNEL_COUNT = 26
} ttt_kernel;

TTT_API int ttt_timing_enable(int on);
TTT_API int ttt_timing_read(int kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H */

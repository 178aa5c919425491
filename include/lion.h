/*
 * lion.h -- C ABI of the LION layers (Lion-s, Lion-d, Lion-lit) of libgbla.so
 * (MI355X, gfx950).
 *
 * The layer is the LION family of "Linear Attention for Efficient Bidirectional
 * Sequence Modeling": section "方法详解" (method details), key design 1
 * (bidirectional mask), key design 3 (chunkwise form, Theorem 3.2), the table of
 * the three instantiated models and the feature map under "损失函数/训练策略".
 * For every packed sequence b (rows cu_seqlens[b] .. cu_seqlens[b+1]-1) and
 * every head h:
 *
 *   q, k, v   = x W_Q^h, x W_K^h, x W_V^h                (no conv, no bias)
 *   lambda_i  = sigmoid(x_i . w_lam^h + b_lam^h)         (Lion-s: selective decay)
 *             = sigmoid(b_lam^h)                         (Lion-d: one learnt decay
 *                                                          per head, M_ij = lambda^|i-j|)
 *             = 1                                        (Lion-lit: no decay, M = 1)
 *   phi(u)    = (SiLU(u) + 0.5) / ||SiLU(u) + 0.5||_2    (on q and k, per head vector)
 *   M_ij      = prod_{k=j+1..i} lambda_k (j <= i),  prod_{k=i+1..j} lambda_k (j >= i)
 *               (M = M^F + M^B - I: the diagonal counts once)
 *   P         = (phi(Q) phi(K)^T) (.) M
 *   y_i       = sum_j P_ij v_j / sum_j P_ij              (Scale = row normalisation)
 *
 * The decay of a sequence's first token never enters M. The library evaluates
 * the chunkwise form with chunks of 64 tokens inside each sequence; it equals
 * the full form above up to rounding. Heads are concatenated in y (head h in
 * columns h*d_h .. h*d_h+d_h-1).
 *
 * Conventions are those of gbla.h: DEVICE pointers, row-major, owned by the
 * caller, nothing allocated or kept; work enqueued on `stream`; argument errors
 * returned as gbla_status before anything is enqueued; cu_seqlens read on the
 * device only (malformed offsets schedule no token); deterministic results;
 * large arrays 16-byte aligned, b_lam, db_lam and cu_seqlens 4-byte aligned;
 * total_tokens * max(d_model, 3*H*d_h + H + 64) < 2^31,
 * max(d_model, 3*H*d_h + H + 64) < 2^21 and
 * ceil32(d_model) * (3*H*d_h + H + 64) < 2^31; calls that share a
 * workspace or an activation cache must not overlap in time.
 */
#ifndef LION_H_
#define LION_H_

#include "gbla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* the decay of the model table's three instances */
enum { LION_DECAY_SELECTIVE = 0, /* Lion-s */
       LION_DECAY_FIXED = 1,     /* Lion-d */
       LION_DECAY_NONE = 2 };    /* Lion-lit */

typedef struct {
  int32_t num_seqs;     /* N >= 1 packed sequences (empty sequences allowed) */
  int32_t total_tokens; /* T = cu_seqlens[N] >= 0 */
  int32_t d_model;      /* d: multiple of 8, >= 8 */
  int32_t num_heads;    /* H >= 1 */
  int32_t head_dim;     /* d_h: 32 or 64 */
  int32_t dtype;        /* GBLA_DTYPE_F32 or GBLA_DTYPE_BF16 */
  int32_t chunk;        /* tokens per chunk: must be 64 */
  int32_t decay;        /* LION_DECAY_SELECTIVE, LION_DECAY_FIXED or LION_DECAY_NONE */
} lion_problem;

/* Bytes of device workspace needed by lion_forward (backward = 0) or
 * lion_backward (backward = 1). */
GBLA_API gbla_status lion_workspace_size(const lion_problem* p, int backward, size_t* bytes);

/* Bytes of the activation cache `act` written by lion_forward and read by
 * lion_backward: the raw projections q, k, v (dtype), log lambda and the row
 * sums (float32, [T, H]) and the carried chunk states (float32). Its layout is
 * internal to the library. */
GBLA_API gbla_status lion_activation_size(const lion_problem* p, size_t* bytes);

/* Forward pass.
 *   x        [T, d]        input rows (dtype)
 *   cu_seqlens [N+1] int32 sequence offsets
 *   w_q, w_k, w_v [d, H*d_h] projections; head h owns columns h*d_h.. (dtype)
 *   w_lam    [H, d]        decay weights (dtype), Lion-s only (may be NULL otherwise)
 *   b_lam    [H]           decay bias (Lion-s) or decay logit (Lion-d), float32;
 *                          may be NULL for Lion-lit
 *   y        [T, H*d_h]    output (dtype, overwritten)
 *   act      activation cache (lion_activation_size bytes, overwritten), needed
 *            by lion_backward; NULL for inference (the workspace then holds it)
 *   workspace, workspace_bytes: at least lion_workspace_size(p, 0) bytes */
GBLA_API gbla_status lion_forward(const lion_problem* p, const void* x, const int32_t* cu_seqlens, const void* w_q,
                                  const void* w_k, const void* w_v, const void* w_lam, const float* b_lam, void* y,
                                  void* act, void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass: gradients of sum(y * dy) for the forward above, by the chain
 * rule through the definitions in the header comment (with d lambda / d a =
 * lambda (1 - lambda) for the decay logit a). Inputs as in lion_forward plus
 *   act      the cache written by lion_forward for the same inputs (required)
 *   y        the output of that lion_forward (dtype)
 *   dy       [T, H*d_h]    upstream gradient (dtype)
 * Outputs (all overwritten, never accumulated):
 *   dx       [T, d] (dtype);  dw_q, dw_k, dw_v [d, H*d_h];
 *   dw_lam   [H, d]  Lion-s only (may be NULL otherwise, not written)
 *   db_lam   [H]     Lion-s and Lion-d (may be NULL for Lion-lit, not written)
 *   (all float32 except dx)
 *   workspace, workspace_bytes: at least lion_workspace_size(p, 1) bytes */
GBLA_API gbla_status lion_backward(const lion_problem* p, const void* x, const int32_t* cu_seqlens, const void* w_q,
                                   const void* w_k, const void* w_v, const void* w_lam, const float* b_lam,
                                   const void* act, const void* y, const void* dy, void* dx, float* dw_q, float* dw_k,
                                   float* dw_v, float* dw_lam, float* db_lam, void* workspace, size_t workspace_bytes,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LION_H_ */

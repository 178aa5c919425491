/*
 * gbla.h -- C ABI of the MI355X (gfx950) Gated Bidirectional Linear Attention
 * library (libgbla.so).
 *
 * The layer is the one of "Gated Bidirectional Linear Attention for Generative
 * Retrieval", section "核心方法" (core method), Eqs. (4)-(6). For every packed
 * sequence b (rows cu_seqlens[b] .. cu_seqlens[b+1]-1) and every head h:
 *
 *   x~      = causal depthwise Conv1d(x), kernel 4                (Eq. (4))
 *   q, k, v = x~ W_Q^h, x~ W_K^h, x~ W_V^h                       (Eq. (4), per-head weights)
 *   g_j     = sigmoid(x~_j . w_g^h + b_g^h)                      (key gate of Eq. (5))
 *          or softmax over the sequence's tokens j of x~_j . w_g^h + b_g^h
 *             (GBLA_GATE_SOFTMAX: the gate exactly as Eq. (5) writes it)
 *   S       = sum_j g_j phi(k_j) v_j^T,  z = sum_j g_j phi(k_j)  (Eq. (6), phi(u) = elu(u) + 1)
 *   O_i     = phi(q_i)^T S / phi(q_i)^T z                        (Eq. (5), state-first order of Eq. (3))
 *   y_i     = O_i, or with the gated RMSNorm output (component (3), Eq. (7))
 *   y_i     = gamma (.) O_i / sqrt(mean_c O_ic^2 + eps) (.) SiLU(x~_i W_R^h)
 *             (RMS over the head's d_h features, eps inside the root, gamma [d_h]
 *             a learnable scale shared by the heads, or none)
 *
 * The conv restarts at every sequence start (zero left padding, tap 3 multiplies
 * the current token, tap k the token 3-k steps back) and S, z cover only the
 * sequence's own tokens. No 1/sqrt(d_h) scale, no epsilon, no projection bias;
 * y concatenates the heads (head h in columns h*d_h .. h*d_h+d_h-1).
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers (HIP), row-major, owned by the
 *    caller; the library allocates nothing and keeps no pointer after a call
 *    returns. Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and nothing synchronises with the host, so outputs are ready only
 *    when that stream is.
 *  - Activations, weights and y/dx use the problem's dtype (float32 or
 *    bfloat16); accumulation is float32; b_g, saved state and all weight
 *    gradients are float32.
 *  - Argument errors are detected on the host before anything is enqueued and
 *    returned as a gbla_status; GBLA_ERR_HIP reports a failed launch.
 *  - cu_seqlens must satisfy cu[0] = 0, cu[b] <= cu[b+1], cu[N] = total_tokens.
 *    It is read on the device only; if it is malformed, no token is scheduled
 *    (outputs are unspecified but no memory outside the arguments is touched).
 *  - Results are deterministic: every reduction runs in a fixed order with no
 *    floating-point atomics, so repeated calls are bitwise identical.
 *  - Large arrays must be 16-byte aligned; b_g, db_g, dconv_w, gamma, dgamma
 *    and cu_seqlens 4-byte aligned.
 *  - Sizes: total_tokens * max(d_model, S*H*d_h + H + 64) < 2^31,
 *    max(d_model, S*H*d_h + H + 64) < 2^21 and
 *    ceil32(d_model) * (S*H*d_h + H + 64) < 2^31, S = 3 (4 with the gated
 *    output); otherwise GBLA_ERR_BAD_SHAPE.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef GBLA_H_
#define GBLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define GBLA_API __attribute__((visibility("default")))
#else
#define GBLA_API
#endif

typedef enum {
  GBLA_OK = 0,
  GBLA_ERR_NULL_ARG = 1,            /* a required pointer is NULL */
  GBLA_ERR_BAD_SHAPE = 2,           /* sizes out of the supported range */
  GBLA_ERR_UNSUPPORTED = 3,         /* dtype, head_dim, gate or conv width not supported */
  GBLA_ERR_MISALIGNED = 4,          /* pointer alignment violated */
  GBLA_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes below the size query */
  GBLA_ERR_HIP = 6,                 /* a HIP launch failed */
  GBLA_ERR_SCRATCH_LIMIT = 7        /* gbla_forward_noalloc: problem larger than its static scratch */
} gbla_status;

enum { GBLA_DTYPE_F32 = 0, GBLA_DTYPE_BF16 = 1 };
/* key gate of Eq. (5): per-token sigmoid, or softmax over the sequence. The
 * output does not change if every gate of a sequence is scaled by the same
 * factor, so the softmax gate is evaluated as exp(s_j - m) with m the
 * sequence's largest logit, and its normaliser never needs to be formed; its
 * bias gradient db_g is zero up to rounding (the softmax is shift invariant). */
enum { GBLA_GATE_SIGMOID = 0, GBLA_GATE_SOFTMAX = 1 };
/* readout: O itself, or the gated RMSNorm output of Eq. (7) */
enum { GBLA_OUTPUT_PLAIN = 0, GBLA_OUTPUT_GATED_RMSNORM = 1 };

typedef struct {
  int32_t num_seqs;     /* N >= 1 packed sequences (empty sequences allowed) */
  int32_t total_tokens; /* T = cu_seqlens[N] >= 0 */
  int32_t d_model;      /* d: multiple of 8, >= 8 */
  int32_t num_heads;    /* H >= 1 */
  int32_t head_dim;     /* d_h: 32 or 64 */
  int32_t dtype;        /* GBLA_DTYPE_F32 or GBLA_DTYPE_BF16 */
  int32_t gate;         /* GBLA_GATE_SIGMOID or GBLA_GATE_SOFTMAX */
  int32_t conv_width;   /* must be 4 */
  int32_t output_gate;  /* GBLA_OUTPUT_PLAIN or GBLA_OUTPUT_GATED_RMSNORM */
  float norm_eps;       /* eps of the gated output's RMSNorm: finite, >= 0 (ignored when plain) */
} gbla_problem;

/* Human-readable name of a status code (static string). */
GBLA_API const char* gbla_status_string(int status);

/* Library ABI version (increments on any signature change). */
GBLA_API int gbla_version(void);

/* Bytes of the `saved` buffer written by gbla_forward and read by
 * gbla_backward: N * H * (d_h*d_h + d_h) float32 values, laid out
 * [N][H][S (d_h x d_h, row i = key feature, column = value feature) | z (d_h)].
 * With GBLA_GATE_SOFTMAX, S and z are built from the unnormalised gates
 * exp(s_j - m) (so they are the softmax-gated states times sum_j exp(s_j - m))
 * and N * H more floats follow: m, the largest gate logit of every (sequence,
 * head), 0 for an empty sequence. */
GBLA_API gbla_status gbla_saved_size(const gbla_problem* p, size_t* bytes);

/* Bytes of device workspace needed by gbla_forward (backward = 0) or
 * gbla_backward (backward = 1); enough whether or not an activation cache is
 * passed. */
GBLA_API gbla_status gbla_workspace_size(const gbla_problem* p, int backward, size_t* bytes);

/* Bytes of the optional activation cache `act`: the conv output, phi(q),
 * phi(k), v, with the gated output also x~ W_R (dtype), and the gates
 * (float32) of every token, and the batch's table of 256-token chunks, kept
 * by gbla_forward so that gbla_backward needs no recomputation. Its layout is
 * internal to the library. */
GBLA_API gbla_status gbla_activation_size(const gbla_problem* p, size_t* bytes);

/* Forward pass, Eqs. (4)-(6).
 *   x        [T, d]        input rows (dtype)
 *   cu_seqlens [N+1] int32 sequence offsets
 *   conv_w   [d, 4]        depthwise conv taps (dtype)
 *   w_q, w_k, w_v [d, H*d_h] projections; head h owns columns h*d_h.. (dtype)
 *   w_g      [H, d]        gate weights (dtype);  b_g [H] gate bias (float32)
 *   w_r      [d, H*d_h]    Eq. (7) gate weights, head h in columns h*d_h.. (dtype);
 *                          required with GBLA_OUTPUT_GATED_RMSNORM, NULL otherwise
 *   gamma    [d_h]         Eq. (7) RMSNorm scale (float32), or NULL for none;
 *                          must be NULL without the gated output
 *   y        [T, H*d_h]    output (dtype, overwritten)
 *   saved    see gbla_saved_size (float32, overwritten): the states S and z
 *   act      optional activation cache (gbla_activation_size bytes, overwritten)
 *            for a later gbla_backward; NULL for inference
 *   workspace, workspace_bytes: at least gbla_workspace_size(p, 0) bytes */
GBLA_API gbla_status gbla_forward(const gbla_problem* p, const void* x, const int32_t* cu_seqlens, const void* conv_w,
                                  const void* w_q, const void* w_k, const void* w_v, const void* w_g, const float* b_g,
                                  const void* w_r, const float* gamma, void* y, float* saved, void* act,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---- Allocation-free forward -------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward pass and results as gbla_forward (same kernels, bitwise equal), with
 * no workspace argument. Its workspace is a static device array of
 * GBLA_STATIC_SCRATCH_BYTES built into the library; every GPU the library runs
 * on holds its own copy until the process ends. The call allocates nothing and
 * calls no allocating routine.
 * It needs gbla_workspace_size(p, 0) bytes of that array without an activation
 * cache, and gbla_workspace_size(p, 0) - gbla_activation_size(p) bytes with one
 * (the activations then go to `act`); a larger problem returns
 * GBLA_ERR_SCRATCH_LIMIT before anything is enqueued. All calls on one GPU
 * share its array and keep no state in it between calls (nothing is read
 * before it is written), so calls that overlap in time on one GPU (on
 * different streams or from different threads) race and must be ordered by
 * the caller. Arguments, layouts and other errors as gbla_forward. */
#define GBLA_STATIC_SCRATCH_BYTES (128u << 20)
GBLA_API gbla_status gbla_forward_noalloc(const gbla_problem* p, const void* x, const int32_t* cu_seqlens,
                                          const void* conv_w, const void* w_q, const void* w_k, const void* w_v,
                                          const void* w_g, const float* b_g, const void* w_r, const float* gamma,
                                          void* y, float* saved, void* act, void* stream);

/* Backward pass: gradients of sum(y * dy) for the forward above, obtained by
 * the chain rule through Eqs. (4)-(6). Inputs as in gbla_forward plus
 *   saved    the state written by gbla_forward for the same inputs (float32)
 *   act      the activation cache written by that gbla_forward, or NULL to
 *            recompute the activations from x (same results)
 *   dy       [T, H*d_h]    upstream gradient (dtype)
 * Outputs (all overwritten, never accumulated):
 *   dx       [T, d] (dtype);  dconv_w [d, 4];  dw_q, dw_k, dw_v [d, H*d_h];
 *   dw_g     [H, d];  db_g [H]   (all float32)
 *   dw_r     [d, H*d_h] (float32): required with the gated output, NULL otherwise
 *   dgamma   [d_h] (float32): required exactly when gamma is given
 *   workspace, workspace_bytes: at least gbla_workspace_size(p, 1) bytes */
GBLA_API gbla_status gbla_backward(const gbla_problem* p, const void* x, const int32_t* cu_seqlens, const void* conv_w,
                                   const void* w_q, const void* w_k, const void* w_v, const void* w_g, const float* b_g,
                                   const void* w_r, const float* gamma, const float* saved, const void* act,
                                   const void* dy, void* dx, float* dconv_w, float* dw_q, float* dw_k, float* dw_v,
                                   float* dw_g, float* db_g, float* dw_r, float* dgamma, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---- Optional per-stage timing (benchmarking aid) ----------------------
 * gbla_profile_begin opens a process-wide window of at most max_records
 * stage launches. While it is open, every stage of the forward and backward
 * entry points (GBLA and LION-s) records a HIP event before and after its
 * kernels on the caller's stream.
 * gbla_profile_end waits for those events, writes per-stage total device
 * milliseconds and launch counts for min(max_stages, *n_stages) stages
 * (names: gbla_profile_stage_name), and closes the window. Launches beyond
 * max_records are not timed. While no window is open the entry points touch
 * no shared state (one atomic flag read per stage, no lock), so calls on
 * separate workspaces and streams may run concurrently; opening and closing a
 * window is not meant to race with itself.
 * Errors: GBLA_ERR_BAD_SHAPE (max_records out of [1, 2^20], or end without
 * begin), GBLA_ERR_NULL_ARG, GBLA_ERR_HIP (event creation/query failed). */
GBLA_API gbla_status gbla_profile_begin(int max_records);
/* Same window, but only the stages whose bit (1 << stage) is set in stage_mask
 * record events (each recorded event costs device time, so a narrow mask keeps
 * the timed work close to an unprofiled run). */
GBLA_API gbla_status gbla_profile_begin_stages(int max_records, uint64_t stage_mask);
GBLA_API gbla_status gbla_profile_end(double* ms_per_stage, int* launches_per_stage, int max_stages, int* n_stages);
GBLA_API const char* gbla_profile_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* GBLA_H_ */

/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer: forward,
 * expert-choice routing and the training backward.
 *
 * The layer (pages: botmartz "Mixture of Experts (MoE) and Mixtral", sections
 * "MoE Architecture" and "Expert Routing"; roadtointelligence "Mixture of
 * Experts", router formula and output equation; matteuscruz "Mixture of
 * Experts", "Architecture: router + experts" and "Load balancing"):
 *
 *   l = x W_g^T + b_g                          router scores, fp32
 *   p = softmax(l); top-k of p                 slots in descending order,
 *                                              lowest expert index on ties
 *   g_i = p_{e_i} / sum_j p_{e_j}              renormalised gates
 *   capacity: per expert the first C (token, slot) pairs in token order are
 *             kept, the rest dropped (they contribute zero)
 *   E_e(x) = W2[e] act(W1[e] x + b1[e]) + b2[e]   act = exact GELU or ReLU
 *   y = sum_{kept i} g_i E_{e_i}(x)  (+ S(x), an always-on shared expert)
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers, row-major and contiguous, owned
 *    by the caller.  The library allocates and frees nothing, keeps no state
 *    between calls and is re-entrant; two calls that share a workspace or an
 *    output buffer on different streams race.  (moe_forward_noalloc is the
 *    one exception: it keeps a static device scratch array per GPU.)
 *  - Expert weights use the nn.Linear layout [out, in]: W1 [E, d_ff, d_model],
 *    W2 [E, d_model, d_ff]; b1 [E, d_ff], b2 [E, d_model].  They, x and y are
 *    fp32 (MOE_F32) or bf16 (MOE_BF16, raw 16-bit patterns) as cfg->dtype
 *    says.  Router weight W_g [E, d_model] and bias b_g [E] are always fp32.
 *    Every bias pointer may be NULL (zero bias).
 *  - Expert indices are 0-based.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *    enqueued: no call synchronises, reads device memory on the host or
 *    allocates, so a sequence of calls can be captured in a HIP graph.
 *  - Results are reproducible bit for bit for the same inputs and config: no
 *    floating-point atomics, every sum in a fixed order.
 *  - Arguments are validated before anything is enqueued; a failed check
 *    returns a negative moe_status and enqueues nothing.  A failed launch
 *    returns MOE_ERR_HIP (hipGetLastError has the detail).  Nothing is printed.
 *  - Workspace: ws must be 256-byte aligned device memory of at least
 *    moe_workspace_bytes(cfg) bytes (one size serves every entry point).  Its
 *    contents need no initialisation and are garbage after the call.
 *  - Limits: 1 <= n_experts <= 1024, 1 <= top_k <= min(n_experts, 32),
 *    d_model, d_ff and shared_d_ff multiples of 8, T * (top_k + 1) < 2^31
 *    (under MOE_ROUTE_EXPERT: E * C + T < 2^31), x / weight / y pointers
 *    16-byte aligned.
 *  - moe_route, moe_dispatch and moe_combine take token-choice configs only
 *    (MOE_ERR_UNSUPPORTED under MOE_ROUTE_EXPERT); moe_expert_ffn and
 *    moe_forward take both.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null required pointer, bad size, misalignment */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside the limits above */
  MOE_ERR_WORKSPACE = -3,   /* ws NULL, misaligned or smaller than needed */
  MOE_ERR_HIP = -4,         /* a HIP launch failed */
  MOE_ERR_SCRATCH = -5      /* moe_forward_noalloc: the layer needs more workspace than
                               MOE_NOALLOC_SCRATCH_BYTES */
} moe_status;

enum { MOE_F32 = 0, MOE_BF16 = 1 };
enum { MOE_ACT_GELU = 0 /* 0.5 z (1 + erf(z / sqrt 2)) */, MOE_ACT_RELU = 1 };

/*
 * Routing direction.
 *  MOE_ROUTE_TOKEN: each token takes its top-k experts (the layer above).
 *  MOE_ROUTE_EXPERT: expert-choice routing (matteuscruz "Mixture of Experts",
 *    "Load balancing", expert choice routing): each expert takes the C tokens
 *    with the highest router probability p[t, e], C = capacity when
 *    capacity >= 0, else floor(T * top_k / E) (top_k read as the capacity
 *    factor), at most T; among equal fp32 probabilities the lower token index
 *    wins.  y[t] = sum over the experts that took t, in ascending expert order,
 *    of p[t, e] E_e(x_t) (+ S(x_t)); renormalize is ignored.  A token may be
 *    taken by any number of experts, including none.
 */
enum { MOE_ROUTE_TOKEN = 0, MOE_ROUTE_EXPERT = 1 };

typedef struct {
  int64_t T;           /* tokens (batch * seq_len, flattened) */
  int32_t d_model;     /* d */
  int32_t d_ff;        /* routed expert hidden size F */
  int32_t n_experts;   /* E */
  int32_t top_k;       /* k */
  int32_t act;         /* MOE_ACT_GELU or MOE_ACT_RELU */
  int32_t dtype;       /* MOE_F32 or MOE_BF16 */
  int32_t capacity;    /* < 0: unlimited; else max kept rows per routed expert */
  int32_t renormalize; /* 1: g_i = p_i / sum p over the top-k; 0: g_i = p_i */
  int32_t shared_d_ff; /* hidden size of the always-on shared expert, 0 = none */
  int32_t routing;     /* MOE_ROUTE_TOKEN or MOE_ROUTE_EXPERT */
} moe_config;

typedef struct {
  const float *Wg, *bg;                /* [E, d] fp32, [E] fp32 or NULL */
  const void *W1, *b1, *W2, *b2;       /* routed experts, see layout above */
  const void *Ws1, *bs1, *Ws2, *bs2;   /* shared expert [Fs, d], [Fs], [d, Fs], [d] */
} moe_weights;

/* Optional per-call outputs of moe_forward; every member may be NULL. */
typedef struct {
  int32_t *topk_idx; /* [T, k] chosen experts; must be NULL under MOE_ROUTE_EXPERT */
  float *topk_w;     /* [T, k] gates; must be NULL under MOE_ROUTE_EXPERT */
  int32_t *counts;   /* [E] routed (token, slot) pairs per expert (C each under
                        MOE_ROUTE_EXPERT) */
  int32_t *kept;     /* [E] pairs that survived the capacity limit (C each under
                        MOE_ROUTE_EXPERT) */
  float *mean_prob;  /* [E] mean router probability over tokens (NaN if T = 0) */
  float *balance;    /* [1] unbiased variance of mean_prob over experts (NaN if E = 1) */
  float *cv2;        /* [1] squared coefficient of variation of counts: unbiased variance
                        over experts / mean^2, in fp64 (NaN if E = 1 or no pairs);
                        invest-in.ai "Common Usage Examples" (cv_squared of expert
                        counts), matteuscruz "Load balancing" */
  int32_t *ec_idx;   /* [E, C] under MOE_ROUTE_EXPERT: the tokens expert e took, ascending;
                        must be NULL under MOE_ROUTE_TOKEN */
  float *ec_w;       /* [E, C] under MOE_ROUTE_EXPERT: their gates p[t, e] (fp32);
                        must be NULL under MOE_ROUTE_TOKEN */
} moe_stats;

/* Workspace bytes that every entry point below accepts for this config
 * (0 on an invalid config). */
size_t moe_workspace_bytes(const moe_config *cfg);

/*
 * Router and gating: scores, softmax, top-k, renormalise (botmartz "Expert
 * Routing"; roadtointelligence router formula, "Tiny example").
 *   x [T, d] (cfg->dtype); Wg [E, d] fp32; bg [E] fp32 or NULL
 *   topk_idx [T, k] int32 out; topk_w [T, k] fp32 out
 *   probs [T, E] fp32 out or NULL: the full softmax
 *   mean_prob [E] and balance [1] fp32 out or NULL: load statistics
 *     (botmartz "Load Balancing": mean of the probabilities over tokens and
 *     the square of their standard deviation over experts)
 */
moe_status moe_route(const moe_config *cfg, const void *x, const float *Wg, const float *bg,
                     int32_t *topk_idx, float *topk_w, float *probs, float *mean_prob,
                     float *balance, void *ws, size_t ws_bytes, void *stream);

/*
 * Dispatch: group (token, slot) pairs by expert under the capacity limit
 * (matteuscruz "Load balancing", expert capacity buffer; roadtointelligence
 * "Keeping the experts busy": overflow tokens are dropped).
 *   topk_idx [T, k] int32 in, values in [0, E).  An out-of-range id is
 *     dropped (inv = -1); the grouping of the other pairs is then unspecified,
 *     but nothing is written outside the arrays described here.
 *   counts [E], kept [E] int32 out
 *   offsets [E + 2] int32 out: rows of expert e are offsets[e] .. offsets[e+1]-1,
 *     offsets[E] = routed rows R, offsets[E+1] = R + (shared_d_ff ? T : 0)
 *   row_token, row_slot [T*k + (shared_d_ff ? T : 0)] int32 out: token and slot
 *     of each row; rows are expert-major and token-ascending inside an expert;
 *     the shared expert's rows R + t have token t and slot -1
 *   inv [T, k] int32 out: row of each (token, slot), -1 if dropped
 */
moe_status moe_dispatch(const moe_config *cfg, const int32_t *topk_idx, int32_t *counts,
                        int32_t *kept, int32_t *offsets, int32_t *row_token, int32_t *row_slot,
                        int32_t *inv, void *ws, size_t ws_bytes, void *stream);

/*
 * Expert MLPs over the grouped rows (botmartz "Expert Routing" expert
 * networks; codingnowai "Code"; roadtointelligence shared expert):
 *   y_rows[r, :] = gate_r * (W2[e] act(W1[e] x[row_token[r]] + b1[e]) + b2[e])
 * with gate_r = topk_w[row_token[r], row_slot[r]] for routed rows and 1 for
 * shared rows (which use Ws1, bs1, Ws2, bs2).
 *   x [T, d]; offsets, row_token, row_slot as produced by moe_dispatch;
 *   topk_w [T, k] fp32; y_rows [T*k + (shared_d_ff ? T : 0), d] fp32 out (only
 *   the first offsets[E+1] rows are written).
 * Under MOE_ROUTE_EXPERT the routed rows are moe_forward's selection: row
 * e*C + j is token ec_idx[e, j] with gate_r = topk_w[r] = ec_w[e, j]
 * (topk_w [E*C] fp32), offsets[e] = e*C, offsets[E] = E*C, offsets[E+1] =
 * E*C (+ T with a shared expert, whose rows E*C + t are token t); row_slot is
 * not read (may be NULL); y_rows has E*C (+ T) rows.
 */
moe_status moe_expert_ffn(const moe_config *cfg, const void *x, const moe_weights *w,
                          const int32_t *offsets, const int32_t *row_token,
                          const int32_t *row_slot, const float *topk_w, float *y_rows, void *ws,
                          size_t ws_bytes, void *stream);

/*
 * Combine: y[t] = sum over slots i = 0..k-1 with inv[t,i] >= 0 of
 * y_rows[inv[t,i]], then + y_rows[offsets[E] + t] if there is a shared expert,
 * summed in that order in fp32, no atomics (roadtointelligence output
 * equation; botmartz "Expert Routing" accumulation into zeros_like(x)).
 *   y [T, d] out in cfg->dtype.  Needs no workspace.
 */
moe_status moe_combine(const moe_config *cfg, const float *y_rows, const int32_t *inv,
                       const int32_t *offsets, void *y, void *stream);

/*
 * The whole layer: route, dispatch, expert MLPs, combine.  y [T, d] out in
 * cfg->dtype; stats may be NULL or have NULL members (topk_idx and topk_w must
 * be NULL under MOE_ROUTE_EXPERT, ec_idx and ec_w under MOE_ROUTE_TOKEN, else
 * MOE_ERR_INVALID_ARG).
 */
moe_status moe_forward(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
                       moe_stats *stats, void *ws, size_t ws_bytes, void *stream);

/* Device scratch that moe_forward_noalloc uses in place of a workspace. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same layer, same kernels and same results bit for bit as moe_forward, with
 * the workspace taken from a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends.  The
 * caller still passes x, y and the weights (and the optional stats).
 *  - Rejects a config with moe_workspace_bytes(cfg) > MOE_NOALLOC_SCRATCH_BYTES
 *    with MOE_ERR_SCRATCH before enqueuing anything.
 *  - Calls no hipMalloc, hipFree or allocating routine.  The first call on a
 *    device (with that device current) looks up the array's address there
 *    (hipGetSymbolAddress) and keeps it; make that first call outside graph
 *    capture.
 *  - Every call on one GPU shares that GPU's array and leaves its contents
 *    behind; nothing in it needs to start at zero (the kernels clear what
 *    they count).  Calls that overlap on one GPU (different streams, or
 *    threads racing on one stream) race on the array: serialise them.
 */
moe_status moe_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x,
                               void *y, moe_stats *stats, void *stream);

/* ---------------------------------------------------------------------------
 * Training: forward that keeps what the backward needs, and the backward.
 *
 * The backward returns the gradients of
 *     L = sum_t <dy_t, y_t> + aux_coef * balance
 * (dy: the upstream gradient of y; balance: the moe_stats statistic, the
 * unbiased variance over experts of the mean router probability, which the
 * pages add to the task loss with a small coefficient: botmartz "Load
 * Balancing: The Hidden Challenge", total_loss = task_loss + 0.01 *
 * balance_loss; roadtointelligence "Keeping the experts busy"; matteuscruz
 * "Load balancing").  The top-k selection and the capacity drops are held
 * fixed, as autograd treats them: a dropped slot gets no gate gradient but
 * still counts in the renormalisation sum.  With E = 1 the balance term has
 * no gradient.  Under MOE_ROUTE_EXPERT the selection is held fixed and each
 * taken pair's gate is p[t, e] (no renormalisation).
 */

/* Gradients written by moe_backward; each member may be NULL (not computed).
 * Each has the layout and dtype of its tensor: dx [T, d] and the expert weight
 * and bias gradients in cfg->dtype, dWg [E, d] and dbg [E] fp32.  The shared
 * expert's members must be NULL when shared_d_ff = 0.  dx and the weight
 * gradients dW1, dW2, dWs1, dWs2 must be 16-byte aligned.  Gradients overwrite
 * (they are not accumulated into). */
typedef struct {
  void *dx;
  float *dWg, *dbg;
  void *dW1, *db1, *dW2, *db2;
  void *dWs1, *dbs1, *dWs2, *dbs2;
} moe_grads;

/* Workspace bytes of moe_forward_train + moe_backward (0 on an invalid
 * config).  Besides the forward's buffers it holds the
 * pre-activations, the softmax and transposed copies of the grouped
 * activations (each expert's rows padded to a multiple of 64). */
size_t moe_train_workspace_bytes(const moe_config *cfg);

/*
 * moe_forward that also leaves in ws what moe_backward reads: the routing
 * (or the expert-choice selection), the grouping, the softmax, the
 * pre-activations z and hidden
 * activations h of every row, and the gated expert outputs.  Same arguments
 * and outputs as moe_forward; ws must have moe_train_workspace_bytes(cfg)
 * bytes and stay untouched until the moe_backward call that consumes it.
 */
moe_status moe_forward_train(const moe_config *cfg, const moe_weights *w, const void *x, void *y,
                             moe_stats *stats, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of the moe_forward_train call that filled ws (same cfg, w and x).
 *   dy [T, d] in cfg->dtype (16-byte aligned); aux_coef: the balance term's
 *   coefficient (0 = none; NaN is rejected); grads: see moe_grads.
 * Enqueued on `stream` after that forward; ws is garbage afterwards (run
 * moe_forward_train again before another backward).  With T = 0 the requested
 * parameter gradients are zero.
 */
moe_status moe_backward(const moe_config *cfg, const moe_weights *w, const void *x,
                        const void *dy, float aux_coef, moe_grads *grads, void *ws,
                        size_t ws_bytes, void *stream);

/* Static description of a status code. */
const char *moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */

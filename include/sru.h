/*
 * sru.h -- C ABI of libsru, the MI355X (gfx950) implementation of one Simple
 * Recurrent Unit layer's hot path.
 *
 * The layer is the one defined in Lei, "When Attention Meets Fast Recurrence:
 * Training Language Models with Reduced Compute", background section on SRU,
 * Eqs. 1-5:
 *
 *   U^T = [W; W'; W''] X^T                              (Eq. 1)
 *   f[t] = sigma(U[t,0] + v  (.) c[t-1] + b )           (Eq. 2)
 *   r[t] = sigma(U[t,1] + v' (.) c[t-1] + b')           (Eq. 3)
 *   c[t] = f[t] (.) c[t-1] + (1 - f[t]) (.) U[t,2]      (Eq. 4)
 *   h[t] = r[t] (.) c[t] + (1 - r[t]) (.) (alpha x[t])  (Eq. 5, alpha = 1 is
 *                                                        the paper's form)
 *
 * plus the chain-rule backward of Eqs. 2-5 and a linear mode (v = v' = 0) in
 * which the recurrence is an associative scan and is evaluated in time chunks,
 * the parallel-training idea of "Parallelizing Legendre Memory Unit Training"
 * (abstract).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *   allocates nothing and keeps no state across calls except a thread-local
 *   error string.
 * - Tensors are dense, row-major, innermost dimension last, and every base
 *   pointer must be 16-byte aligned.
 * - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *   null stream).  Calls return after enqueueing and never synchronise; a
 *   fault inside a kernel surfaces at the caller's next synchronisation.
 * - Arguments are validated before anything is launched; on any error
 *   nothing is written and the status says why (sru_last_error() has the
 *   detail).  No exception or abort crosses the ABI.
 * - Shapes: L (time), B (batch), d (hidden size) >= 1; ndir = 2 when
 *   `bidirectional` is 1, else 1.  Direction 1 walks t = L-1 .. 0 and its c0
 *   is the state before t = L-1.  x is shared by both directions.
 *
 * Layouts
 *   X, x     [L, B, d]                 (the layer input; X viewed as [L*B, d])
 *   W        [ndir*3*d, d]             row n = output feature n; per
 *                                      direction the blocks are f | r | cand.
 *   U, dU    [L, B, ndir, 3, d]        == the projection output [L*B, ndir*3*d]
 *   v, b     [ndir, 2, d]              row 0 = forget gate, row 1 = reset gate
 *   c0       [ndir, B, d]
 *   h, c_seq [L, B, ndir, d]           c_seq[t] is the state after step t
 *   c_last   [ndir, B, d]
 *   dh       [L, B, ndir, d]
 *   dx       [L, B, d]
 *   dv, db   [ndir, 2, d]
 *   dc0, dc_last [ndir, B, d]
 */
#ifndef SRU_H_
#define SRU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SRU_OK = 0,
    SRU_ERR_INVALID_ARG = 1,   /* bad shape, NULL required pointer, misalignment */
    SRU_ERR_UNSUPPORTED = 2,   /* dtype combination not implemented              */
    SRU_ERR_NO_DEVICE = 3,     /* no HIP device visible                          */
    SRU_ERR_LAUNCH = 4,        /* a kernel launch failed                         */
    SRU_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than required        */
    SRU_STATUS_RANGE_ = -2147483647 - 1   /* not a status; see SRU_DTYPE_RANGE_ */
} sru_status;

/* Each enum below ends in a *_RANGE_ member that is not a valid code: it
 * makes every int32 a representable value of the type, so that a code a C
 * caller passes outside the listed ones is refused by the argument checks
 * (SRU_ERR_INVALID_ARG) instead of being undefined in the library's C++. */
typedef enum { SRU_F32 = 0, SRU_BF16 = 1, SRU_DTYPE_RANGE_ = -2147483647 - 1 } sru_dtype;
typedef enum { SRU_FWD = 0, SRU_BWD = 1, SRU_PASS_RANGE_ = -2147483647 - 1 } sru_pass;
typedef enum {
    SRU_PROJ_FWD = 0,        /* C (+)= A W^T  : U = X~ W^T, A = X [L*B, d]           */
    SRU_PROJ_BWD_DATA = 1,   /* C (+)= A W    : dX = dU W, A = dU [L*B, ndir*3*d]    */
    SRU_PROJ_BWD_DATA_WT = 2, /* C (+)= A Wt^T : as BWD_DATA, with W passed transposed */
    SRU_PROJ_RANGE_ = -2147483647 - 1
} sru_proj_op;
typedef enum {
    SRU_WS_BACKWARD = 1,    /* sru_backward                      */
    SRU_WS_LINEAR_FWD = 2,  /* sru_linear_scan(SRU_FWD, chunk)   */
    SRU_WS_LINEAR_BWD = 3,  /* sru_linear_scan(SRU_BWD, chunk)   */
    SRU_WS_BWD_WEIGHT = 4,  /* sru_project_bwd_weight            */
    SRU_WS_FACTORED_WEIGHT = 5, /* sru_project_factored_bwd_weight, either
                                   gradient; `chunk` carries the inner dimension d' */
    SRU_WS_RANGE_ = -2147483647 - 1
} sru_ws_op;
typedef enum {
    SRU_FACT_Q = 0,      /* Q  [L*B, d']       (+)= X~  . Wq^T   Wq [d', d]        */
    SRU_FACT_U = 1,      /* U  [L*B, ndir*3d]  (+)= Q~  . Wo^T   Wo [ndir*3d, d']  */
    SRU_FACT_BWD_Q = 2,  /* dQ [L*B, d']       (+)= dU~ . Wo                       */
    SRU_FACT_BWD_X = 3,  /* dX [L*B, d]        (+)= dQ~ . Wq                       */
    SRU_FACT_RANGE_ = -2147483647 - 1
} sru_fact_op;
typedef enum {
    SRU_FACT_WGRAD_Q = 0,   /* dWq [d', d]      (+)= dQ~^T . X~ */
    SRU_FACT_WGRAD_O = 1,   /* dWo [ndir*3d, d'] (+)= dU~^T . Q~ */
    SRU_FACT_WGRAD_RANGE_ = -2147483647 - 1
} sru_fact_wgrad_op;

typedef struct {
    int64_t L, B, d;
    int32_t bidirectional;   /* 0 or 1 */
    float alpha;             /* highway scale; 1 reproduces Eq. 5 */
} sru_shape;

/* Options of the SRU++ attention (sru_attention_forward). */
typedef struct {
    int64_t d_inner;         /* attention dimension d' >= 1                        */
    int64_t mem_len;         /* Lm >= 0: the previous segment's steps in front of
                                this segment's keys and values                      */
    int32_t causal;          /* 1: step t sees the Lm context steps and steps <= t;
                                0: every step sees all Lm + L                       */
    int32_t layernorm;       /* 1: R = layernorm(Q + alpha A) with gamma, beta      */
    float attn_alpha;        /* alpha of the residual Q + alpha A (learned scalar,
                                initially 0 in the paper)                           */
    float ln_eps;            /* layer-norm epsilon (> 0 when layernorm = 1)         */
} sru_attn_cfg;

/*
 * Projection, Eq. 1 (SRU++ paper, background section): all three gate
 * matrices of both directions and all timesteps in one GEMM.
 *   SRU_PROJ_FWD:      C[L*B, ndir*3d] (+)= A[L*B, d] . W^T
 *   SRU_PROJ_BWD_DATA: C[L*B, d]       (+)= A[L*B, ndir*3d] . W
 *     (the input gradient through Eq. 1; pass accumulate = 1 with C = the dx
 *      returned by sru_backward to obtain the full input gradient).
 *   SRU_PROJ_BWD_DATA_WT: the same product with W supplied as its transpose
 *     Wt [d, ndir*3d] (from sru_transpose_weight); both operands are then
 *     contiguous along the reduction and the faster kernel path is used.
 * w_dt = SRU_BF16: bf16 MFMA with fp32 accumulation; A (fp32 or bf16) is
 *   rounded to bf16 (nearest even) as it is loaded.
 * w_dt = SRU_F32: fp32 arithmetic throughout (A widened if bf16).
 * c_dt must be SRU_F32.  accumulate = 0 overwrites C, 1 adds to it.
 */
sru_status sru_project(const sru_shape *shape, sru_proj_op op,
                       const void *A, sru_dtype a_dt,
                       const void *W, sru_dtype w_dt,
                       void *C, sru_dtype c_dt,
                       int32_t accumulate, void *stream);

/*
 * Weight gradient of the projection, Eq. 1 (SRU++ paper, background
 * section): U = X~ W^T, so dW = dU^T X~, summed over all L*B rows:
 *   dW[ndir*3d, d] (+)= dU[L*B, ndir*3d]^T . X[L*B, d]
 *   (row n of dW is the weight row that produced column n of U; the same
 *    row order as W in sru_project).
 * dU: du_dt in {F32, BF16} (sru_backward's dU or its dU_lp copy); X: x_dt in
 *   {F32, BF16}, the projection's input; dW: fp32, must not overlap dU or X.
 * math_dt = SRU_BF16: bf16 MFMA with fp32 accumulation on operands rounded
 *   to bf16 (nearest even) as they are loaded; the reduction over L*B may
 *   be split across blocks, the partial sums then added in a fixed order
 *   (bit-reproducible run to run).
 * math_dt = SRU_F32: fp32 arithmetic throughout (bf16 inputs widened).
 * accumulate = 0 overwrites dW, 1 adds to it.
 * workspace: sru_workspace_size(shape, SRU_WS_BWD_WEIGHT, 0) bytes of device
 *   memory, 256-byte aligned (may be NULL when that size is 0); scratch: the
 *   split partial sums, then room for X rounded to bf16, which a bf16 dU with
 *   an fp32 X is multiplied with when the workspace has that room (the same
 *   values the product would round X to; a smaller workspace that still
 *   holds the partial sums is accepted and takes the product without it).
 */
sru_status sru_project_bwd_weight(const sru_shape *shape,
                                  const void *dU, sru_dtype du_dt,
                                  const void *X, sru_dtype x_dt,
                                  float *dW, sru_dtype math_dt, int32_t accumulate,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Factorised projection (SRU++ paper, Fig. 2(b), and the output projection of
 * its attention layer with the attention weight alpha = 0):
 *   Q = X~ Wq^T (inner dimension d_inner = d' < d), U = Q~ Wo^T,
 * so Wo Wq takes the place of Eq. 1's W.  Each call is one product of the
 * forward or of the input-side backward (layouts in sru_fact_op; Q and dQ are
 * [L*B, d'] row-major, the other tensors as for sru_project).  The backward
 * chain: dQ = dU Wo, then dX = dQ Wq (accumulate = 1 onto sru_backward's dx
 * gives the full input gradient).
 * w_dt = SRU_BF16: bf16 MFMA with fp32 accumulation; A (fp32 or bf16) is
 *   rounded to bf16 (nearest even) as it is loaded ("~" above).
 * w_dt = SRU_F32: fp32 arithmetic throughout (A widened if bf16).
 * C is fp32 and must not overlap A or W.  accumulate = 0 overwrites C, 1
 * adds to it.  d_inner >= 1.
 */
sru_status sru_project_factored(const sru_shape *shape, int64_t d_inner, sru_fact_op op,
                                const void *A, sru_dtype a_dt,
                                const void *W, sru_dtype w_dt,
                                float *C, int32_t accumulate, void *stream);

/*
 * Weight gradients of the factorised projection (chain rule through both
 * products): which = SRU_FACT_WGRAD_Q: dWq (+)= dQ^T X~, G = dQ [L*B, d'],
 * Y = X [L*B, d]; SRU_FACT_WGRAD_O: dWo (+)= dU^T Q~, G = dU [L*B, ndir*3d],
 * Y = Q [L*B, d'].  Arithmetic, accumulation, reproducibility and the
 * workspace as for sru_project_bwd_weight; the workspace size is
 * sru_workspace_size(shape, SRU_WS_FACTORED_WEIGHT, d_inner).
 */
sru_status sru_project_factored_bwd_weight(const sru_shape *shape, int64_t d_inner,
                                           sru_fact_wgrad_op which,
                                           const void *G, sru_dtype g_dt,
                                           const void *Y, sru_dtype y_dt,
                                           float *dW, sru_dtype math_dt, int32_t accumulate,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream);

/*
 * The U-producer of an SRU++ layer (SRU++ paper, section on SRU++): single
 * head scaled dot-product attention, then the output projection:
 *   Q = X~ Wq^T                         Q  fp32 [L*B, d'] (written)
 *   [K | V] = Q~ [Wk; Wv]^T             KV bf16 [Lm + L, B, 2d']: rows t < Lm
 *                                       are read (the previous segment's keys
 *                                       and values, context the paper's
 *                                       training carries over); rows Lm + t
 *                                       are written for this segment's steps
 *   A_b = softmax(Q~_b K~_b^T / sqrt(d')) V~_b   per sequence b, with the
 *                                       visibility of sru_attn_cfg.causal
 *   R = Q + alpha A, or layernorm(Q + alpha A) (biased variance, gain gamma,
 *       shift beta, both fp32 [d'])    R  fp32 [L*B, d'] (written)
 *   U = R~ Wo^T                         U  [L, B, ndir, 3, d] (written), fp32,
 *                                          or bf16 (u_dt; rounded to nearest
 *                                          even from the fp32 sum) as the bf16
 *                                          U that sru_forward takes
 * X [L*B, d] fp32 or bf16 (x_dt).  Wq [d', d], Wkv [2d', d'] (Wk's rows, then
 * Wv's), Wo [ndir*3d, d']: bf16 only.  "~" marks operands rounded to bf16
 * (nearest even) as the bf16 MFMA products load them; the attention weights
 * are rounded to bf16 before they multiply V.  The softmax and the
 * residual / normalisation are fp32.  For d' in {64, 128, 256, 512} the
 * scores never leave the chip: the weights are then exp(s - m) for a running
 * maximum m that is raised in steps (so each lies in [0, 2^8]), rounded to
 * bf16, and A is their product with V divided by the sum of the same rounded
 * weights; other d' normalise the weights before rounding them.
 * gamma, beta: required when cfg->layernorm, else ignored (may be NULL).
 * workspace: sru_attention_workspace_size(shape, cfg) bytes, 256-byte
 *   aligned: for d' in {64, 128, 256, 512} a transposed copy of V (bf16, the
 *   keys padded to a multiple of 32) and R~ (R rounded to bf16, the operand
 *   of the U product); otherwise the scores [B, L, Lm + L] (fp32), the
 *   weights (bf16) and A.
 * Outputs must not overlap each other or the inputs.
 */
sru_status sru_attention_forward(const sru_shape *shape, const sru_attn_cfg *cfg,
                                 const void *X, sru_dtype x_dt,
                                 const void *Wq, const void *Wkv, const void *Wo,
                                 const float *gamma, const float *beta,
                                 float *Q, void *KV, float *R, void *U, sru_dtype u_dt,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of sru_attention_forward; 0 on invalid arguments
 * (sru_last_error() says why). */
size_t sru_attention_workspace_size(const sru_shape *shape, const sru_attn_cfg *cfg);

/*
 * Backward of sru_attention_forward (the chain rule through it; the paper
 * trains the attention, its alpha and the layer norm end to end, section on
 * SRU++): given dU, the gradient of the forward's U, writes
 *   dX [L*B, d]           the input gradient (accumulate_dx = 1 adds it to
 *                         dX, e.g. onto the highway dx of sru_backward, the
 *                         layer input being shared)
 *   dWq [d', d], dWkv [2d', d'] (Wk's rows, then Wv's), dWo [ndir*3d, d']
 *   dalpha (one float), and when cfg->layernorm dgamma, dbeta [d']
 * all fp32, overwritten, in device memory.  The previous segment's keys and
 * values (KV's first mem_len rows) are treated as constants: no gradient
 * flows into them.
 * Inputs: the forward's X, weights, gamma (beta is not needed) and its
 * outputs Q, KV, R, unchanged; dU [L*B, ndir*3d] fp32 or bf16 (du_dt).  The
 * weights, attention and A are recomputed from Q and KV.  Every product
 * rounds its operands to bf16 as it loads them (bf16 MFMA, fp32 sums); the
 * softmax, normalisation and residual gradients are fp32.  The rounding is
 * passed through as the identity.  dalpha, dgamma and dbeta are sums added
 * in a fixed order (bit-reproducible run to run).
 * cfg->d_inner <= 1024 (SRU_ERR_UNSUPPORTED above).
 * workspace: sru_attention_backward_workspace_size(shape, cfg) bytes,
 * 256-byte aligned; scratch.  Outputs must not overlap each other or the
 * inputs.
 */
sru_status sru_attention_backward(const sru_shape *shape, const sru_attn_cfg *cfg,
                                  const void *X, sru_dtype x_dt,
                                  const void *Wq, const void *Wkv, const void *Wo,
                                  const float *gamma,
                                  const float *Q, const void *KV, const float *R,
                                  const void *dU, sru_dtype du_dt,
                                  float *dX, int32_t accumulate_dx,
                                  float *dWq, float *dWkv, float *dWo,
                                  float *dalpha, float *dgamma, float *dbeta,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of sru_attention_backward; 0 on invalid arguments. */
size_t sru_attention_backward_workspace_size(const sru_shape *shape, const sru_attn_cfg *cfg);

/*
 * One step of a unidirectional layer for decoding: the recurrence run as an
 * RNN at inference ("Parallelizing Legendre Memory Unit Training", abstract),
 * i.e. Eq. 1 and Eqs. 2-5 for a single time step with the state carried
 * between calls (SRU++ paper, background section):
 *   u = x~ W^T for the step's B rows, then per channel
 *   c_next = f c_prev + (1 - f) u_cand, h = r c_next + (1 - r) alpha x.
 * shape->L must be 1 and shape->bidirectional 0 (a decoding step sees no
 * future input).  x [B, d] fp32 or bf16; W [3d, d] fp32 or bf16 (the same
 * weights as sru_project); v, b fp32 [2, d]; c_prev fp32 [B, d] or NULL
 * (zero state); h, c_next fp32 [B, d].  With bf16 W, x is rounded to bf16
 * (nearest even) for the product, as in sru_project; the highway term uses
 * x.  The products are fp32 sums.  c_next may be the same buffer as c_prev
 * (the state updated in place); no other output may overlap an input or the
 * other output.
 */
sru_status sru_step(const sru_shape *shape,
                    const void *x, sru_dtype x_dt,
                    const void *W, sru_dtype w_dt,
                    const float *v, const float *b, const float *c_prev,
                    float *h, float *c_next, void *stream);

/*
 * Forward recurrence, Eqs. 2-5, for every (direction, batch, channel) chain.
 *   U: u_dt in {F32, BF16}; x: x_dt in {F32, BF16}; v, b, c0: fp32.
 *   c0 may be NULL (zero initial state).
 *   h: fp32 (h_dt must be SRU_F32).
 *   c_seq: fp32 or NULL (needed only when a backward pass follows).
 *   c_last: fp32 or NULL.
 * State and arithmetic are fp32.
 */
sru_status sru_forward(const sru_shape *shape,
                       const void *U, sru_dtype u_dt,
                       const void *x, sru_dtype x_dt,
                       const float *v, const float *b, const float *c0,
                       void *h, sru_dtype h_dt,
                       float *c_seq, float *c_last,
                       void *stream);

/*
 * Backward recurrence: the chain rule through Eqs. 2-5, walking each chain
 * in the reverse of its direction's order (the pages give no backward; it
 * is derived).  Needs the forward's c_seq.
 *   dh: fp32 [L, B, ndir, d] (required); dc_last: fp32 or NULL (zero).
 *   dU: fp32 [L, B, ndir, 3, d] (required, overwritten).
 *   dU_lp: bf16 [L, B, ndir, 3, d] or NULL: a copy of dU rounded to bf16
 *       (nearest even), i.e. exactly the operand the bf16 backward-data
 *       projection multiplies; passing it as A there halves that GEMM's
 *       operand bytes.
 *   dx: fp32 [L, B, d] (required, overwritten): the highway part
 *       alpha (1 - r) dh summed over directions.  The part through the
 *       projection comes from sru_project(SRU_PROJ_BWD_DATA, accumulate = 1).
 *   dv, db: fp32 [ndir, 2, d] or NULL (overwritten; summed over t and b in
 *       a fixed order, so results are bit-reproducible run to run).
 *   dc0: fp32 [ndir, B, d] or NULL.
 *   workspace: at least sru_workspace_size(shape, SRU_WS_BACKWARD, 0) bytes
 *       of device memory, 256-byte aligned; scratch, except for its error
 *       word (SRU_WS_ERROR_OFFSET below).
 * For longer sequences the backward runs as a chunked scan of the state's
 * adjoint, in which each chunk takes its incoming adjoint from the chunk
 * after it through the workspace (a bounded wait); the error word reports a
 * wait that ran out.
 */
sru_status sru_backward(const sru_shape *shape,
                        const void *U, sru_dtype u_dt,
                        const void *x, sru_dtype x_dt,
                        const float *v, const float *b, const float *c0,
                        const float *c_seq, const float *dh, const float *dc_last,
                        float *dU, void *dU_lp, float *dx, float *dv, float *db, float *dc0,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * sru_backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight training loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results (bit for bit) as sru_backward,
 * with its scratch in a static device array of the library instead of a
 * caller workspace.
 *   The array holds SRU_BACKWARD_STATIC_SCRATCH_BYTES (16 MiB) per GPU; it
 *   is created the first time the library's code runs on that GPU and kept
 *   until the process ends.  Shapes whose sru_workspace_size(shape,
 *   SRU_WS_BACKWARD, 0) exceeds it are rejected with SRU_ERR_WORKSPACE
 *   (e.g. L = 512, B = 32, d = 1024 needs 6.3 MB and fits).
 *   Every call on one GPU uses that GPU's one array: calls that overlap in
 *   time on one GPU (other streams, other threads) race and give undefined
 *   results; calls ordered on one stream are safe.  Each call clears what it
 *   needs; nothing carries over between calls.
 *   error_word: device pointer to a 32-bit word (4-byte aligned) or NULL.
 *   When given, it is cleared by the call and set nonzero if a bounded wait
 *   between chunks ran out (then the outputs are invalid), as the error word
 *   of sru_backward's workspace is.
 *   Nothing here calls hipMalloc or hipFree; all other arguments are those of
 *   sru_backward.
 */
#define SRU_BACKWARD_STATIC_SCRATCH_BYTES (16u << 20)
sru_status sru_backward_static(const sru_shape *shape,
                               const void *U, sru_dtype u_dt,
                               const void *x, sru_dtype x_dt,
                               const float *v, const float *b, const float *c0,
                               const float *c_seq, const float *dh, const float *dc_last,
                               float *dU, void *dU_lp, float *dx, float *dv, float *db,
                               float *dc0, uint32_t *error_word, void *stream);

/*
 * Linear mode (v = v' = 0): f and r depend on U only, so c[t] =
 * a[t] c[t-1] + (1 - a[t]) U[t,2] is a first-order linear recurrence and is
 * evaluated as a scan over time chunks of `chunk` steps (per chunk: local scan
 * and its aggregate, then the carry between chunks, then the chunk's outputs).
 * The result equals the sequential recurrence up to rounding for any chunk.
 * ("Parallelizing Legendre Memory Unit Training", abstract: linear recurrent
 * components can be trained in parallel and run as an RNN at inference.)
 *   pass = SRU_FWD: reads U, x, b, c0 (nullable); writes h (fp32), c_seq
 *     (nullable), c_last (nullable).  dh .. dc0 must be NULL or are ignored.
 *   pass = SRU_BWD: reads U, x, b, c0 (nullable), c_seq (required), dh
 *     (required), dc_last (nullable); writes dU (required), dx (required,
 *     highway part summed over directions), db (nullable), dc0 (nullable).
 *     h and c_last are ignored.
 *   chunk >= 1.  workspace: sru_workspace_size(shape, SRU_WS_LINEAR_FWD or
 *   SRU_WS_LINEAR_BWD, chunk) bytes, 256-byte aligned.
 * With chunk == 256 and d % 64 == 0 the three steps run as one kernel per
 * direction: each chunk takes its incoming state from the preceding chunk
 * through the workspace (a bounded wait); the error word reports a wait that
 * ran out (SRU_WS_ERROR_OFFSET below).
 */
sru_status sru_linear_scan(const sru_shape *shape, sru_pass pass, int32_t chunk,
                           const void *U, sru_dtype u_dt,
                           const void *x, sru_dtype x_dt,
                           const float *b, const float *c0,
                           void *h, sru_dtype h_dt, float *c_seq, float *c_last,
                           const float *dh, const float *dc_last,
                           float *dU, float *dx, float *db, float *dc0,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Wt[d, ndir*3d] = W[ndir*3d, d]^T, for SRU_PROJ_BWD_DATA_WT (the weights
 * of Eq. 1 laid out with the reduction index of the backward-data product
 * contiguous).  w_dt gives the element type of both (bf16 or fp32).  W and
 * Wt must not overlap.
 */
sru_status sru_transpose_weight(const sru_shape *shape, const void *W, sru_dtype w_dt,
                                void *Wt, void *stream);

/*
 * dst[i] = bf16(src[i]) for i < n, rounded to nearest even: the operand X~ of
 * Eq. 1 (SRU++ paper, background section) as the bf16 projection multiplies
 * it.  A caller that keeps X~ hands it to sru_project (half the bytes of fp32
 * X, the same product) and to sru_project_bwd_weight (the same X~ the
 * gradient needs).  src fp32, dst bf16, both 16-byte aligned, not
 * overlapping; n >= 1.
 */
sru_status sru_round_bf16(int64_t n, const float *src, void *dst, void *stream);

/*
 * The error word of sru_backward and sru_linear_scan: the 32-bit word at
 * byte offset SRU_WS_ERROR_OFFSET of the workspace passed to the call (the
 * first 256 bytes of those workspaces are a control block).  Every such call
 * clears it before its first kernel runs; once the call's work has completed
 * (after the caller synchronises with `stream`) it is 0, or nonzero if a
 * bounded wait between chunks ran out, in which case that call's outputs are
 * invalid.  The kernels stop waiting rather than hang, so the call still
 * completes.  The word keeps its value until the next call on that workspace.
 */
#define SRU_WS_ERROR_OFFSET 0

/* Workspace bytes needed by `op` for `shape` (and `chunk`: the chunk length
 * for the linear mode, the inner dimension d' for SRU_WS_FACTORED_WEIGHT);
 * 0 either when none is needed or on invalid arguments (then
 * sru_last_error() is not empty and says why). */
size_t sru_workspace_size(const sru_shape *shape, sru_ws_op op, int32_t chunk);

/* Static text for a status code. */
const char *sru_status_string(sru_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *sru_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SRU_H_ */

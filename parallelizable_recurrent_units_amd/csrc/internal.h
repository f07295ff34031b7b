// internal.h -- launcher interfaces between the C-ABI layer and the kernels.
// Host-side only types; nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sru {

typedef uint16_t bf16_bits_t;

// Every workspace of sru_backward and sru_linear_scan starts with a control
// block of kCtrlWords 32-bit words (256 bytes): word kErrWord is the call's
// error word (cleared by every call; nonzero after it only if a bounded
// look-back wait between chunks ran out), word kTicketWord the chunk ticket
// of the single-pass scans.  The kernels' own data follows at byte 256.
constexpr int64_t kCtrlWords = 64;
constexpr int64_t kErrWord = 0, kTicketWord = 4;

// Arguments of the forward / backward recurrence launchers.  Element counts
// and offsets are int64; layouts are those of include/sru.h.
struct RecArgs {
    int64_t L, B, d;
    int ndir;
    float alpha;
    const void *U;
    bool u_bf16;
    const void *x;
    bool x_bf16;
    const float *v, *b, *c0;
    // forward outputs
    float *h, *c_seq, *c_last;
    // backward
    const float *c_seq_in, *dh, *dc_last;
    float *dU, *dx, *dc0;
    bf16_bits_t *dU_lp;  // optional bf16 copy of dU (nearest even)
    float *partials;     // [ndir, B, 4, d] per-chain sums over t
    uint32_t *err_word;  // the workspace's error word: zeroed by the kernels
                         // that have no look-back (nothing else writes it)
    int dir;             // backward: the one direction this launch walks
    bool dx_accumulate;  // backward: add to dx instead of overwriting
};

hipError_t launch_forward(const RecArgs &a, hipStream_t s);
// One direction per call (a.dir); writes dU, dx (overwrite or accumulate),
// dc0 and the per-chain parameter-gradient partials.
hipError_t launch_backward_dir(const RecArgs &a, hipStream_t s);
// Both directions in one launch (ndir == 2, short fp32 sequences): writes dU,
// dx (overwritten), dc0 and the partials.
bool backward_bidi_ok(const RecArgs &a);
hipError_t launch_backward_bidi(const RecArgs &a, hipStream_t s);
// The backward as a chunked scan of the adjoint (d % 64 == 0, sizes within
// 32-bit segment offsets; with fp32 U and x only for longer sequences): both
// directions, dv/db included.  ws holds
// backward_scan_workspace_bytes(L, B, d, ndir) bytes.
bool backward_scan_ok(int64_t L, int64_t B, int64_t d, int ndir, bool fp32_inputs);
size_t backward_scan_workspace_bytes(int64_t L, int64_t B, int64_t d, int ndir);
hipError_t launch_backward_scan(const RecArgs &a, void *ws, float *dv, float *db, hipStream_t s);
// dv, db [ndir, 2, d] = sum over b (increasing) of partials.
hipError_t launch_param_reduce(const float *partials, int64_t B, int64_t d, int ndir,
                               float *dv, float *db, hipStream_t s);

struct LinArgs {
    int64_t L, B, d;
    int ndir;
    float alpha;
    int64_t chunk;
    const void *U;
    bool u_bf16;
    const void *x;
    bool x_bf16;
    const float *b, *c0;
    float *h, *c_seq, *c_last;
    const float *dh, *dc_last;
    float *dU, *dx, *db, *dc0;
    void *ws;
};

size_t linear_workspace_bytes(int64_t L, int64_t B, int64_t d, int ndir, int64_t chunk,
                              bool backward);
hipError_t launch_linear_forward(const LinArgs &a, hipStream_t s);
hipError_t launch_linear_backward(const LinArgs &a, hipStream_t s);

// C[M, N] (+)= A[M, K] . op(B)
//   b_kn = false: B stored [N, K] (C = A B^T)     -- projection forward
//   b_kn = true : B stored [K, N] (C = A B)       -- projection backward-data
// Row strides lda, ldb, ldc (elements; 0 = dense) and `batch` independent
// products whose operands start sa, sb, sc elements apart.
struct GemmArgs {
    int64_t M, N, K;
    const void *A;
    bool a_bf16;
    const void *Bm;
    bool b_bf16;
    bool b_kn;
    float *C;
    bool accumulate;
    int64_t lda = 0, ldb = 0, ldc = 0;
    int64_t batch = 1, sa = 0, sb = 0, sc = 0;
    // Causal products, where row m of C sees columns n <= c + m (-1: off).
    // causal_skip = c: tiles with no such column may be left unwritten (their
    // C is never read).  causal_klim = c: A's row m holds zeros past
    // k = c + m, so a row tile's reduction may stop there.  Hints: only the
    // kernels that copy bf16 operands straight into LDS use them.
    int64_t causal_skip = -1, causal_klim = -1;
};

// bf16 B: bf16 MFMA (A rounded to bf16 as it is loaded); fp32 B: fp32 FMA.
hipError_t launch_gemm(const GemmArgs &g, hipStream_t s);
// As launch_gemm for fp32 or bf16 A, bf16 B given as [N, K], no
// accumulation, with C written as bf16 (rounded to nearest even); C points to
// bf16 storage.  For bf16 A the product takes the same kernel as launch_gemm
// would for the same operands, so the bf16 C is the fp32 C rounded.
hipError_t launch_gemm_bf16_out(const GemmArgs &g, hipStream_t s);
// C[M, N] (+)= A^T B with A given as [K, M] and B as [K, N] (each bf16 or
// fp32): the weight gradient dW = dU^T Xt.  f32_math: fp32 FMA throughout;
// otherwise bf16 MFMA on operands rounded to bf16 while staged, with the
// reduction over K split across blocks when the output alone would not
// fill the chip (ws then holds the partial products).
size_t wgrad_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Bytes after the partial sums that hold a bf16 copy of an fp32 B when
// launch_gemm_wgrad is given b_copy (0 where the copy would not be used: the
// product then keeps the register-staged kernel).  With b_copy the
// workspace must hold wgrad_workspace_bytes rounded up to 256, then these.
size_t wgrad_b_copy_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_wgrad(const GemmArgs &g, bool f32_math, float *ws, hipStream_t s,
                             bool b_copy = false);
// C[M, N] (+)= A^T B with A given as [K, M] and B as [K, N] (bf16 or fp32
// each, rounded to bf16 while staged; row strides and batches as in
// GemmArgs), bf16 MFMA, no split of the reduction and no workspace.
hipError_t launch_gemm_tn(const GemmArgs &g, hipStream_t s);
// As launch_gemm_tn for bf16 A and B, no accumulation, with C written as bf16
// (rounded to nearest even; C points to bf16 storage, row stride ldc): the
// same kernel and products as launch_gemm_tn, so the bf16 C is its fp32 C
// rounded.
hipError_t launch_gemm_tn_bf16_out(const GemmArgs &g, hipStream_t s);
// The SRU++ attention U-producer (attention.hip); layouts as in sru.h.
struct AttnArgs {
    int64_t L, B, d, dp, Lm, n3;   // n3 = ndir * 3 * d
    int causal, layernorm;
    float alpha, eps;
    const void *X;
    bool x_bf16;
    const bf16_bits_t *Wq, *Wkv, *Wo;
    const float *gamma, *beta;
    float *Q, *R;
    void *U;                       // fp32, or bf16 when u_bf16
    bool u_bf16;
    void *KV;                      // bf16 [Lm + L, B, 2 dp]
    void *workspace;               // attention_workspace_bytes
};
size_t attention_workspace_bytes(int64_t L, int64_t B, int64_t dp, int64_t Lm);
hipError_t launch_attention_forward(const AttnArgs &a, hipStream_t s);

// Its backward (attention.hip): the forward's Q, KV and R plus dU in; dX and
// the parameter gradients out.  Layouts as in sru.h.
constexpr int64_t kAttnBwdMaxInner = 1024;   // d' the row kernels hold in registers
struct AttnBwdArgs {
    int64_t L, B, d, dp, Lm, n3;
    int causal, layernorm;
    float alpha, eps;
    const void *X;
    bool x_bf16;
    const bf16_bits_t *Wq, *Wkv, *Wo;
    const float *gamma;
    const float *Q, *R;
    const bf16_bits_t *KV;
    const void *dU;
    bool du_bf16;
    float *dX;
    bool dx_accumulate;
    float *dWq, *dWkv, *dWo, *dalpha, *dgamma, *dbeta;
    void *workspace;
};
size_t attention_backward_workspace_bytes(int64_t L, int64_t B, int64_t d, int64_t dp,
                                          int64_t Lm, int64_t n3);
hipError_t launch_attention_backward(const AttnBwdArgs &a, hipStream_t s);

// One decoding step of a unidirectional layer (step.hip).
struct StepArgs {
    int64_t B, d;
    const void *x, *W;             // x [B, d]; W [3d, d]
    bool x_bf16, w_bf16;
    const float *v, *b;            // [2, d]
    const float *c_prev;           // [B, d] or null (zero state)
    float *h, *c_next;             // [B, d]; c_next may be c_prev
    float alpha;
};
hipError_t launch_step(const StepArgs &a, hipStream_t s);

// dst[i] = bf16(src[i]), nearest even (dst: 2-byte elements).
hipError_t launch_round_bf16(int64_t n, const float *src, void *dst, hipStream_t s);
// dst[cols, rows] = src[rows, cols]^T (2-byte or 4-byte elements).
hipError_t launch_transpose(int64_t rows, int64_t cols, const void *src, void *dst, bool two_byte,
                            hipStream_t s);

}  // namespace sru

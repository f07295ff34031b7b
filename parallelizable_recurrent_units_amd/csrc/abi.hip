// abi.hip -- the C entry points declared in include/sru.h: argument
// validation, dtype dispatch, workspace sizing and launches on the caller's
// stream.  Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/sru.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

sru_status fail(sru_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

sru_status ok()
{
    g_last_error[0] = '\0';
    return SRU_OK;
}

constexpr int64_t kMaxElems = (int64_t)1 << 56;   // far below int64 overflow
constexpr int64_t kMaxBlocks = ((int64_t)1 << 31) - 1;

bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > kMaxElems / a) return false;
    *out = a * b;
    return true;
}

// Validates the shape; fills ndir and the element counts used below.
struct Dims {
    int ndir;
    int64_t LB, chains, u_elems;
};

sru_status check_shape(const sru_shape *s, Dims *dm)
{
    if (!s) return fail(SRU_ERR_INVALID_ARG, "shape is NULL");
    if (s->L < 1 || s->B < 1 || s->d < 1)
        return fail(SRU_ERR_INVALID_ARG, "L, B, d must be >= 1 (got L=%lld B=%lld d=%lld)",
                    (long long)s->L, (long long)s->B, (long long)s->d);
    if (s->bidirectional != 0 && s->bidirectional != 1)
        return fail(SRU_ERR_INVALID_ARG, "bidirectional must be 0 or 1 (got %d)",
                    (int)s->bidirectional);
    if (!isfinite(s->alpha)) return fail(SRU_ERR_INVALID_ARG, "alpha must be finite");
    dm->ndir = s->bidirectional ? 2 : 1;
    int64_t lbd, x3;
    if (!mul_ok(s->L, s->B, &dm->LB) || !mul_ok(dm->LB, s->d, &lbd) ||
        !mul_ok(lbd, 3 * dm->ndir, &dm->u_elems) || !mul_ok(s->B, s->d, &x3))
        return fail(SRU_ERR_INVALID_ARG, "tensor sizes overflow");
    dm->chains = x3 * dm->ndir;
    // the widest grids: one thread per chain (256 per block) and one wave
    // per 64 chains; both far below the grid limit for any legal size here.
    if ((dm->chains + 63) / 64 > kMaxBlocks)
        return fail(SRU_ERR_INVALID_ARG, "too many chains for one launch");
    return SRU_OK;
}

bool valid_dtype(int d) { return d == SRU_F32 || d == SRU_BF16; }

sru_status need_ptr(const void *p, const char *name)
{
    if (!p) return fail(SRU_ERR_INVALID_ARG, "%s must not be NULL", name);
    if (((uintptr_t)p) & 15u)
        return fail(SRU_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
    return SRU_OK;
}

sru_status opt_ptr(const void *p, const char *name)
{
    if (p && (((uintptr_t)p) & 15u))
        return fail(SRU_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
    return SRU_OK;
}

#define SRU_TRY(expr)                       \
    do {                                    \
        sru_status st_ = (expr);            \
        if (st_ != SRU_OK) return st_;      \
    } while (0)

sru_status need_device()
{
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return fail(SRU_ERR_NO_DEVICE, "no HIP device available (%s)",
                    e != hipSuccess ? hipGetErrorString(e) : "device count is 0");
    }
    return SRU_OK;
}

sru_status launched(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(SRU_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// The chunked-scan layout bounds the one-lane-per-chain layout
// ([ndir, B, 4, d] partials) of the generic kernels.
size_t backward_ws(const sru_shape *s, const Dims &dm)
{
    return round256(sru::backward_scan_workspace_bytes(s->L, s->B, s->d, dm.ndir));
}

// The projection-shaped products of the factorised projection and of the
// weight gradients: C[M, N] (+)= op(A) op(B) in one of three layouts.
enum class Layout {
    NT,   // A [M, K], B [N, K]
    NN,   // A [M, K], B [K, N]
    TN    // A [K, M], B [K, N] (the weight gradients)
};

size_t elem_bytes(sru_dtype t) { return t == SRU_BF16 ? 2 : 4; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// A device buffer as the checks below see it: base, bytes, name.  A NULL
// pointer or a zero size is skipped.
struct Span {
    const void *p;
    size_t n;
    const char *name;
};

// Fails when a written buffer overlaps another written buffer or any input.
sru_status no_overlap(const Span *out, int nout, const Span *in, int nin)
{
    for (int i = 0; i < nout; ++i) {
        if (!out[i].p || !out[i].n) continue;
        for (int j = i + 1; j < nout; ++j)
            if (out[j].p && out[j].n && overlaps(out[i].p, out[i].n, out[j].p, out[j].n))
                return fail(SRU_ERR_INVALID_ARG, "%s overlaps %s", out[i].name, out[j].name);
        for (int j = 0; j < nin; ++j)
            if (in[j].p && in[j].n && overlaps(out[i].p, out[i].n, in[j].p, in[j].n))
                return fail(SRU_ERR_INVALID_ARG, "%s overlaps %s", out[i].name, in[j].name);
    }
    return SRU_OK;
}

// Workspace a product needs (the weight gradient's partial sums) ...
size_t product_ws(Layout lay, int64_t M, int64_t N, int64_t K)
{
    return lay == Layout::TN ? round256(sru::wgrad_workspace_bytes(M, N, K)) : 0;
}
// ... and what the workspace queries report: room for a bf16 copy of an
// fp32 B as well, which the weight gradient uses when it is given that much
size_t product_ws_query(Layout lay, int64_t M, int64_t N, int64_t K)
{
    return product_ws(lay, M, N, K) + (lay == Layout::TN ? sru::wgrad_b_copy_bytes(M, N, K) : 0);
}

// Validates and launches one product.  bf16 math: MFMA on operands rounded
// to bf16 as they are loaded (B must be bf16 unless the layout is TN); fp32
// math: fp32 FMA on widened operands.  C is fp32 and must not overlap A or B.
sru_status run_product(Layout lay, int64_t M, int64_t N, int64_t K, const void *A,
                       sru_dtype a_dt, const char *a_name, const void *B, sru_dtype b_dt,
                       const char *b_name, float *C, const char *c_name, sru_dtype math_dt,
                       int32_t accumulate, void *workspace, size_t workspace_bytes,
                       hipStream_t stream, const char *what)
{
    if (!valid_dtype(a_dt) || !valid_dtype(b_dt) || !valid_dtype(math_dt))
        return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    if (accumulate != 0 && accumulate != 1)
        return fail(SRU_ERR_INVALID_ARG, "accumulate must be 0 or 1");
    SRU_TRY(need_ptr(A, a_name));
    SRU_TRY(need_ptr(B, b_name));
    SRU_TRY(need_ptr(C, c_name));
    const bool f32_math = math_dt == SRU_F32;
    if (lay != Layout::TN && f32_math != (b_dt == SRU_F32))
        return fail(SRU_ERR_UNSUPPORTED, "%s: the weight dtype selects the arithmetic", what);
    int64_t ae, be, ce;
    if (!mul_ok(M, K, &ae) || !mul_ok(N, K, &be) || !mul_ok(M, N, &ce))
        return fail(SRU_ERR_INVALID_ARG, "%s: tensor sizes overflow", what);
    // grids: fp32 kernel x over M / 64 (y over N / 64 <= 65535); MFMA kernels
    // one dimension over (M / 128) x (N / 128) tiles; the split reduction
    // over M x N / 256
    if ((M + 63) / 64 > kMaxBlocks || (N + 63) / 64 > 65535 || (ce + 255) / 256 > kMaxBlocks)
        return fail(SRU_ERR_INVALID_ARG, "%s: matrix too large for one launch", what);
    if (overlaps(C, (size_t)ce * 4, A, (size_t)ae * elem_bytes(a_dt)) ||
        overlaps(C, (size_t)ce * 4, B, (size_t)be * elem_bytes(b_dt)))
        return fail(SRU_ERR_INVALID_ARG, "%s: %s overlaps %s or %s", what, c_name, a_name, b_name);
    const size_t need = f32_math ? 0 : product_ws(lay, M, N, K);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(SRU_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need,
                        workspace_bytes, workspace ? "" : ", NULL");
        SRU_TRY(opt_ptr(workspace, "workspace"));
    }
    SRU_TRY(need_device());
    sru::GemmArgs g;
    g.M = M;
    g.N = N;
    g.K = K;
    g.A = A;
    g.a_bf16 = a_dt == SRU_BF16;
    g.Bm = B;
    g.b_bf16 = b_dt == SRU_BF16;
    g.b_kn = lay != Layout::NT;
    g.C = C;
    g.accumulate = accumulate != 0;
    if (lay == Layout::TN) {
        const bool b_copy = workspace && workspace_bytes >= product_ws_query(lay, M, N, K);
        return launched(sru::launch_gemm_wgrad(g, f32_math, (float *)workspace, stream, b_copy),
                        what);
    }
    return launched(sru::launch_gemm(g, stream), what);
}

}  // namespace

extern "C" {

const char *sru_status_string(sru_status st)
{
    switch (st) {
    case SRU_OK: return "SRU_OK";
    case SRU_ERR_INVALID_ARG: return "SRU_ERR_INVALID_ARG";
    case SRU_ERR_UNSUPPORTED: return "SRU_ERR_UNSUPPORTED";
    case SRU_ERR_NO_DEVICE: return "SRU_ERR_NO_DEVICE";
    case SRU_ERR_LAUNCH: return "SRU_ERR_LAUNCH";
    case SRU_ERR_WORKSPACE: return "SRU_ERR_WORKSPACE";
    }
    return "SRU_ERR_UNKNOWN";
}

const char *sru_last_error(void) { return g_last_error; }

size_t sru_workspace_size(const sru_shape *shape, sru_ws_op op, int32_t chunk)
{
    Dims dm;
    if (check_shape(shape, &dm) != SRU_OK) return 0;
    switch (op) {
    case SRU_WS_BACKWARD:
        ok();
        return backward_ws(shape, dm);
    case SRU_WS_LINEAR_FWD:
    case SRU_WS_LINEAR_BWD:
        if (chunk < 1) {
            fail(SRU_ERR_INVALID_ARG, "chunk must be >= 1 (got %d)", (int)chunk);
            return 0;
        }
        ok();
        return round256(sru::linear_workspace_bytes(shape->L, shape->B, shape->d, dm.ndir,
                                                    chunk, op == SRU_WS_LINEAR_BWD));
    case SRU_WS_BWD_WEIGHT:
        ok();
        return product_ws_query(Layout::TN, 3 * dm.ndir * shape->d, shape->d, dm.LB);
    case SRU_WS_FACTORED_WEIGHT: {
        const int64_t di = chunk;   // the inner dimension d'
        if (di < 1) {
            fail(SRU_ERR_INVALID_ARG, "the inner dimension must be >= 1 (got %d)", (int)chunk);
            return 0;
        }
        const size_t a = product_ws_query(Layout::TN, di, shape->d, dm.LB);
        const size_t b = product_ws_query(Layout::TN, 3 * dm.ndir * shape->d, di, dm.LB);
        ok();
        return a > b ? a : b;
    }
    }
    fail(SRU_ERR_INVALID_ARG, "unknown workspace op %d", (int)op);
    return 0;
}

sru_status sru_project(const sru_shape *shape, sru_proj_op op, const void *A, sru_dtype a_dt,
                       const void *W, sru_dtype w_dt, void *C, sru_dtype c_dt,
                       int32_t accumulate, void *stream)
{
    Dims dm;
    SRU_TRY(check_shape(shape, &dm));
    if (op != SRU_PROJ_FWD && op != SRU_PROJ_BWD_DATA && op != SRU_PROJ_BWD_DATA_WT)
        return fail(SRU_ERR_INVALID_ARG, "unknown projection op %d", (int)op);
    if (!valid_dtype(a_dt) || !valid_dtype(w_dt) || !valid_dtype(c_dt))
        return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    if (accumulate != 0 && accumulate != 1)
        return fail(SRU_ERR_INVALID_ARG, "accumulate must be 0 or 1");
    SRU_TRY(need_ptr(A, "A"));
    SRU_TRY(need_ptr(W, "W"));
    SRU_TRY(need_ptr(C, "C"));
    if (c_dt != SRU_F32) return fail(SRU_ERR_UNSUPPORTED, "C must be fp32");
    // grid: x over row tiles (>= 64 rows each), y over column tiles (<= 65535)
    if ((dm.LB + 63) / 64 > kMaxBlocks || (3 * dm.ndir * shape->d + 63) / 64 > 65535)
        return fail(SRU_ERR_INVALID_ARG, "matrix too large for one projection launch");
    const int64_t n3 = 3 * dm.ndir * shape->d;
    {   // C [L*B, n3 or d] against A [L*B, d or n3] and W (n3 * d elements)
        const size_t lbd = (size_t)(dm.LB * shape->d), lbn = (size_t)dm.u_elems;
        const bool fwd = op == SRU_PROJ_FWD;
        const Span out[] = {{C, (fwd ? lbn : lbd) * 4, "C"}};
        const Span in[] = {{A, (fwd ? lbd : lbn) * elem_bytes(a_dt), "A"},
                           {W, (size_t)(n3 * shape->d) * elem_bytes(w_dt), "W"}};
        SRU_TRY(no_overlap(out, 1, in, 2));
    }
    SRU_TRY(need_device());
    sru::GemmArgs g;
    g.M = dm.LB;
    g.A = A;
    g.a_bf16 = a_dt == SRU_BF16;
    g.Bm = W;
    g.b_bf16 = w_dt == SRU_BF16;
    g.C = (float *)C;
    g.accumulate = accumulate != 0;
    if (op == SRU_PROJ_FWD) {
        g.N = n3;
        g.K = shape->d;
        g.b_kn = false;
    } else {
        g.N = shape->d;
        g.K = n3;
        g.b_kn = op == SRU_PROJ_BWD_DATA;   // the _WT form passes W as [N, K]
    }
    return launched(sru::launch_gemm(g, (hipStream_t)stream), "projection");
}

sru_status sru_project_bwd_weight(const sru_shape *shape, const void *dU, sru_dtype du_dt,
                                  const void *X, sru_dtype x_dt, float *dW, sru_dtype math_dt,
                                  int32_t accumulate, void *workspace, size_t workspace_bytes,
                                  void *stream)
{
    Dims dm;
    SRU_TRY(check_shape(shape, &dm));
    return run_product(Layout::TN, 3 * dm.ndir * shape->d, shape->d, dm.LB, dU, du_dt, "dU", X,
                       x_dt, "X", dW, "dW", math_dt, accumulate, workspace, workspace_bytes,
                       (hipStream_t)stream, "weight gradient");
}

sru_status sru_project_factored(const sru_shape *shape, int64_t d_inner, sru_fact_op op,
                                const void *A, sru_dtype a_dt, const void *W, sru_dtype w_dt,
                                float *C, int32_t accumulate, void *stream)
{
    Dims dm;
    SRU_TRY(check_shape(shape, &dm));
    if (d_inner < 1)
        return fail(SRU_ERR_INVALID_ARG, "the inner dimension must be >= 1 (got %lld)",
                    (long long)d_inner);
    const int64_t d = shape->d, n3 = 3 * dm.ndir * d, LB = dm.LB;
    switch (op) {
    case SRU_FACT_Q:
        return run_product(Layout::NT, LB, d_inner, d, A, a_dt, "X", W, w_dt, "Wq", C, "Q", w_dt,
                           accumulate, nullptr, 0, (hipStream_t)stream, "factored Q");
    case SRU_FACT_U:
        return run_product(Layout::NT, LB, n3, d_inner, A, a_dt, "Q", W, w_dt, "Wo", C, "U", w_dt,
                           accumulate, nullptr, 0, (hipStream_t)stream, "factored U");
    case SRU_FACT_BWD_Q:
        return run_product(Layout::NN, LB, d_inner, n3, A, a_dt, "dU", W, w_dt, "Wo", C, "dQ",
                           w_dt, accumulate, nullptr, 0, (hipStream_t)stream, "factored dQ");
    case SRU_FACT_BWD_X:
        return run_product(Layout::NN, LB, d, d_inner, A, a_dt, "dQ", W, w_dt, "Wq", C, "dX",
                           w_dt, accumulate, nullptr, 0, (hipStream_t)stream, "factored dX");
    }
    return fail(SRU_ERR_INVALID_ARG, "unknown factored op %d", (int)op);
}

sru_status sru_project_factored_bwd_weight(const sru_shape *shape, int64_t d_inner,
                                           sru_fact_wgrad_op which, const void *G,
                                           sru_dtype g_dt, const void *Y, sru_dtype y_dt,
                                           float *dW, sru_dtype math_dt, int32_t accumulate,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream)
{
    Dims dm;
    SRU_TRY(check_shape(shape, &dm));
    if (d_inner < 1)
        return fail(SRU_ERR_INVALID_ARG, "the inner dimension must be >= 1 (got %lld)",
                    (long long)d_inner);
    const int64_t d = shape->d, n3 = 3 * dm.ndir * d, LB = dm.LB;
    switch (which) {
    case SRU_FACT_WGRAD_Q:
        return run_product(Layout::TN, d_inner, d, LB, G, g_dt, "dQ", Y, y_dt, "X", dW, "dWq",
                           math_dt, accumulate, workspace, workspace_bytes, (hipStream_t)stream,
                           "factored dWq");
    case SRU_FACT_WGRAD_O:
        return run_product(Layout::TN, n3, d_inner, LB, G, g_dt, "dU", Y, y_dt, "Q", dW, "dWo",
                           math_dt, accumulate, workspace, workspace_bytes, (hipStream_t)stream,
                           "factored dWo");
    }
    return fail(SRU_ERR_INVALID_ARG, "unknown factored weight gradient %d", (int)which);
}

}  // extern "C"

namespace {

// Validates the attention options and the sizes derived from them.
sru_status check_attn(const sru_shape *shape, const sru_attn_cfg *cfg, Dims *dm)
{
    SRU_TRY(check_shape(shape, dm));
    if (!cfg) return fail(SRU_ERR_INVALID_ARG, "cfg is NULL");
    if (cfg->d_inner < 1)
        return fail(SRU_ERR_INVALID_ARG, "d_inner must be >= 1 (got %lld)",
                    (long long)cfg->d_inner);
    if (cfg->mem_len < 0)
        return fail(SRU_ERR_INVALID_ARG, "mem_len must be >= 0 (got %lld)",
                    (long long)cfg->mem_len);
    if (cfg->causal != 0 && cfg->causal != 1)
        return fail(SRU_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (cfg->layernorm != 0 && cfg->layernorm != 1)
        return fail(SRU_ERR_INVALID_ARG, "layernorm must be 0 or 1");
    if (!isfinite(cfg->attn_alpha)) return fail(SRU_ERR_INVALID_ARG, "attn_alpha must be finite");
    if (cfg->layernorm && !(cfg->ln_eps > 0.0f && isfinite(cfg->ln_eps)))
        return fail(SRU_ERR_INVALID_ARG, "ln_eps must be finite and > 0");
    const int64_t L = shape->L, B = shape->B, dp = cfg->d_inner;
    int64_t lk, s1, s2, kv, q;
    if (!mul_ok(cfg->mem_len + L, B, &lk) || !mul_ok(lk, 2 * dp, &kv) || !mul_ok(dm->LB, dp, &q) ||
        !mul_ok(B * L, cfg->mem_len + L, &s1) || !mul_ok(s1, 4, &s2) ||
        !mul_ok(dp, shape->d, &q) || !mul_ok(3 * dm->ndir * shape->d, dp, &q))
        return fail(SRU_ERR_INVALID_ARG, "attention sizes overflow");
    // grids: per-sequence products batch over blockIdx.y; one wave per row
    if (B > 65535) return fail(SRU_ERR_INVALID_ARG, "B must be <= 65535 for the attention");
    if ((s1 + 3) / 4 > kMaxBlocks || (dm->LB + 63) / 64 > kMaxBlocks ||
        (3 * dm->ndir * shape->d + 63) / 64 > 65535 || (2 * dp + 63) / 64 > 65535 ||
        (cfg->mem_len + L + 63) / 64 > 65535)
        return fail(SRU_ERR_INVALID_ARG, "attention too large for one launch");
    return SRU_OK;
}

}  // namespace

extern "C" {

size_t sru_attention_workspace_size(const sru_shape *shape, const sru_attn_cfg *cfg)
{
    Dims dm;
    if (check_attn(shape, cfg, &dm) != SRU_OK) return 0;
    ok();
    return round256(
        sru::attention_workspace_bytes(shape->L, shape->B, cfg->d_inner, cfg->mem_len));
}

sru_status sru_attention_forward(const sru_shape *shape, const sru_attn_cfg *cfg, const void *X,
                                 sru_dtype x_dt, const void *Wq, const void *Wkv, const void *Wo,
                                 const float *gamma, const float *beta, float *Q, void *KV,
                                 float *R, void *U, sru_dtype u_dt, void *workspace,
                                 size_t workspace_bytes, void *stream)
{
    Dims dm;
    SRU_TRY(check_attn(shape, cfg, &dm));
    if (!valid_dtype(x_dt) || !valid_dtype(u_dt)) return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    SRU_TRY(need_ptr(X, "X"));
    SRU_TRY(need_ptr(Wq, "Wq"));
    SRU_TRY(need_ptr(Wkv, "Wkv"));
    SRU_TRY(need_ptr(Wo, "Wo"));
    SRU_TRY(need_ptr(Q, "Q"));
    SRU_TRY(need_ptr(KV, "KV"));
    SRU_TRY(need_ptr(R, "R"));
    SRU_TRY(need_ptr(U, "U"));
    if (cfg->layernorm) {
        SRU_TRY(need_ptr(gamma, "gamma"));
        SRU_TRY(need_ptr(beta, "beta"));
    }
    const int64_t L = shape->L, B = shape->B, d = shape->d, dp = cfg->d_inner;
    const int64_t Lm = cfg->mem_len, n3 = 3 * dm.ndir * d;
    {   // the written outputs against each other and every input
        const Span out[] = {{Q, (size_t)(dm.LB * dp) * 4, "Q"},
                            {KV, (size_t)((Lm + L) * B * 2 * dp) * 2, "KV"},
                            {R, (size_t)(dm.LB * dp) * 4, "R"},
                            {U, (size_t)(dm.LB * n3) * (u_dt == SRU_BF16 ? 2 : 4), "U"}};
        const Span in[] = {{X, (size_t)(dm.LB * d) * (x_dt == SRU_BF16 ? 2 : 4), "X"},
                           {Wq, (size_t)(dp * d) * 2, "Wq"},
                           {Wkv, (size_t)(2 * dp * dp) * 2, "Wkv"},
                           {Wo, (size_t)(n3 * dp) * 2, "Wo"},
                           {gamma, cfg->layernorm ? (size_t)dp * 4 : 0, "gamma"},
                           {beta, cfg->layernorm ? (size_t)dp * 4 : 0, "beta"}};
        SRU_TRY(no_overlap(out, 4, in, 6));
    }
    const size_t need = round256(sru::attention_workspace_bytes(L, B, dp, Lm));
    if (!workspace || workspace_bytes < need)
        return fail(SRU_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need,
                    workspace_bytes, workspace ? "" : ", NULL");
    if (((uintptr_t)workspace) & 255u)
        return fail(SRU_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    SRU_TRY(need_device());
    sru::AttnArgs a;
    a.L = L, a.B = B, a.d = d, a.dp = dp, a.Lm = Lm, a.n3 = n3;
    a.causal = cfg->causal, a.layernorm = cfg->layernorm;
    a.alpha = cfg->attn_alpha, a.eps = cfg->ln_eps;
    a.X = X, a.x_bf16 = x_dt == SRU_BF16;
    a.Wq = (const sru::bf16_bits_t *)Wq;
    a.Wkv = (const sru::bf16_bits_t *)Wkv;
    a.Wo = (const sru::bf16_bits_t *)Wo;
    a.gamma = gamma, a.beta = beta;
    a.Q = Q, a.R = R, a.U = U, a.u_bf16 = u_dt == SRU_BF16, a.KV = KV, a.workspace = workspace;
    return launched(sru::launch_attention_forward(a, (hipStream_t)stream), "attention");
}

size_t sru_attention_backward_workspace_size(const sru_shape *shape, const sru_attn_cfg *cfg)
{
    Dims dm;
    if (check_attn(shape, cfg, &dm) != SRU_OK) return 0;
    ok();
    return round256(sru::attention_backward_workspace_bytes(
        shape->L, shape->B, shape->d, cfg->d_inner, cfg->mem_len, 3 * dm.ndir * shape->d));
}

sru_status sru_attention_backward(const sru_shape *shape, const sru_attn_cfg *cfg, const void *X,
                                  sru_dtype x_dt, const void *Wq, const void *Wkv, const void *Wo,
                                  const float *gamma, const float *Q, const void *KV,
                                  const float *R, const void *dU, sru_dtype du_dt, float *dX,
                                  int32_t accumulate_dx, float *dWq, float *dWkv, float *dWo,
                                  float *dalpha, float *dgamma, float *dbeta, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    Dims dm;
    SRU_TRY(check_attn(shape, cfg, &dm));
    if (!valid_dtype(x_dt) || !valid_dtype(du_dt)) return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    if (accumulate_dx != 0 && accumulate_dx != 1)
        return fail(SRU_ERR_INVALID_ARG, "accumulate_dx must be 0 or 1");
    if (cfg->d_inner > sru::kAttnBwdMaxInner)
        return fail(SRU_ERR_UNSUPPORTED, "the attention backward takes d_inner <= %lld (got %lld)",
                    (long long)sru::kAttnBwdMaxInner, (long long)cfg->d_inner);
    SRU_TRY(need_ptr(X, "X"));
    SRU_TRY(need_ptr(Wq, "Wq"));
    SRU_TRY(need_ptr(Wkv, "Wkv"));
    SRU_TRY(need_ptr(Wo, "Wo"));
    SRU_TRY(need_ptr(Q, "Q"));
    SRU_TRY(need_ptr(KV, "KV"));
    SRU_TRY(need_ptr(R, "R"));
    SRU_TRY(need_ptr(dU, "dU"));
    SRU_TRY(need_ptr(dX, "dX"));
    SRU_TRY(need_ptr(dWq, "dWq"));
    SRU_TRY(need_ptr(dWkv, "dWkv"));
    SRU_TRY(need_ptr(dWo, "dWo"));
    SRU_TRY(need_ptr(dalpha, "dalpha"));
    if (cfg->layernorm) {
        SRU_TRY(need_ptr(gamma, "gamma"));
        SRU_TRY(need_ptr(dgamma, "dgamma"));
        SRU_TRY(need_ptr(dbeta, "dbeta"));
    }
    const int64_t L = shape->L, B = shape->B, d = shape->d, dp = cfg->d_inner;
    const int64_t Lm = cfg->mem_len, n3 = 3 * dm.ndir * d;
    const size_t need = round256(sru::attention_backward_workspace_bytes(L, B, d, dp, Lm, n3));
    if (!workspace || workspace_bytes < need)
        return fail(SRU_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need,
                    workspace_bytes, workspace ? "" : ", NULL");
    if (((uintptr_t)workspace) & 255u)
        return fail(SRU_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    {   // the written outputs against each other and every input
        const size_t lbp = (size_t)(dm.LB * dp) * 4;
        const Span out[] = {{dX, (size_t)(dm.LB * d) * 4, "dX"},
                            {dWq, (size_t)(dp * d) * 4, "dWq"},
                            {dWkv, (size_t)(2 * dp * dp) * 4, "dWkv"},
                            {dWo, (size_t)(n3 * dp) * 4, "dWo"},
                            {dalpha, 4, "dalpha"},
                            {cfg->layernorm ? dgamma : nullptr, (size_t)dp * 4, "dgamma"},
                            {cfg->layernorm ? dbeta : nullptr, (size_t)dp * 4, "dbeta"},
                            {workspace, need, "workspace"}};
        const Span in[] = {{X, (size_t)(dm.LB * d) * elem_bytes(x_dt), "X"},
                           {Wq, (size_t)(dp * d) * 2, "Wq"},
                           {Wkv, (size_t)(2 * dp * dp) * 2, "Wkv"},
                           {Wo, (size_t)(n3 * dp) * 2, "Wo"},
                           {gamma, cfg->layernorm ? (size_t)dp * 4 : 0, "gamma"},
                           {Q, lbp, "Q"},
                           {KV, (size_t)((Lm + L) * B * 2 * dp) * 2, "KV"},
                           {R, lbp, "R"},
                           {dU, (size_t)(dm.LB * n3) * elem_bytes(du_dt), "dU"}};
        SRU_TRY(no_overlap(out, 8, in, 9));
    }
    SRU_TRY(need_device());
    sru::AttnBwdArgs a;
    a.L = L, a.B = B, a.d = d, a.dp = dp, a.Lm = Lm, a.n3 = n3;
    a.causal = cfg->causal, a.layernorm = cfg->layernorm;
    a.alpha = cfg->attn_alpha, a.eps = cfg->ln_eps;
    a.X = X, a.x_bf16 = x_dt == SRU_BF16;
    a.Wq = (const sru::bf16_bits_t *)Wq;
    a.Wkv = (const sru::bf16_bits_t *)Wkv;
    a.Wo = (const sru::bf16_bits_t *)Wo;
    a.gamma = gamma;
    a.Q = Q, a.R = R, a.KV = (const sru::bf16_bits_t *)KV;
    a.dU = dU, a.du_bf16 = du_dt == SRU_BF16;
    a.dX = dX, a.dx_accumulate = accumulate_dx != 0;
    a.dWq = dWq, a.dWkv = dWkv, a.dWo = dWo, a.dalpha = dalpha;
    a.dgamma = dgamma, a.dbeta = dbeta;
    a.workspace = workspace;
    return launched(sru::launch_attention_backward(a, (hipStream_t)stream), "attention backward");
}

sru_status sru_step(const sru_shape *shape, const void *x, sru_dtype x_dt, const void *W,
                    sru_dtype w_dt, const float *v, const float *b, const float *c_prev, float *h,
                    float *c_next, void *stream)
{
    Dims dm;
    SRU_TRY(check_shape(shape, &dm));
    if (shape->L != 1) return fail(SRU_ERR_INVALID_ARG, "a step has L = 1 (got %lld)",
                                   (long long)shape->L);
    if (shape->bidirectional)
        return fail(SRU_ERR_INVALID_ARG, "a decoding step is unidirectional");
    if (!valid_dtype(x_dt) || !valid_dtype(w_dt)) return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    SRU_TRY(need_ptr(x, "x"));
    SRU_TRY(need_ptr(W, "W"));
    SRU_TRY(need_ptr(v, "v"));
    SRU_TRY(need_ptr(b, "b"));
    SRU_TRY(opt_ptr(c_prev, "c_prev"));
    SRU_TRY(need_ptr(h, "h"));
    SRU_TRY(need_ptr(c_next, "c_next"));
    const int64_t B = shape->B, d = shape->d;
    int64_t w_el;
    if (!mul_ok(3 * d, d, &w_el)) return fail(SRU_ERR_INVALID_ARG, "tensor sizes overflow");
    if ((d + 3) / 4 > kMaxBlocks) return fail(SRU_ERR_INVALID_ARG, "d too large for one launch");
    const size_t bd = (size_t)(B * d) * 4;
    if (overlaps(h, bd, c_next, bd)) return fail(SRU_ERR_INVALID_ARG, "h overlaps c_next");
    if (c_prev && c_prev != c_next && overlaps(c_prev, bd, c_next, bd))
        return fail(SRU_ERR_INVALID_ARG, "c_next overlaps c_prev without being it");
    {
        const void *ins[] = {x, W, v, b, c_prev};
        const size_t sz[] = {(size_t)(B * d) * (x_dt == SRU_BF16 ? 2 : 4),
                             (size_t)w_el * (w_dt == SRU_BF16 ? 2 : 4), (size_t)(2 * d) * 4,
                             (size_t)(2 * d) * 4, c_prev ? bd : 0};
        for (int i = 0; i < 5; ++i) {
            if (!ins[i] || !sz[i]) continue;
            if (overlaps(h, bd, ins[i], sz[i]) ||
                (i < 4 && overlaps(c_next, bd, ins[i], sz[i])))
                return fail(SRU_ERR_INVALID_ARG, "an output overlaps an input");
        }
    }
    SRU_TRY(need_device());
    sru::StepArgs a;
    a.B = B, a.d = d;
    a.x = x, a.W = W;
    a.x_bf16 = x_dt == SRU_BF16, a.w_bf16 = w_dt == SRU_BF16;
    a.v = v, a.b = b, a.c_prev = c_prev;
    a.h = h, a.c_next = c_next;
    a.alpha = shape->alpha;
    return launched(sru::launch_step(a, (hipStream_t)stream), "step");
}

sru_status sru_round_bf16(int64_t n, const float *src, void *dst, void *stream)
{
    if (n < 1 || n > kMaxElems) return fail(SRU_ERR_INVALID_ARG, "n must be in [1, 2^56]");
    SRU_TRY(need_ptr(src, "src"));
    SRU_TRY(need_ptr(dst, "dst"));
    if (overlaps(src, (size_t)n * 4, dst, (size_t)n * 2))
        return fail(SRU_ERR_INVALID_ARG, "src and dst overlap");
    SRU_TRY(need_device());
    return launched(sru::launch_round_bf16(n, src, dst, (hipStream_t)stream), "bf16 rounding");
}

sru_status sru_transpose_weight(const sru_shape *shape, const void *W, sru_dtype w_dt, void *Wt,
                                void *stream)
{
    Dims dm;
    SRU_TRY(check_shape(shape, &dm));
    if (!valid_dtype(w_dt)) return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    SRU_TRY(need_ptr(W, "W"));
    SRU_TRY(need_ptr(Wt, "Wt"));
    const int64_t rows = 3 * dm.ndir * shape->d, cols = shape->d;
    const size_t bytes = (size_t)rows * (size_t)cols * (w_dt == SRU_BF16 ? 2 : 4);
    const uintptr_t a = (uintptr_t)W, b = (uintptr_t)Wt;
    if (a < b + bytes && b < a + bytes) return fail(SRU_ERR_INVALID_ARG, "W and Wt overlap");
    if ((cols + 63) / 64 > 65535 * 1024LL || (rows + 63) / 64 > 65535)
        return fail(SRU_ERR_INVALID_ARG, "matrix too large for one transpose launch");
    SRU_TRY(need_device());
    return launched(sru::launch_transpose(rows, cols, W, Wt, w_dt == SRU_BF16, (hipStream_t)stream),
                    "weight transpose");
}

sru_status sru_forward(const sru_shape *shape, const void *U, sru_dtype u_dt, const void *x,
                       sru_dtype x_dt, const float *v, const float *b, const float *c0, void *h,
                       sru_dtype h_dt, float *c_seq, float *c_last, void *stream)
{
    Dims dm;
    SRU_TRY(check_shape(shape, &dm));
    if (!valid_dtype(u_dt) || !valid_dtype(x_dt) || !valid_dtype(h_dt))
        return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    SRU_TRY(need_ptr(U, "U"));
    SRU_TRY(need_ptr(x, "x"));
    SRU_TRY(need_ptr(v, "v"));
    SRU_TRY(need_ptr(b, "b"));
    SRU_TRY(opt_ptr(c0, "c0"));
    SRU_TRY(need_ptr(h, "h"));
    SRU_TRY(opt_ptr(c_seq, "c_seq"));
    SRU_TRY(opt_ptr(c_last, "c_last"));
    if (h_dt != SRU_F32) return fail(SRU_ERR_UNSUPPORTED, "h must be fp32");
    {
        const size_t lbd = (size_t)(dm.LB * shape->d), hs = lbd * dm.ndir * 4;
        const size_t cs = (size_t)dm.chains * 4, ps = (size_t)(dm.ndir * 2 * shape->d) * 4;
        const Span out[] = {{h, hs, "h"}, {c_seq, hs, "c_seq"}, {c_last, cs, "c_last"}};
        const Span in[] = {{U, (size_t)dm.u_elems * elem_bytes(u_dt), "U"},
                           {x, lbd * elem_bytes(x_dt), "x"}, {v, ps, "v"}, {b, ps, "b"},
                           {c0, cs, "c0"}};
        SRU_TRY(no_overlap(out, 3, in, 5));
    }
    SRU_TRY(need_device());
    sru::RecArgs a{};
    a.L = shape->L;
    a.B = shape->B;
    a.d = shape->d;
    a.ndir = dm.ndir;
    a.alpha = shape->alpha;
    a.U = U;
    a.u_bf16 = u_dt == SRU_BF16;
    a.x = x;
    a.x_bf16 = x_dt == SRU_BF16;
    a.v = v;
    a.b = b;
    a.c0 = c0;
    a.h = (float *)h;
    a.c_seq = c_seq;
    a.c_last = c_last;
    return launched(sru::launch_forward(a, (hipStream_t)stream), "forward recurrence");
}

}  // extern "C"

namespace {

// The arguments of sru_backward and sru_backward_static, the workspace aside.
struct BwdCall {
    const sru_shape *shape;
    const void *U;
    sru_dtype u_dt;
    const void *x;
    sru_dtype x_dt;
    const float *v, *b, *c0, *c_seq, *dh, *dc_last;
    float *dU;
    void *dU_lp;
    float *dx, *dv, *db, *dc0;
};

// Validates everything but the workspace; *ws_need = the workspace bytes.
sru_status check_backward(const BwdCall &c, Dims *dm, size_t *ws_need, const void *workspace)
{
    SRU_TRY(check_shape(c.shape, dm));
    if (!valid_dtype(c.u_dt) || !valid_dtype(c.x_dt))
        return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    SRU_TRY(need_ptr(c.U, "U"));
    SRU_TRY(need_ptr(c.x, "x"));
    SRU_TRY(need_ptr(c.v, "v"));
    SRU_TRY(need_ptr(c.b, "b"));
    SRU_TRY(opt_ptr(c.c0, "c0"));
    SRU_TRY(need_ptr(c.c_seq, "c_seq"));
    SRU_TRY(need_ptr(c.dh, "dh"));
    SRU_TRY(opt_ptr(c.dc_last, "dc_last"));
    SRU_TRY(need_ptr(c.dU, "dU"));
    SRU_TRY(opt_ptr(c.dU_lp, "dU_lp"));
    SRU_TRY(need_ptr(c.dx, "dx"));
    SRU_TRY(opt_ptr(c.dv, "dv"));
    SRU_TRY(opt_ptr(c.db, "db"));
    SRU_TRY(opt_ptr(c.dc0, "dc0"));
    *ws_need = backward_ws(c.shape, *dm);
    const size_t lbd = (size_t)(dm->LB * c.shape->d), hs = lbd * dm->ndir * 4;
    const size_t cs = (size_t)dm->chains * 4, ps = (size_t)(dm->ndir * 2 * c.shape->d) * 4;
    const size_t ue = (size_t)dm->u_elems;
    const Span out[] = {{c.dU, ue * 4, "dU"},       {c.dU_lp, ue * 2, "dU_lp"},
                        {c.dx, lbd * 4, "dx"},      {c.dv, ps, "dv"},
                        {c.db, ps, "db"},           {c.dc0, cs, "dc0"},
                        {workspace, *ws_need, "workspace"}};
    const Span in[] = {{c.U, ue * elem_bytes(c.u_dt), "U"}, {c.x, lbd * elem_bytes(c.x_dt), "x"},
                       {c.v, ps, "v"},     {c.b, ps, "b"},   {c.c0, cs, "c0"},
                       {c.c_seq, hs, "c_seq"}, {c.dh, hs, "dh"}, {c.dc_last, cs, "dc_last"}};
    return no_overlap(out, 7, in, 8);
}

// Launches a validated backward.  ws: backward_ws bytes of scratch whose
// first 256 bytes are the control block; err: the call's error word (in that
// block, or elsewhere).
sru_status run_backward(const BwdCall &c, const Dims &dm, void *ws, uint32_t *err,
                        hipStream_t s)
{
    const sru_shape *shape = c.shape;
    sru::RecArgs a{};
    a.L = shape->L;
    a.B = shape->B;
    a.d = shape->d;
    a.ndir = dm.ndir;
    a.alpha = shape->alpha;
    a.U = c.U;
    a.u_bf16 = c.u_dt == SRU_BF16;
    a.x = c.x;
    a.x_bf16 = c.x_dt == SRU_BF16;
    a.v = c.v;
    a.b = c.b;
    a.c0 = c.c0;
    a.c_seq_in = c.c_seq;
    a.dh = c.dh;
    a.dc_last = c.dc_last;
    a.dU = c.dU;
    a.dU_lp = (sru::bf16_bits_t *)c.dU_lp;
    a.dx = c.dx;
    a.dc0 = c.dc0;
    // the per-chain kernels' partial sums follow the control block; they
    // clear the error word themselves (they have no look-back)
    a.partials = (float *)ws + sru::kCtrlWords;
    a.err_word = err;
    if (sru::backward_scan_ok(a.L, a.B, a.d, a.ndir, !a.u_bf16 && !a.x_bf16))
        return launched(sru::launch_backward_scan(a, ws, c.dv, c.db, s), "backward scan");
    if (sru::backward_bidi_ok(a)) {
        hipError_t e = sru::launch_backward_bidi(a, s);
        if (e == hipSuccess && (c.dv || c.db))
            e = sru::launch_param_reduce(a.partials, shape->B, shape->d, dm.ndir, c.dv, c.db, s);
        return launched(e, "backward recurrence");
    }
    // The highway gradient of x sums both directions: the last direction
    // writes dx, the ones before it add to it (stream order serialises them).
    for (int dir = dm.ndir - 1; dir >= 0; --dir) {
        a.dir = dir;
        a.dx_accumulate = dir != dm.ndir - 1;
        hipError_t e = sru::launch_backward_dir(a, s);
        if (e != hipSuccess) return launched(e, "backward recurrence");
    }
    if (c.dv || c.db) {
        hipError_t e =
            sru::launch_param_reduce(a.partials, shape->B, shape->d, dm.ndir, c.dv, c.db, s);
        if (e != hipSuccess) return launched(e, "parameter-gradient reduction");
    }
    return ok();
}

}  // namespace

extern "C" {

sru_status sru_backward(const sru_shape *shape, const void *U, sru_dtype u_dt, const void *x,
                        sru_dtype x_dt, const float *v, const float *b, const float *c0,
                        const float *c_seq, const float *dh, const float *dc_last, float *dU,
                        void *dU_lp, float *dx, float *dv, float *db, float *dc0, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    const BwdCall c{shape, U, u_dt, x, x_dt, v, b, c0, c_seq, dh, dc_last, dU, dU_lp, dx, dv, db,
                    dc0};
    Dims dm;
    size_t need = 0;
    SRU_TRY(check_backward(c, &dm, &need, workspace));
    if (!workspace || workspace_bytes < need)
        return fail(SRU_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need,
                    workspace_bytes, workspace ? "" : ", NULL");
    SRU_TRY(opt_ptr(workspace, "workspace"));
    SRU_TRY(need_device());
    return run_backward(c, dm, workspace, (uint32_t *)workspace + sru::kErrWord,
                        (hipStream_t)stream);
}

}  // extern "C"

namespace {

// The scratch of sru_backward_static: one array per GPU, alive until the
// process ends, shared by every call on that GPU.  In host code `scratch`
// names only a host-side stand-in; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
__device__ __align__(256) unsigned char scratch[SRU_BACKWARD_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

sru_status static_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return fail(SRU_ERR_NO_DEVICE, "no current HIP device for the static scratch (%s)",
                    e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(SRU_ERR_LAUNCH, "static scratch address on device %d: %s", dev,
                        hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SRU_OK;
}

}  // namespace

extern "C" {

sru_status sru_backward_static(const sru_shape *shape, const void *U, sru_dtype u_dt,
                               const void *x, sru_dtype x_dt, const float *v, const float *b,
                               const float *c0, const float *c_seq, const float *dh,
                               const float *dc_last, float *dU, void *dU_lp, float *dx,
                               float *dv, float *db, float *dc0, uint32_t *error_word,
                               void *stream)
{
    const BwdCall c{shape, U, u_dt, x, x_dt, v, b, c0, c_seq, dh, dc_last, dU, dU_lp, dx, dv, db,
                    dc0};
    Dims dm;
    size_t need = 0;
    SRU_TRY(check_backward(c, &dm, &need, nullptr));
    if (need > (size_t)SRU_BACKWARD_STATIC_SCRATCH_BYTES)
        return fail(SRU_ERR_WORKSPACE,
                    "this shape needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use sru_backward with a workspace)",
                    need, (size_t)SRU_BACKWARD_STATIC_SCRATCH_BYTES);
    if (((uintptr_t)error_word) & 3u)
        return fail(SRU_ERR_INVALID_ARG, "error_word must be 4-byte aligned");
    if (error_word) {
        const Span out[] = {{error_word, 4, "error_word"}};
        const size_t lbd = (size_t)(dm.LB * shape->d), ue = (size_t)dm.u_elems;
        const size_t cs = (size_t)dm.chains * 4, ps = (size_t)(dm.ndir * 2 * shape->d) * 4;
        const Span other[] = {{U, ue * elem_bytes(u_dt), "U"}, {x, lbd * elem_bytes(x_dt), "x"},
                              {dU, ue * 4, "dU"}, {dU_lp, ue * 2, "dU_lp"}, {dx, lbd * 4, "dx"},
                              {dv, ps, "dv"}, {db, ps, "db"}, {dc0, cs, "dc0"}};
        SRU_TRY(no_overlap(out, 1, other, 8));
    }
    SRU_TRY(need_device());
    void *ws = nullptr;
    SRU_TRY(static_scratch(&ws));
    uint32_t *err = error_word ? error_word : (uint32_t *)ws + sru::kErrWord;
    return run_backward(c, dm, ws, err, (hipStream_t)stream);
}

sru_status sru_linear_scan(const sru_shape *shape, sru_pass pass, int32_t chunk, const void *U,
                           sru_dtype u_dt, const void *x, sru_dtype x_dt, const float *b,
                           const float *c0, void *h, sru_dtype h_dt, float *c_seq, float *c_last,
                           const float *dh, const float *dc_last, float *dU, float *dx, float *db,
                           float *dc0, void *workspace, size_t workspace_bytes, void *stream)
{
    Dims dm;
    SRU_TRY(check_shape(shape, &dm));
    if (pass != SRU_FWD && pass != SRU_BWD)
        return fail(SRU_ERR_INVALID_ARG, "unknown pass %d", (int)pass);
    if (chunk < 1) return fail(SRU_ERR_INVALID_ARG, "chunk must be >= 1 (got %d)", (int)chunk);
    if (!valid_dtype(u_dt) || !valid_dtype(x_dt))
        return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
    SRU_TRY(need_ptr(U, "U"));
    SRU_TRY(need_ptr(x, "x"));
    SRU_TRY(need_ptr(b, "b"));
    SRU_TRY(opt_ptr(c0, "c0"));
    const int64_t nC = (shape->L + chunk - 1) / chunk;
    int64_t lanes;
    if (!mul_ok(nC, shape->B * shape->d, &lanes) || (lanes + 255) / 256 > kMaxBlocks)
        return fail(SRU_ERR_INVALID_ARG, "too many (chain, chunk) pairs for one launch");
    const bool bwd = pass == SRU_BWD;
    if (!bwd) {
        if (!valid_dtype(h_dt)) return fail(SRU_ERR_INVALID_ARG, "unknown dtype");
        SRU_TRY(need_ptr(h, "h"));
        SRU_TRY(opt_ptr(c_seq, "c_seq"));
        SRU_TRY(opt_ptr(c_last, "c_last"));
        if (h_dt != SRU_F32) return fail(SRU_ERR_UNSUPPORTED, "h must be fp32");
    } else {
        SRU_TRY(need_ptr(c_seq, "c_seq"));
        SRU_TRY(need_ptr(dh, "dh"));
        SRU_TRY(opt_ptr(dc_last, "dc_last"));
        SRU_TRY(need_ptr(dU, "dU"));
        SRU_TRY(need_ptr(dx, "dx"));
        SRU_TRY(opt_ptr(db, "db"));
        SRU_TRY(opt_ptr(dc0, "dc0"));
    }
    const size_t need = round256(sru::linear_workspace_bytes(shape->L, shape->B, shape->d,
                                                             dm.ndir, chunk, bwd));
    if (!workspace || workspace_bytes < need)
        return fail(SRU_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need,
                    workspace_bytes, workspace ? "" : ", NULL");
    SRU_TRY(opt_ptr(workspace, "workspace"));
    {
        const size_t lbd = (size_t)(dm.LB * shape->d), hs = lbd * dm.ndir * 4;
        const size_t cs = (size_t)dm.chains * 4, ps = (size_t)(dm.ndir * 2 * shape->d) * 4;
        const size_t ue = (size_t)dm.u_elems;
        const Span in_common[] = {{U, ue * elem_bytes(u_dt), "U"}, {x, lbd * elem_bytes(x_dt), "x"},
                                  {b, ps, "b"}, {c0, cs, "c0"}};
        if (!bwd) {
            const Span out[] = {{h, hs, "h"}, {c_seq, hs, "c_seq"}, {c_last, cs, "c_last"},
                                {workspace, need, "workspace"}};
            SRU_TRY(no_overlap(out, 4, in_common, 4));
        } else {
            const Span out[] = {{dU, ue * 4, "dU"}, {dx, lbd * 4, "dx"}, {db, ps, "db"},
                                {dc0, cs, "dc0"}, {workspace, need, "workspace"}};
            const Span in[] = {in_common[0], in_common[1], in_common[2], in_common[3],
                               {c_seq, hs, "c_seq"}, {dh, hs, "dh"}, {dc_last, cs, "dc_last"}};
            SRU_TRY(no_overlap(out, 5, in, 7));
        }
    }
    SRU_TRY(need_device());
    sru::LinArgs a{};
    a.L = shape->L;
    a.B = shape->B;
    a.d = shape->d;
    a.ndir = dm.ndir;
    a.alpha = shape->alpha;
    a.chunk = chunk;
    a.U = U;
    a.u_bf16 = u_dt == SRU_BF16;
    a.x = x;
    a.x_bf16 = x_dt == SRU_BF16;
    a.b = b;
    a.c0 = c0;
    a.ws = workspace;
    if (!bwd) {
        a.h = (float *)h;
        a.c_seq = c_seq;
        a.c_last = c_last;
        return launched(sru::launch_linear_forward(a, (hipStream_t)stream), "linear scan forward");
    }
    a.c_seq = c_seq;
    a.dh = dh;
    a.dc_last = dc_last;
    a.dU = dU;
    a.dx = dx;
    a.db = db;
    a.dc0 = dc0;
    return launched(sru::launch_linear_backward(a, (hipStream_t)stream), "linear scan backward");
}

}  // extern "C"

// C ABI of the dual-branch W4A4 layer: host-side validation, size queries and
// kernel dispatch.  No call allocates device memory or synchronizes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "mg_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(MG_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MG_CHECK_PTR(p, name)                                                       \
    do {                                                                            \
        if ((p) == nullptr) return fail(MG_ERR_ARG, "%s: null pointer", name);      \
        if (!aligned16(p)) return fail(MG_ERR_ALIGN, "%s: not 16-byte aligned", name); \
    } while (0)

int check_dtype(int32_t dtype) {
    if (dtype != MG_F32 && dtype != MG_BF16) return fail(MG_ERR_DTYPE, "dtype %d is not MG_F32/MG_BF16", dtype);
    return MG_OK;
}

int check_K(int32_t K) {
    if (K <= 0 || K % 32 != 0) return fail(MG_ERR_SHAPE, "K=%d must be a positive multiple of 32", K);
    if (K > mg::kMaxK) return fail(MG_ERR_UNSUPPORTED, "K=%d exceeds %d", K, mg::kMaxK);
    return MG_OK;
}

int check_desc(const mg_plan_desc* d) {
    if (!d) return fail(MG_ERR_ARG, "null plan descriptor");
    if (int e = check_K(d->K)) return e;
    if (d->N <= 0 || d->N % 32 != 0) return fail(MG_ERR_SHAPE, "N=%d must be a positive multiple of 32", d->N);
    if (d->k < 0 || d->k > d->K) return fail(MG_ERR_SHAPE, "k=%d must be in [0, K=%d]", d->k, d->K);
    if (d->layout != MG_W_1X32 && d->layout != MG_W_32X32 && d->layout != MG_W_128X1)
        return fail(MG_ERR_ARG, "layout %d is not MG_W_1X32/MG_W_32X32/MG_W_128X1", d->layout);
    if (d->smooth != 0 && d->smooth != 1) return fail(MG_ERR_ARG, "smooth must be 0 or 1");
    if (d->score != MG_SCORE_MAX && d->score != MG_SCORE_SMOOTHED)
        return fail(MG_ERR_ARG, "score %d is not MG_SCORE_MAX/MG_SCORE_SMOOTHED", d->score);
    if (d->smooth && !(d->alpha > 0.0 && d->alpha < 1.0))
        return fail(MG_ERR_ARG, "alpha=%g must be in (0, 1)", d->alpha);
    return MG_OK;
}

int check_plan(const mg_plan* p, bool need_w) {
    if (!p) return fail(MG_ERR_ARG, "null plan");
    if (int e = check_desc(&p->d)) return e;
    MG_CHECK_PTR(p->s, "plan.s");
    MG_CHECK_PTR(p->rcp, "plan.rcp");
    MG_CHECK_PTR(p->pos, "plan.pos");
    if (p->d.k > 0) MG_CHECK_PTR(p->O, "plan.O");
    if (need_w) {
        MG_CHECK_PTR(p->Wq, "plan.Wq");
        MG_CHECK_PTR(p->Ws, "plan.Ws");
        if (p->d.k > 0) MG_CHECK_PTR(p->WO, "plan.WO");
        if (p->d.layout != MG_W_1X32) MG_CHECK_PTR(p->Wst, "plan.Wst");
    }
    return MG_OK;
}

// The GEMM addresses each operand with 32-bit offsets below 3 GiB.
int check_gemm_size(const mg_plan* p, int64_t M) {
    const int64_t lim = 0xC0000000ll;
    const int64_t K = p->d.K, N = p->d.N, k = p->d.k;
    if (mg::frag_bytes(M, K / 2) >= lim || mg::frag_bytes(N, K / 2) >= lim || mg::frag_bytes(M, 2 * k) >= lim ||
        mg::frag_bytes(N, 2 * k) >= lim || mg::sc_bytes(M, p->d.K) >= lim || mg::sc_bytes(p->d.N, p->d.K) >= lim)
        return fail(MG_ERR_UNSUPPORTED, "operands of M=%lld, N=%d, K=%d, k=%d exceed 3 GiB", (long long)M, p->d.N,
                    p->d.K, p->d.k);
    return MG_OK;
}

int check_act(const mg_plan* p, const mg_act* a) {
    if (!a) return fail(MG_ERR_ARG, "null activation workspace");
    MG_CHECK_PTR(a->Aq, "act.Aq");
    MG_CHECK_PTR(a->As, "act.As");
    if (p->d.k > 0) MG_CHECK_PTR(a->XO, "act.XO");
    return MG_OK;
}

}  // namespace

namespace mg {

int check_forward(const mg_plan* p, const void* X, int32_t dtype, int64_t M, const void* Y, int32_t y_dtype) {
    if (int e = check_plan(p, true)) return e;
    if (int e = check_dtype(dtype)) return e;
    if (int e = check_dtype(y_dtype)) return e;
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    if (M == 0) return MG_OK;
    MG_CHECK_PTR(X, "X");
    MG_CHECK_PTR(Y, "Y");
    return check_gemm_size(p, M);
}

int fail_msg(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int blocks_per_cu(const void* kern) {
    struct Entry { const void* k; int dev; int n; };
    static thread_local Entry cache[32] = {};
    static thread_local int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    for (int i = 0; i < used; ++i)
        if (cache[i].k == kern && cache[i].dev == dev) return cache[i].n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 256, 0) != hipSuccess || n < 1) n = 1;
    if (used < 32) cache[used++] = Entry{kern, dev, n};
    return n;
}

int device_cu_count() {
    static thread_local int cached_dev = -1;
    static thread_local int cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

}  // namespace mg

extern "C" {

int mg_version(void) { return 400; }   // 0.4.0: operands in fragment order

const char* mg_last_error(void) { return g_err; }

int mg_plan_bytes(const mg_plan_desc* d, size_t out[8]) {
    if (int e = check_desc(d)) return e;
    if (!out) return fail(MG_ERR_ARG, "null output array");
    const size_t K = (size_t)d->K, N = (size_t)d->N, k = (size_t)d->k;
    out[0] = 4 * K;                                        // s
    out[1] = 4 * K;                                        // rcp
    out[2] = 4 * k;                                        // O
    out[3] = 4 * K;                                        // pos
    out[4] = (size_t)mg::frag_bytes((int64_t)N, d->K / 2);  // Wq, fragment order
    out[5] = (size_t)mg::sc_bytes((int64_t)N, d->K);       // Ws, in 256-row x 16-block windows
    out[6] = d->layout == MG_W_32X32 ? (N / 32) * (K / 32)       // Wst
           : d->layout == MG_W_128X1 ? N * ((K + 127) / 128) : 0;
    out[7] = (size_t)mg::frag_bytes((int64_t)N, 2 * (int64_t)d->k);   // WO, fragment order
    return MG_OK;
}

int mg_act_bytes(const mg_plan_desc* d, int64_t M, size_t out[3]) {
    if (int e = check_desc(d)) return e;
    if (!out) return fail(MG_ERR_ARG, "null output array");
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    out[0] = (size_t)mg::frag_bytes(M, d->K / 2);          // Aq, fragment order
    out[1] = (size_t)mg::sc_bytes(M, d->K);                // As, in 256-row x 16-block windows
    out[2] = (size_t)mg::frag_bytes(M, 2 * (int64_t)d->k);  // XO, fragment order
    return MG_OK;
}

int mg_calib_reset(float* act_max, int32_t K, hipStream_t stream) {
    if (int e = check_K(K)) return e;
    MG_CHECK_PTR(act_max, "act_max");
    hipError_t h = mg::launch_fill_u32(reinterpret_cast<uint32_t*>(act_max), 0u, K, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_calib_reset");
}

int mg_calib_act(const void* X, int32_t dtype, int64_t M, int32_t K, float* act_max, hipStream_t stream) {
    if (int e = check_dtype(dtype)) return e;
    if (int e = check_K(K)) return e;
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    MG_CHECK_PTR(act_max, "act_max");
    if (M == 0) return MG_OK;
    MG_CHECK_PTR(X, "X");
    hipError_t h = mg::launch_colmax(X, dtype, M, K, act_max, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_calib_act");
}

int mg_weight_range(const void* W, int32_t dtype, int32_t N, int32_t K, float* w_max, hipStream_t stream) {
    if (int e = check_dtype(dtype)) return e;
    if (int e = check_K(K)) return e;
    if (N <= 0) return fail(MG_ERR_SHAPE, "N=%d must be positive", N);
    MG_CHECK_PTR(W, "W");
    MG_CHECK_PTR(w_max, "w_max");
    hipError_t h = mg::launch_fill_u32(reinterpret_cast<uint32_t*>(w_max), 0u, K, stream);
    if (h == hipSuccess) h = mg::launch_colmax(W, dtype, N, K, w_max, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_weight_range");
}

static int check_pct(const mg_pct* st) {
    if (st == nullptr) return fail(MG_ERR_ARG, "mg_pct: null pointer");
    if (int e = check_K(st->K)) return e;
    if (st->reserved != 0) return fail(MG_ERR_ARG, "mg_pct.reserved must be 0");
    MG_CHECK_PTR(st->hist, "mg_pct.hist");
    MG_CHECK_PTR(st->sel, "mg_pct.sel");
    return MG_OK;
}

static int check_pass(int32_t pass) {
    if (pass != 0 && pass != 1) return fail(MG_ERR_ARG, "pass=%d must be 0 or 1", pass);
    return MG_OK;
}

int mg_pct_reset(const mg_pct* st, hipStream_t stream) {
    if (int e = check_pct(st)) return e;
    hipError_t h = mg::launch_pct_reset(st->hist, st->K, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_pct_reset");
}

int mg_pct_count(const mg_pct* st, int32_t pass, const uint16_t* X, int64_t M, hipStream_t stream) {
    if (int e = check_pct(st)) return e;
    if (int e = check_pass(pass)) return e;
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    // at most 65535 row chunks of at most 65535 rows (16-bit per-workgroup counters)
    if (M > 65535ll * 65535ll) return fail(MG_ERR_UNSUPPORTED, "M=%lld exceeds 65535^2 rows per call", (long long)M);
    if (M == 0) return MG_OK;
    MG_CHECK_PTR(X, "X");
    hipError_t h = mg::launch_pct_count(X, M, st->K, pass, st->sel, st->hist, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_pct_count");
}

int mg_pct_select(const mg_pct* st, int32_t pass, double q, float* score, hipStream_t stream) {
    if (int e = check_pct(st)) return e;
    if (int e = check_pass(pass)) return e;
    if (!(q > 0.0 && q <= 1.0)) return fail(MG_ERR_ARG, "q=%g must lie in (0, 1]", q);
    if (pass == 1) MG_CHECK_PTR(score, "score");
    hipError_t h = mg::launch_pct_select(st->K, pass, q, st->hist, st->sel, pass == 1 ? score : nullptr, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_pct_select");
}

int mg_smooth_scales(const mg_plan* p, const float* act_max, const float* w_max, hipStream_t stream) {
    if (int e = check_plan(p, false)) return e;
    if (p->d.smooth) {
        MG_CHECK_PTR(act_max, "act_max");
        MG_CHECK_PTR(w_max, "w_max");
    }
    hipError_t h = mg::launch_smooth(act_max, w_max, p->d.K, p->d.alpha, p->d.smooth, p->s, p->rcp, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_smooth_scales");
}

int mg_outlier_set(const mg_plan* p, const float* act_max, hipStream_t stream) {
    if (int e = check_plan(p, false)) return e;
    MG_CHECK_PTR(act_max, "act_max");
    hipError_t h = mg::launch_topk(act_max, p->d.score == MG_SCORE_SMOOTHED ? p->s : nullptr, p->d.K, p->d.k,
                                   p->O, p->pos, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_outlier_set");
}

int mg_fold_pack(const mg_plan* p, const void* W, int32_t dtype, hipStream_t stream) {
    if (int e = check_plan(p, true)) return e;
    if (int e = check_dtype(dtype)) return e;
    MG_CHECK_PTR(W, "W");
    hipError_t h = mg::launch_fold_pack(W, dtype, p->d.N, p->d.K, p->d.k, p->d.layout, p->s, p->pos, p->Wq,
                                        p->Ws, p->Wst, p->WO, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_fold_pack");
}

int mg_plan_build(const mg_plan* p, const float* act_max, const float* w_max, const void* W, int32_t dtype,
                  hipStream_t stream) {
    if (int e = check_plan(p, true)) return e;
    if (int e = check_dtype(dtype)) return e;
    MG_CHECK_PTR(act_max, "act_max");
    if (p->d.smooth) MG_CHECK_PTR(w_max, "w_max");
    MG_CHECK_PTR(W, "W");
    if (int e = mg_smooth_scales(p, act_max, w_max, stream)) return e;
    if (int e = mg_outlier_set(p, act_max, stream)) return e;
    return mg_fold_pack(p, W, dtype, stream);
}

int mg_quantize_act(const mg_plan* p, const void* X, int32_t dtype, int64_t M, const mg_act* a,
                    hipStream_t stream) {
    if (int e = check_plan(p, false)) return e;
    if (int e = check_dtype(dtype)) return e;
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    if (M == 0) return MG_OK;
    MG_CHECK_PTR(X, "X");
    if (int e = check_act(p, a)) return e;
    hipError_t h = mg::launch_quant(X, dtype, M, p->d.K, p->d.k, p->s, p->rcp, p->pos, a->Aq, a->As, a->XO,
                                    stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_quantize_act");
}

int mg_quantize_act_stats(const mg_plan* p, const void* X, int32_t dtype, int64_t M, const mg_act* a,
                          float* act_max, hipStream_t stream) {
    if (int e = check_plan(p, false)) return e;
    if (int e = check_dtype(dtype)) return e;
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    MG_CHECK_PTR(act_max, "act_max");
    if (M == 0) return MG_OK;
    MG_CHECK_PTR(X, "X");
    if (int e = check_act(p, a)) return e;
    hipError_t h = mg::launch_quant(X, dtype, M, p->d.K, p->d.k, p->s, p->rcp, p->pos, a->Aq, a->As, a->XO,
                                    stream, false, act_max);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_quantize_act_stats");
}

int mg_gelu_quantize_act(const mg_plan* p, const uint16_t* Y, int64_t M, const mg_act* a, hipStream_t stream) {
    if (int e = check_plan(p, false)) return e;
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    if (M == 0) return MG_OK;
    MG_CHECK_PTR(Y, "Y");
    if (int e = check_act(p, a)) return e;
    hipError_t h = mg::launch_quant(Y, MG_BF16, M, p->d.K, p->d.k, p->s, p->rcp, p->pos, a->Aq, a->As, a->XO,
                                    stream, true);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_gelu_quantize_act");
}

int mg_dual_gemm_gelu_quant(const mg_plan* p0, const mg_act* a0, int64_t M, const mg_plan* p2, const mg_act* a2,
                            hipStream_t stream) {
    if (int e = check_plan(p0, true)) return e;
    if (int e = check_plan(p2, false)) return e;
    if (p2->d.K != p0->d.N)
        return fail(MG_ERR_SHAPE, "the next layer's K=%d must equal this layer's N=%d", p2->d.K, p0->d.N);
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    if (M == 0) return MG_OK;
    if (int e = check_act(p0, a0)) return e;
    if (int e = check_act(p2, a2)) return e;
    if (int e = check_gemm_size(p0, M)) return e;
    if (int e = check_gemm_size(p2, M)) return e;
    hipError_t h = mg::launch_dual_gemm_gelu_quant(a0->Aq, a0->As, a0->XO, p0->Wq, p0->Ws, p0->WO, M, p0->d.N,
                                                   p0->d.K, p0->d.k, p2->s, p2->rcp, p2->pos, p2->d.k, a2->Aq,
                                                   a2->As, a2->XO, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_dual_gemm_gelu_quant");
}

int mg_dual_gemm(const mg_plan* p, const mg_act* a, int64_t M, void* Y, int32_t y_dtype, hipStream_t stream) {
    if (int e = check_plan(p, true)) return e;
    if (int e = check_dtype(y_dtype)) return e;
    if (M < 0) return fail(MG_ERR_SHAPE, "M=%lld must be >= 0", (long long)M);
    if (M == 0) return MG_OK;
    if (int e = check_act(p, a)) return e;
    if (int e = check_gemm_size(p, M)) return e;
    MG_CHECK_PTR(Y, "Y");
    hipError_t h = mg::launch_dual_gemm(a->Aq, a->As, a->XO, p->Wq, p->Ws, p->WO, M, p->d.N, p->d.K, p->d.k, Y,
                                        y_dtype, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_dual_gemm");
}

int mg_forward(const mg_plan* p, const void* X, int32_t dtype, int64_t M, const mg_act* a, void* Y,
               int32_t y_dtype, hipStream_t stream) {
    // every check of both steps before anything is launched
    if (int e = mg::check_forward(p, X, dtype, M, Y, y_dtype)) return e;
    if (M == 0) return MG_OK;
    if (int e = check_act(p, a)) return e;
    if (int e = mg_quantize_act(p, X, dtype, M, a, stream)) return e;
    return mg_dual_gemm(p, a, M, Y, y_dtype, stream);
}

int mg_gelu_tanh_bf16(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t stream) {
    if (n < 0) return fail(MG_ERR_SHAPE, "n=%lld must be >= 0", (long long)n);
    if (n == 0) return MG_OK;
    MG_CHECK_PTR(in, "in");
    MG_CHECK_PTR(out, "out");
    hipError_t h = mg::launch_gelu(in, out, n, stream);
    return h == hipSuccess ? MG_OK : hip_fail(h, "mg_gelu_tanh_bf16");
}

}  // extern "C"

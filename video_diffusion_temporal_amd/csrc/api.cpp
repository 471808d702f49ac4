// libvinf C ABI: argument validation and dispatch (host only).
//
// Every check runs before anything is enqueued, so a rejected call has no
// effect on the device.  Launchers live next to their kernels.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace vinf_host {

static thread_local char g_last_error[512];

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
}

vinf_status fail(vinf_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

vinf_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VINF_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return VINF_OK;
}

// Shared shape checks; fills the tensor byte size.
static vinf_status check_shape(const char* fn, int F, int H, int W, int C, vinf_dtype dt, size_t* bytes) {
    if (dt != VINF_F32 && dt != VINF_BF16) return fail(VINF_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
    if (F < 1 || H < 1 || W < 1 || C < 1)
        return fail(VINF_ERR_INVALID_ARG, "%s: sizes must be >= 1 (F=%d H=%d W=%d C=%d)", fn, F, H, W, C);
    const int vec = dt == VINF_BF16 ? 8 : 4;
    if (C % vec)
        return fail(VINF_ERR_UNSUPPORTED, "%s: C=%d must be a multiple of %d (16-byte vectors)", fn, C, vec);
    // F*H*W*C elements, checked against 2^62 bytes before multiplying further.
    const double n = (double)F * H * W * C;
    if (n * dtype_bytes(dt) > 4.0e18) return fail(VINF_ERR_INVALID_ARG, "%s: tensor too large", fn);
    if ((double)H * W > 2147483647.0) return fail(VINF_ERR_UNSUPPORTED, "%s: H*W too large", fn);
    *bytes = (size_t)F * H * W * C * dtype_bytes(dt);
    return VINF_OK;
}

static vinf_status check_tensor(const char* fn, const char* name, const void* p, bool required) {
    if (!p) return required ? fail(VINF_ERR_INVALID_ARG, "%s: %s is NULL", fn, name) : VINF_OK;
    if (!aligned(p, 16)) return fail(VINF_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name);
    return VINF_OK;
}

static vinf_status check_f32(const char* fn, const char* name, const void* p) {
    if (p && !aligned(p, 4)) return fail(VINF_ERR_INVALID_ARG, "%s: %s is not 4-byte aligned", fn, name);
    return VINF_OK;
}

static vinf_status check_f64(const char* fn, const char* name, const void* p, bool required) {
    if (!p) return required ? fail(VINF_ERR_INVALID_ARG, "%s: %s is NULL", fn, name) : VINF_OK;
    if (!aligned(p, 8)) return fail(VINF_ERR_INVALID_ARG, "%s: %s is not 8-byte aligned", fn, name);
    return VINF_OK;
}

// First frame of the local window of query frame t in an F-frame video
// (n_local consecutive frames centred on t, shifted inward at the ends).
static int64_t window_start(int64_t t, int64_t F, int64_t n_local) {
    int64_t st = t - n_local / 2, hi = F - n_local > 0 ? F - n_local : 0;
    return st < 0 ? 0 : (st > hi ? hi : st);
}

// Context frames a clip's local windows reach before and after it.
static void clip_halo(int64_t F, int64_t f0, int64_t Fc, int64_t n_local, int64_t* pre, int64_t* post) {
    if (n_local <= 0) {
        *pre = *post = 0;
        return;
    }
    const int64_t nl = n_local < F ? n_local : F;
    const int64_t a = window_start(f0, F, n_local), b = window_start(f0 + Fc - 1, F, n_local) + nl;
    *pre = f0 - a;
    *post = b - (f0 + Fc) > 0 ? b - (f0 + Fc) : 0;
}

#define VINF_TRY(expr)                         \
    do {                                       \
        vinf_status s_ = (expr);               \
        if (s_ != VINF_OK) return s_;          \
    } while (0)

}  // namespace vinf_host

using namespace vinf_host;

extern "C" {

size_t vinf_groupnorm_workspace_bytes(int F, int H, int W, int C, int groups, vinf_dtype dt) {
    size_t bytes;
    if (check_shape("vinf_groupnorm_workspace_bytes", F, H, W, C, dt, &bytes) != VINF_OK) return 0;
    if (groups < 1 || C % groups) return 0;
    return groupnorm_workspace((int64_t)F * H * W, C, groups, dt);
}

vinf_status vinf_groupnorm_global(const void* x, void* y, const float* gamma, const float* beta, float* mean_out,
                                  float* rstd_out, int F, int H, int W, int C, int groups, float eps, vinf_dtype dt,
                                  void* workspace, size_t workspace_bytes, vinf_stream stream) {
    const char* fn = "vinf_groupnorm_global";
    size_t bytes;
    VINF_TRY(check_shape(fn, F, H, W, C, dt, &bytes));
    VINF_TRY(check_tensor(fn, "x", x, true));
    VINF_TRY(check_tensor(fn, "y", y, true));
    VINF_TRY(check_f32(fn, "gamma", gamma));
    VINF_TRY(check_f32(fn, "beta", beta));
    VINF_TRY(check_f32(fn, "mean_out", mean_out));
    VINF_TRY(check_f32(fn, "rstd_out", rstd_out));
    if (groups < 1 || C % groups) return fail(VINF_ERR_INVALID_ARG, "%s: C=%d not divisible by groups=%d", fn, C, groups);
    if (!(eps >= 0.f)) return fail(VINF_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
    const int vec = dt == VINF_BF16 ? 8 : 4;
    if (C / vec > 1024) return fail(VINF_ERR_UNSUPPORTED, "%s: C=%d exceeds %d", fn, C, 1024 * vec);
    if (y != x && overlap(x, bytes, y, bytes))
        return fail(VINF_ERR_INVALID_ARG, "%s: y partially overlaps x (only y == x is allowed)", fn);
    const size_t need = groupnorm_workspace((int64_t)F * H * W, C, groups, dt);
    if (!workspace || workspace_bytes < need)
        return fail(VINF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(VINF_ERR_WORKSPACE, "%s: workspace is not 256-byte aligned", fn);
    const size_t stat_bytes = (size_t)groups * sizeof(float);
    if (overlap(workspace, need, x, bytes) || overlap(workspace, need, y, bytes) ||
        overlap(mean_out, stat_bytes, x, bytes) || overlap(mean_out, stat_bytes, y, bytes) ||
        overlap(rstd_out, stat_bytes, x, bytes) || overlap(rstd_out, stat_bytes, y, bytes) ||
        overlap(workspace, need, mean_out, stat_bytes) || overlap(workspace, need, rstd_out, stat_bytes))
        return fail(VINF_ERR_INVALID_ARG, "%s: workspace / statistics overlap a tensor", fn);
    return launch_groupnorm(x, y, gamma, beta, mean_out, rstd_out, (int64_t)F * H * W, C, groups, eps, dt, workspace,
                            (hipStream_t)stream);
}

vinf_status vinf_groupnorm_global_noalloc(const void* x, void* y, const float* gamma, const float* beta,
                                          float* mean_out, float* rstd_out, int F, int H, int W, int C, int groups,
                                          float eps, vinf_dtype dt, vinf_stream stream) {
    const char* fn = "vinf_groupnorm_global_noalloc";
    size_t bytes;
    VINF_TRY(check_shape(fn, F, H, W, C, dt, &bytes));
    VINF_TRY(check_tensor(fn, "x", x, true));
    VINF_TRY(check_tensor(fn, "y", y, true));
    VINF_TRY(check_f32(fn, "gamma", gamma));
    VINF_TRY(check_f32(fn, "beta", beta));
    VINF_TRY(check_f32(fn, "mean_out", mean_out));
    VINF_TRY(check_f32(fn, "rstd_out", rstd_out));
    if (groups < 1 || C % groups) return fail(VINF_ERR_INVALID_ARG, "%s: C=%d not divisible by groups=%d", fn, C, groups);
    if (!(eps >= 0.f)) return fail(VINF_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
    const int vec = dt == VINF_BF16 ? 8 : 4;
    if (C / vec > 1024) return fail(VINF_ERR_UNSUPPORTED, "%s: C=%d exceeds %d", fn, C, 1024 * vec);
    if (y != x && overlap(x, bytes, y, bytes))
        return fail(VINF_ERR_INVALID_ARG, "%s: y partially overlaps x (only y == x is allowed)", fn);
    const size_t stat_bytes = (size_t)groups * sizeof(float);
    if (overlap(mean_out, stat_bytes, x, bytes) || overlap(mean_out, stat_bytes, y, bytes) ||
        overlap(rstd_out, stat_bytes, x, bytes) || overlap(rstd_out, stat_bytes, y, bytes))
        return fail(VINF_ERR_INVALID_ARG, "%s: statistics overlap a tensor", fn);
    return launch_groupnorm_noalloc(x, y, gamma, beta, mean_out, rstd_out, (int64_t)F * H * W, C, groups, eps, dt,
                                    (hipStream_t)stream);
}

vinf_status vinf_groupnorm_stats(const void* x, float* mean_out, float* rstd_out, int F, int H, int W, int C,
                                 int groups, float eps, vinf_dtype dt, void* workspace, size_t workspace_bytes,
                                 vinf_stream stream) {
    const char* fn = "vinf_groupnorm_stats";
    size_t bytes;
    VINF_TRY(check_shape(fn, F, H, W, C, dt, &bytes));
    VINF_TRY(check_tensor(fn, "x", x, true));
    if (!mean_out || !rstd_out) return fail(VINF_ERR_INVALID_ARG, "%s: mean_out and rstd_out are required", fn);
    VINF_TRY(check_f32(fn, "mean_out", mean_out));
    VINF_TRY(check_f32(fn, "rstd_out", rstd_out));
    if (groups < 1 || C % groups) return fail(VINF_ERR_INVALID_ARG, "%s: C=%d not divisible by groups=%d", fn, C, groups);
    if (!(eps >= 0.f)) return fail(VINF_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
    const int vec = dt == VINF_BF16 ? 8 : 4;
    if (C / vec > 1024) return fail(VINF_ERR_UNSUPPORTED, "%s: C=%d exceeds %d", fn, C, 1024 * vec);
    const size_t need = groupnorm_workspace((int64_t)F * H * W, C, groups, dt);
    if (!workspace || workspace_bytes < need)
        return fail(VINF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(VINF_ERR_WORKSPACE, "%s: workspace is not 256-byte aligned", fn);
    const size_t sb = (size_t)groups * sizeof(float);
    if (overlap(workspace, need, x, bytes) || overlap(mean_out, sb, x, bytes) || overlap(rstd_out, sb, x, bytes) ||
        overlap(workspace, need, mean_out, sb) || overlap(workspace, need, rstd_out, sb) ||
        overlap(mean_out, sb, rstd_out, sb))
        return fail(VINF_ERR_INVALID_ARG, "%s: workspace / statistics overlap", fn);
    return launch_groupnorm(x, nullptr, nullptr, nullptr, mean_out, rstd_out, (int64_t)F * H * W, C, groups, eps, dt,
                            workspace, (hipStream_t)stream);
}

// Shared checks of the two clip GroupNorm calls.
static vinf_status check_gn_clip(const char* fn, const void* x, bool need_x, int F, int H, int W, int C, int groups,
                                 int F_total, vinf_dtype dt, void* workspace, size_t workspace_bytes, size_t* bytes,
                                 size_t* need) {
    VINF_TRY(check_shape(fn, F, H, W, C, dt, bytes));
    VINF_TRY(check_tensor(fn, "x", x, need_x));
    if (groups < 1 || C % groups) return fail(VINF_ERR_INVALID_ARG, "%s: C=%d not divisible by groups=%d", fn, C, groups);
    if (F_total < F) return fail(VINF_ERR_INVALID_ARG, "%s: F_total=%d is smaller than the clip's F=%d", fn, F_total, F);
    const int vec = dt == VINF_BF16 ? 8 : 4;
    if (C / vec > 1024) return fail(VINF_ERR_UNSUPPORTED, "%s: C=%d exceeds %d", fn, C, 1024 * vec);
    *need = groupnorm_workspace((int64_t)F * H * W, C, groups, dt);
    if (!workspace || workspace_bytes < *need)
        return fail(VINF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, *need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(VINF_ERR_WORKSPACE, "%s: workspace is not 256-byte aligned", fn);
    if (overlap(workspace, *need, x, *bytes)) return fail(VINF_ERR_INVALID_ARG, "%s: workspace overlaps x", fn);
    return VINF_OK;
}

vinf_status vinf_groupnorm_clip_sums(const void* x, const double* mean_sums, double* sums, int F, int H, int W, int C,
                                     int groups, int F_total, vinf_dtype dt, void* workspace, size_t workspace_bytes,
                                     vinf_stream stream) {
    const char* fn = "vinf_groupnorm_clip_sums";
    size_t bytes, need;
    VINF_TRY(check_gn_clip(fn, x, true, F, H, W, C, groups, F_total, dt, workspace, workspace_bytes, &bytes, &need));
    VINF_TRY(check_f64(fn, "mean_sums", mean_sums, false));
    VINF_TRY(check_f64(fn, "sums", sums, true));
    const size_t sb = (size_t)groups * sizeof(double);
    if (overlap(sums, sb, x, bytes) || overlap(sums, sb, workspace, need) || overlap(sums, sb, mean_sums, sb))
        return fail(VINF_ERR_INVALID_ARG, "%s: sums overlaps x, the workspace or mean_sums", fn);
    const double n_total = (double)F_total * H * W * (C / groups);
    return launch_groupnorm_clip_sums(x, mean_sums, sums, (int64_t)F * H * W, C, groups, n_total, dt, workspace,
                                      (hipStream_t)stream);
}

vinf_status vinf_groupnorm_clip_apply(const void* x, void* y, const float* gamma, const float* beta, const double* sums,
                                      const double* sq_sums, float* mean_out, float* rstd_out, int F, int H, int W,
                                      int C, int groups, int F_total, float eps, vinf_dtype dt, void* workspace,
                                      size_t workspace_bytes, vinf_stream stream) {
    const char* fn = "vinf_groupnorm_clip_apply";
    size_t bytes, need;
    // x == y == NULL: only the statistics (mean_out and rstd_out then required)
    const bool stats_only = !x && !y;
    if (stats_only && (!mean_out || !rstd_out))
        return fail(VINF_ERR_INVALID_ARG, "%s: without x and y, mean_out and rstd_out are required", fn);
    VINF_TRY(check_gn_clip(fn, x, !stats_only, F, H, W, C, groups, F_total, dt, workspace, workspace_bytes, &bytes,
                           &need));
    if (stats_only) bytes = 0;
    VINF_TRY(check_tensor(fn, "y", y, !stats_only));
    VINF_TRY(check_f32(fn, "gamma", gamma));
    VINF_TRY(check_f32(fn, "beta", beta));
    VINF_TRY(check_f32(fn, "mean_out", mean_out));
    VINF_TRY(check_f32(fn, "rstd_out", rstd_out));
    VINF_TRY(check_f64(fn, "sums", sums, true));
    VINF_TRY(check_f64(fn, "sq_sums", sq_sums, true));
    if (!(eps >= 0.f)) return fail(VINF_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
    if (y != x && overlap(x, bytes, y, bytes))
        return fail(VINF_ERR_INVALID_ARG, "%s: y partially overlaps x (only y == x is allowed)", fn);
    const size_t st = (size_t)groups * sizeof(float);
    if (overlap(workspace, need, y, bytes) || overlap(mean_out, st, x, bytes) || overlap(mean_out, st, y, bytes) ||
        overlap(rstd_out, st, x, bytes) || overlap(rstd_out, st, y, bytes) || overlap(workspace, need, mean_out, st) ||
        overlap(workspace, need, rstd_out, st))
        return fail(VINF_ERR_INVALID_ARG, "%s: workspace / statistics overlap a tensor", fn);
    if (overlap(mean_out, st, rstd_out, st)) return fail(VINF_ERR_INVALID_ARG, "%s: mean_out overlaps rstd_out", fn);
    const double n_total = (double)F_total * H * W * (C / groups);
    return launch_groupnorm_clip_apply(x, y, gamma, beta, sums, sq_sums, mean_out, rstd_out, (int64_t)F * H * W, C,
                                       groups, n_total, eps, dt, workspace, (hipStream_t)stream);
}

vinf_status vinf_temporal_conv3(const void* x, const void* ctx_pre, const void* ctx_post, const void* weight,
                                const float* bias, void* y, int F, int H, int W, int C, vinf_dtype dt,
                                vinf_stream stream) {
    const char* fn = "vinf_temporal_conv3";
    size_t bytes;
    VINF_TRY(check_shape(fn, F, H, W, C, dt, &bytes));
    VINF_TRY(check_tensor(fn, "x", x, true));
    VINF_TRY(check_tensor(fn, "y", y, true));
    VINF_TRY(check_tensor(fn, "weight", weight, true));
    VINF_TRY(check_tensor(fn, "ctx_pre", ctx_pre, false));
    VINF_TRY(check_tensor(fn, "ctx_post", ctx_post, false));
    VINF_TRY(check_f32(fn, "bias", bias));
    if (dt == VINF_BF16 && C % 32)
        return fail(VINF_ERR_UNSUPPORTED, "%s: bf16 needs C %% 32 == 0 (MFMA tiles), got C=%d", fn, C);
    const size_t wbytes = (size_t)3 * C * C * dtype_bytes(dt);
    const size_t cbytes = (size_t)H * W * C * dtype_bytes(dt);
    if (overlap(y, bytes, x, bytes) || overlap(y, bytes, weight, wbytes) || overlap(y, bytes, ctx_pre, cbytes) ||
        overlap(y, bytes, ctx_post, cbytes) || overlap(y, bytes, bias, (size_t)C * 4))
        return fail(VINF_ERR_INVALID_ARG, "%s: y overlaps an input", fn);
    return launch_conv3(x, ctx_pre, ctx_post, weight, bias, y, F, H * W, C, dt, (hipStream_t)stream);
}

vinf_status vinf_qkv_project(const void* x, const void* weight, const float* bias, void* q, void* k, void* v,
                             int F, int H, int W, int C, vinf_dtype dt, vinf_stream stream) {
    const char* fn = "vinf_qkv_project";
    size_t bytes;
    VINF_TRY(check_shape(fn, F, H, W, C, dt, &bytes));
    VINF_TRY(check_tensor(fn, "x", x, true));
    VINF_TRY(check_tensor(fn, "weight", weight, true));
    VINF_TRY(check_tensor(fn, "q", q, true));
    VINF_TRY(check_tensor(fn, "k", k, true));
    VINF_TRY(check_tensor(fn, "v", v, true));
    VINF_TRY(check_f32(fn, "bias", bias));
    if (dt == VINF_BF16 && C % 32)
        return fail(VINF_ERR_UNSUPPORTED, "%s: bf16 needs C %% 32 == 0 (MFMA tiles), got C=%d", fn, C);
    const size_t wbytes = (size_t)3 * C * C * dtype_bytes(dt);
    const void* outs[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
        const void* o = outs[i];
        if (overlap(o, bytes, x, bytes) || overlap(o, bytes, weight, wbytes) || overlap(o, bytes, bias, (size_t)3 * C * 4))
            return fail(VINF_ERR_INVALID_ARG, "%s: %c overlaps an input", fn, "qkv"[i]);
        for (int j = 0; j < i; ++j)
            if (overlap(o, bytes, outs[j], bytes))
                return fail(VINF_ERR_INVALID_ARG, "%s: %c overlaps %c", fn, "qkv"[i], "qkv"[j]);
    }
    return launch_qkv_project(x, weight, bias, q, k, v, F, H * W, C, dt, (hipStream_t)stream);
}

size_t vinf_temporal_conv3_gn_workspace_bytes(int C, vinf_dtype dt) {
    if (C < 1 || (dt != VINF_F32 && dt != VINF_BF16)) return 0;
    return conv3_gn_workspace(C, dt);
}

vinf_status vinf_temporal_conv3_gn(const void* x, const void* ctx_pre, const void* ctx_post, const void* weight,
                                   const float* bias, const float* mean, const float* rstd, const float* gamma,
                                   const float* beta, int groups, void* y, int F, int H, int W, int C,
                                   vinf_dtype dt, void* workspace, size_t workspace_bytes, vinf_stream stream) {
    const char* fn = "vinf_temporal_conv3_gn";
    size_t bytes;
    VINF_TRY(check_shape(fn, F, H, W, C, dt, &bytes));
    VINF_TRY(check_tensor(fn, "x", x, true));
    VINF_TRY(check_tensor(fn, "y", y, true));
    VINF_TRY(check_tensor(fn, "weight", weight, true));
    VINF_TRY(check_tensor(fn, "ctx_pre", ctx_pre, false));
    VINF_TRY(check_tensor(fn, "ctx_post", ctx_post, false));
    VINF_TRY(check_f32(fn, "bias", bias));
    VINF_TRY(check_f32(fn, "gamma", gamma));
    VINF_TRY(check_f32(fn, "beta", beta));
    if (!mean || !rstd) return fail(VINF_ERR_INVALID_ARG, "%s: mean and rstd are required", fn);
    VINF_TRY(check_f32(fn, "mean", mean));
    VINF_TRY(check_f32(fn, "rstd", rstd));
    if (groups < 1 || C % groups) return fail(VINF_ERR_INVALID_ARG, "%s: C=%d not divisible by groups=%d", fn, C, groups);
    if (dt == VINF_BF16 && C % 32)
        return fail(VINF_ERR_UNSUPPORTED, "%s: bf16 needs C %% 32 == 0 (MFMA tiles), got C=%d", fn, C);
    const size_t need = conv3_gn_workspace(C, dt);
    if (!workspace || workspace_bytes < need)
        return fail(VINF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(VINF_ERR_WORKSPACE, "%s: workspace is not 256-byte aligned", fn);
    const size_t wbytes = (size_t)3 * C * C * dtype_bytes(dt);
    const size_t cbytes = (size_t)H * W * C * dtype_bytes(dt);
    const size_t gb = (size_t)groups * sizeof(float), vb = (size_t)C * sizeof(float);
    const struct {
        const void* p;
        size_t n;
    } in[] = {{x, bytes}, {ctx_pre, cbytes}, {ctx_post, cbytes}, {weight, wbytes}, {bias, vb},
              {mean, gb}, {rstd, gb}, {gamma, vb}, {beta, vb}};
    for (const auto& r : in) {
        if (overlap(y, bytes, r.p, r.n)) return fail(VINF_ERR_INVALID_ARG, "%s: y overlaps an input", fn);
        if (overlap(workspace, need, r.p, r.n))
            return fail(VINF_ERR_INVALID_ARG, "%s: the workspace overlaps an input", fn);
    }
    if (overlap(workspace, need, y, bytes)) return fail(VINF_ERR_INVALID_ARG, "%s: the workspace overlaps y", fn);
    return launch_conv3_gn(x, ctx_pre, ctx_post, weight, bias, mean, rstd, gamma, beta, groups, y, F, H * W, C, dt,
                           workspace, (hipStream_t)stream);
}

// Shared checks of the attention calls: head layout and key-set sizes.
static vinf_status check_dda_heads(const char* fn, int C, int head_dim, int n_local, int n_global, float scale) {
    if (head_dim != 64) return fail(VINF_ERR_UNSUPPORTED, "%s: head_dim=%d (only 64)", fn, head_dim);
    if (C % head_dim) return fail(VINF_ERR_INVALID_ARG, "%s: C=%d not a multiple of head_dim", fn, C);
    if ((n_local != 16 && n_local != 0) || (n_global != 16 && n_global != 0) || n_local + n_global == 0)
        return fail(VINF_ERR_UNSUPPORTED, "%s: n_local=%d n_global=%d (each 16 or 0, not both 0)", fn, n_local,
                    n_global);
    if (!(scale == scale)) return fail(VINF_ERR_INVALID_ARG, "%s: scale is NaN", fn);
    return VINF_OK;
}

vinf_status vinf_dual_domain_attn(const void* q, const void* k, const void* v, void* o, int F, int H, int W, int C,
                                  int head_dim, int n_local, int n_global, float scale, vinf_dtype dt,
                                  vinf_stream stream) {
    const char* fn = "vinf_dual_domain_attn";
    size_t bytes;
    VINF_TRY(check_shape(fn, F, H, W, C, dt, &bytes));
    VINF_TRY(check_tensor(fn, "q", q, true));
    VINF_TRY(check_tensor(fn, "k", k, true));
    VINF_TRY(check_tensor(fn, "v", v, true));
    VINF_TRY(check_tensor(fn, "o", o, true));
    VINF_TRY(check_dda_heads(fn, C, head_dim, n_local, n_global, scale));
    if (overlap(o, bytes, q, bytes) || overlap(o, bytes, k, bytes) || overlap(o, bytes, v, bytes))
        return fail(VINF_ERR_INVALID_ARG, "%s: o overlaps q, k or v", fn);
    if (scale <= 0.f) scale = 0.125f;  // 1/sqrt(64)
    return launch_dda(q, k, v, nullptr, nullptr, o, F, 0, F, 0, F, H * W, C, n_local, n_global, scale, dt,
                      (hipStream_t)stream);
}

vinf_status vinf_projected_dual_domain_attn(const void* x, const void* weight, const float* bias, void* o, int F,
                                            int H, int W, int C, int head_dim, int n_local, int n_global, float scale,
                                            vinf_dtype dt, vinf_stream stream) {
    const char* fn = "vinf_projected_dual_domain_attn";
    size_t bytes;
    VINF_TRY(check_shape(fn, F, H, W, C, dt, &bytes));
    VINF_TRY(check_tensor(fn, "x", x, true));
    VINF_TRY(check_tensor(fn, "weight", weight, true));
    VINF_TRY(check_tensor(fn, "o", o, true));
    VINF_TRY(check_f32(fn, "bias", bias));
    VINF_TRY(check_dda_heads(fn, C, head_dim, n_local, n_global, scale));
    if (dt != VINF_BF16)
        return fail(VINF_ERR_UNSUPPORTED, "%s: bf16 only (float32: vinf_qkv_project, then vinf_dual_domain_attn)", fn);
    if (n_local != 16 || n_global != 16)
        return fail(VINF_ERR_UNSUPPORTED, "%s: the full key set only (n_local = n_global = 16), got %d and %d", fn,
                    n_local, n_global);
    const size_t wbytes = (size_t)3 * C * C * 2;
    if (overlap(o, bytes, x, bytes) || overlap(o, bytes, weight, wbytes) || overlap(o, bytes, bias, (size_t)3 * C * 4))
        return fail(VINF_ERR_INVALID_ARG, "%s: o overlaps an input", fn);
    if (scale <= 0.f) scale = 0.125f;  // 1/sqrt(64)
    return launch_dda_projected(x, weight, bias, o, F, H * W, C, scale, (hipStream_t)stream);
}

vinf_status vinf_dda_clip_halo(int F_total, int f0, int Fc, int n_local, int* n_pre, int* n_post) {
    const char* fn = "vinf_dda_clip_halo";
    if (!n_pre || !n_post) return fail(VINF_ERR_INVALID_ARG, "%s: NULL output", fn);
    if (F_total < 1 || Fc < 1 || f0 < 0 || (int64_t)f0 + Fc > F_total)
        return fail(VINF_ERR_INVALID_ARG, "%s: clip [%d, %d+%d) not inside a %d-frame video", fn, f0, f0, Fc, F_total);
    if (n_local < 0) return fail(VINF_ERR_INVALID_ARG, "%s: n_local=%d", fn, n_local);
    int64_t pre, post;
    clip_halo(F_total, f0, Fc, n_local, &pre, &post);
    *n_pre = (int)pre;
    *n_post = (int)post;
    return VINF_OK;
}

vinf_status vinf_dual_domain_attn_clip(const void* q, const void* k, const void* v, const void* k_global,
                                       const void* v_global, void* o, int F_total, int f0, int Fc, int n_pre,
                                       int n_post, int H, int W, int C, int head_dim, int n_local, int n_global,
                                       float scale, vinf_dtype dt, vinf_stream stream) {
    const char* fn = "vinf_dual_domain_attn_clip";
    size_t bytes, ext_bytes;
    VINF_TRY(check_shape(fn, Fc, H, W, C, dt, &bytes));
    if (n_pre < 0 || n_post < 0 || (int64_t)n_pre + Fc + n_post > 2147483647)
        return fail(VINF_ERR_INVALID_ARG, "%s: n_pre=%d n_post=%d", fn, n_pre, n_post);
    VINF_TRY(check_shape(fn, n_pre + Fc + n_post, H, W, C, dt, &ext_bytes));
    VINF_TRY(check_tensor(fn, "q", q, true));
    VINF_TRY(check_tensor(fn, "k", k, true));
    VINF_TRY(check_tensor(fn, "v", v, true));
    VINF_TRY(check_tensor(fn, "o", o, true));
    VINF_TRY(check_tensor(fn, "k_global", k_global, false));
    VINF_TRY(check_tensor(fn, "v_global", v_global, false));
    VINF_TRY(check_dda_heads(fn, C, head_dim, n_local, n_global, scale));
    if (f0 < 0 || (int64_t)f0 + Fc > F_total)
        return fail(VINF_ERR_INVALID_ARG, "%s: clip [%d, %d+%d) not inside a %d-frame video", fn, f0, f0, Fc, F_total);
    const int64_t kf0 = (int64_t)f0 - n_pre, kend = (int64_t)f0 + Fc + n_post;
    if (kf0 < 0 || kend > F_total)
        return fail(VINF_ERR_INVALID_ARG, "%s: context frames [%lld, %lld) fall outside the video", fn, (long long)kf0,
                    (long long)kend);
    int64_t need_pre, need_post;
    clip_halo(F_total, f0, Fc, n_local, &need_pre, &need_post);
    if (n_pre < need_pre || n_post < need_post)
        return fail(VINF_ERR_INVALID_ARG, "%s: the local windows need %lld frames before and %lld after, got %d and %d",
                    fn, (long long)need_pre, (long long)need_post, n_pre, n_post);
    if ((k_global == nullptr) != (v_global == nullptr))
        return fail(VINF_ERR_INVALID_ARG, "%s: give both k_global and v_global or neither", fn);
    if (n_global > 0 && !k_global) {
        for (int i = 0; i < n_global; ++i) {
            const int64_t f = (int64_t)i * F_total / n_global;
            if (f < kf0 || f >= kend)
                return fail(VINF_ERR_INVALID_ARG, "%s: global frame %lld is not in k/v and k_global is NULL", fn,
                            (long long)f);
        }
    }
    const size_t gbytes = k_global ? (size_t)(n_global > 0 ? n_global : 16) * H * W * C * dtype_bytes(dt) : 0;
    if (overlap(o, bytes, q, bytes) || overlap(o, bytes, k, ext_bytes) || overlap(o, bytes, v, ext_bytes) ||
        overlap(o, bytes, k_global, gbytes) || overlap(o, bytes, v_global, gbytes))
        return fail(VINF_ERR_INVALID_ARG, "%s: o overlaps an input", fn);
    if (scale <= 0.f) scale = 0.125f;  // 1/sqrt(64)
    return launch_dda(q, k, v, k_global, v_global, o, F_total, f0, Fc, (int)kf0, (int)kend, H * W, C, n_local,
                      n_global, scale, dt, (hipStream_t)stream);
}

vinf_status vinf_attn_broadcast_schedule(int n_steps, int range, unsigned char* recompute) {
    const char* fn = "vinf_attn_broadcast_schedule";
    if (n_steps < 1 || range < 1 || !recompute)
        return fail(VINF_ERR_INVALID_ARG, "%s: n_steps=%d range=%d recompute=%p", fn, n_steps, range,
                    (void*)recompute);
    if (n_steps > 21474836) return fail(VINF_ERR_INVALID_ARG, "%s: n_steps=%d too large", fn, n_steps);
    const int edge = 15 * n_steps / 100;  // steps at each end that always compute
    int since_compute = 0;                // middle-band steps since the last computing one
    for (int i = 0; i < n_steps; ++i) {
        if (i < edge || i >= n_steps - edge) {
            recompute[i] = 1;
            continue;
        }
        if (i == edge || since_compute == range - 1) {
            recompute[i] = 1;
            since_compute = 0;
        } else {
            recompute[i] = 0;
            ++since_compute;
        }
    }
    return VINF_OK;
}

const char* vinf_status_string(vinf_status s) {
    switch (s) {
        case VINF_OK: return "ok";
        case VINF_ERR_INVALID_ARG: return "invalid argument";
        case VINF_ERR_UNSUPPORTED: return "unsupported argument";
        case VINF_ERR_WORKSPACE: return "workspace missing or too small";
        case VINF_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* vinf_last_error(void) { return g_last_error; }

}  // extern "C"

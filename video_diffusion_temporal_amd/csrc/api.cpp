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
    if (head_dim != 64) return fail(VINF_ERR_UNSUPPORTED, "%s: head_dim=%d (only 64)", fn, head_dim);
    if (C % head_dim) return fail(VINF_ERR_INVALID_ARG, "%s: C=%d not a multiple of head_dim", fn, C);
    if (n_local != 16 || n_global != 16)
        return fail(VINF_ERR_UNSUPPORTED, "%s: n_local=%d n_global=%d (only 16 and 16)", fn, n_local, n_global);
    if (!(scale == scale)) return fail(VINF_ERR_INVALID_ARG, "%s: scale is NaN", fn);
    if (overlap(o, bytes, q, bytes) || overlap(o, bytes, k, bytes) || overlap(o, bytes, v, bytes))
        return fail(VINF_ERR_INVALID_ARG, "%s: o overlaps q, k or v", fn);
    if (scale <= 0.f) scale = 0.125f;  // 1/sqrt(64)
    return launch_dda(q, k, v, o, F, H * W, C, scale, dt, (hipStream_t)stream);
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

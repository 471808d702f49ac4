/*
 * libvinf -- the temporal module of a video-diffusion layer, in the form
 * Video-Infinity defines it, as hand-written HIP kernels for gfx950 (MI355X).
 *
 * Source of the method: the write-up of "Video-Infinity: Distributed Long
 * Video Generation" (page "新国立祭出视频生成“无限宝石“：2300帧仅需5分钟，提速100倍").
 * Its temporal modules are Attention (dual-domain), Conv (temporal, with
 * context) and GroupNorm (global statistics); each acts on the frames of
 * every spatial location of a latent [F, H', W', C].  Here the whole video is
 * one clip on one GPU.
 *
 * Conventions shared by every call
 *   Layout     dense, contiguous, channels-last [F][H][W][C]; element
 *              (f, h, w, c) at ((f*H + h)*W + w)*C + c.  No strides.
 *   Types      vinf_dtype selects float32 or bfloat16 for the tensors named
 *              "dt" below; gamma, beta, bias and statistics are float32.
 *              bf16 results are rounded to nearest even from fp32.
 *   Memory     every pointer is device memory owned by the caller; the
 *              library allocates, frees and retains nothing.  Tensor
 *              pointers (x, y, q, k, v, o, weight, ctx_*) must be 16-byte
 *              aligned; float pointers 4-byte aligned.
 *   Streams    `stream` is a hipStream_t (NULL: the null stream).  Calls only
 *              enqueue work and return without synchronising.  The library
 *              holds no state, so calls from several threads are safe.
 *   Errors     arguments are checked on the host before anything is
 *              enqueued; a rejected call returns VINF_ERR_INVALID_ARG or
 *              VINF_ERR_UNSUPPORTED (or VINF_ERR_WORKSPACE) and has no
 *              effect.  A failed launch returns VINF_ERR_HIP.  Faults during
 *              execution surface at the caller's next synchronisation.
 *              vinf_last_error() gives a message for the calling thread's
 *              last failed call.  Nothing throws across this interface.
 */
#ifndef VINF_H
#define VINF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VINF_OK = 0,
    VINF_ERR_INVALID_ARG = 1, /* NULL / non-positive size / misaligned / aliasing / inconsistent */
    VINF_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement */
    VINF_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    VINF_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} vinf_status;

typedef enum { VINF_F32 = 0, VINF_BF16 = 1 } vinf_dtype;

typedef void* vinf_stream; /* a hipStream_t */

/*
 * GroupNorm with statistics over the whole video (GroupNorm-module paragraph:
 * group means first, aggregated to a global mean; then the standard deviation
 * computed with that global mean, aggregated to a global standard deviation).
 *
 *   N_g     = F*H*W*C/groups voxel-channels of group g (channels
 *             [g*C/groups, (g+1)*C/groups))
 *   mean_g  = sum x / N_g                                   (pass 1)
 *   var_g   = sum (x - mean_g)^2 / N_g                      (pass 2, biased)
 *   y       = (x - mean_g) / sqrt(var_g + eps) * gamma_c + beta_c
 *
 * x, y      [F][H][W][C] in dt.  y == x (in place) is allowed; any other
 *           overlap is rejected.
 * gamma,beta  [C] float32 or NULL (1 and 0).
 * mean_out, rstd_out  [groups] float32 or NULL; receive mean_g and
 *           1/sqrt(var_g + eps).
 * workspace device scratch of at least vinf_groupnorm_workspace_bytes(...)
 *           bytes, 256-byte aligned; contents on entry do not matter.
 * Limits    C % groups == 0; C % 8 == 0 (bf16) or C % 4 == 0 (f32);
 *           C <= 8192; eps >= 0.
 * The statistics are summed in a fixed order (per-block fp32 partials, then
 * an fp64 combine), so results are bitwise reproducible run to run.
 */
size_t vinf_groupnorm_workspace_bytes(int F, int H, int W, int C, int groups, vinf_dtype dt);
vinf_status vinf_groupnorm_global(const void* x, void* y, const float* gamma, const float* beta,
                                  float* mean_out, float* rstd_out, int F, int H, int W, int C,
                                  int groups, float eps, vinf_dtype dt, void* workspace,
                                  size_t workspace_bytes, vinf_stream stream);

/*
 * vinf_groupnorm_global for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument and no allocation.  The workspace is a
 * static device array of VINF_NOALLOC_SCRATCH_BYTES inside the library; each
 * GPU the library runs on holds its own copy until the process ends.
 * Arguments, limits and results are those of vinf_groupnorm_global (bit for
 * bit); a shape whose workspace (vinf_groupnorm_workspace_bytes) exceeds
 * VINF_NOALLOC_SCRATCH_BYTES returns VINF_ERR_UNSUPPORTED.  Every call on one
 * GPU uses that GPU's array, so calls that overlap on one GPU (different
 * streams, or host threads) race and must be serialised by the caller; a call
 * writes every byte of it that it reads, so nothing needs clearing between
 * calls.
 */
#define VINF_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
vinf_status vinf_groupnorm_global_noalloc(const void* x, void* y, const float* gamma, const float* beta,
                                          float* mean_out, float* rstd_out, int F, int H, int W, int C,
                                          int groups, float eps, vinf_dtype dt, vinf_stream stream);

/*
 * Temporal convolution, kernel 3, with context padding (Conv-module
 * paragraph: convolution along the frame axis of each spatial location; the
 * clip is padded with the last frames of the previous clip and the first
 * frames of the next one, as many as the receptive field -- one per side for
 * kernel 3).
 *
 *   y[f,h,w,co] = bias[co] + sum_{k=0..2} sum_ci weight[k][co][ci] * xt[f+k-1,h,w,ci]
 *   xt[-1] = ctx_pre, xt[F] = ctx_post (zeros when NULL: the ends of the video)
 *
 * x, y      [F][H][W][C] in dt; y must not overlap x, weight or ctx_*.
 * ctx_pre, ctx_post  [H][W][C] in dt, or NULL.  For a clip of a longer
 *           video they are the previous clip's last frame and the next clip's
 *           first frame; the clip's y then equals the whole video's y for
 *           those frames, bit for bit.
 * weight    [3][C_out=C][C_in=C] in dt (tap k multiplies frame f+k-1; a torch
 *           Conv1d weight [C_out][C_in][3] maps to it by permute(2,0,1)).
 * bias      [C] float32 or NULL.
 * Limits    bf16: C % 32 == 0 (bf16 MFMA tiles); f32: C % 4 == 0.
 */
vinf_status vinf_temporal_conv3(const void* x, const void* ctx_pre, const void* ctx_post,
                                const void* weight, const float* bias, void* y, int F, int H, int W,
                                int C, vinf_dtype dt, vinf_stream stream);

/*
 * GroupNorm statistics only: the two sweeps of vinf_groupnorm_global
 * (mean first, then the deviation about it), writing mean_g and
 * 1/sqrt(var_g + eps) without normalising the tensor.  Arguments, limits and
 * workspace as vinf_groupnorm_global; mean_out and rstd_out are required.
 * The values are bit for bit those vinf_groupnorm_global reports.
 */
vinf_status vinf_groupnorm_stats(const void* x, float* mean_out, float* rstd_out, int F, int H, int W, int C,
                                 int groups, float eps, vinf_dtype dt, void* workspace, size_t workspace_bytes,
                                 vinf_stream stream);

/*
 * The temporal conv of the GroupNorm output, with GroupNorm applied inside
 * the conv (the temporal-modules paragraph puts GroupNorm and Conv in a row;
 * the normalised tensor is never written to memory):
 *
 *   y = conv3(g),  g[f,h,w,c] = x[f,h,w,c] * a_c + b_c,
 *   a_c = rstd_g * gamma_c,  b_c = beta_c - mean_g * a_c   (fp32, rounded to dt)
 *
 * with conv3 as vinf_temporal_conv3.  g is formed and rounded exactly as
 * vinf_groupnorm_global's apply writes it, so the result is bit for bit that
 * of the apply followed by vinf_temporal_conv3.  ctx_pre / ctx_post are raw
 * neighbouring frames, normalised the same way; absent, the pads are zeros of
 * g, as in vinf_temporal_conv3.
 *
 * x, y      [F][H][W][C] in dt (y must not overlap any input).
 * weight    [3][C][C] in dt; bias [C] float32 or NULL.
 * mean, rstd  [groups] float32 (vinf_groupnorm_stats, or
 *           vinf_groupnorm_clip_apply without x for a clip).
 * gamma, beta [C] float32 or NULL (1 and 0).
 * workspace device scratch of vinf_temporal_conv3_gn_workspace_bytes(C, dt)
 *           bytes (the per-channel a_c, b_c), 256-byte aligned, not
 *           overlapping any argument.
 * Limits    as vinf_temporal_conv3; C % groups == 0.
 */
size_t vinf_temporal_conv3_gn_workspace_bytes(int C, vinf_dtype dt);
vinf_status vinf_temporal_conv3_gn(const void* x, const void* ctx_pre, const void* ctx_post,
                                   const void* weight, const float* bias, const float* mean,
                                   const float* rstd, const float* gamma, const float* beta, int groups,
                                   void* y, int F, int H, int W, int C, vinf_dtype dt, void* workspace,
                                   size_t workspace_bytes, vinf_stream stream);

/*
 * Dual-domain temporal attention (dual-domain attention paragraph, and the
 * paragraph that sets both context sizes to 16): at each spatial location and
 * head, query frame t attends over the concatenation of a local context and a
 * global context.
 *
 *   local(t)  = frames st .. st+min(n_local,F)-1,
 *               st = clamp(t - n_local/2, 0, max(F - n_local, 0))
 *               (centred on t, shifted inward at the ends of the video)
 *   global    = frames floor(i*F/n_global), i = 0..n_global-1
 *   J(t)      = local(t) ++ global   (a multiset: a frame in both counts twice)
 *   o[t]      = sum_{j in J(t)} e^{s_j} v[j] / sum_{j in J(t)} e^{s_j},
 *   s_j       = scale * q[t] . k[j]  over the head's head_dim channels
 *
 * q, k, v   [F][H][W][C] in dt, already projected; head h owns channels
 *           [h*head_dim, (h+1)*head_dim).
 * o         [F][H][W][C] in dt, before any output projection; must not
 *           overlap q, k or v.
 * scale     <= 0 selects 1/sqrt(head_dim).
 * Limits    head_dim == 64, C % 64 == 0; n_local and n_global each 16 or 0,
 *           not both 0 (anything else: VINF_ERR_UNSUPPORTED).  F >= 1 (F < 16
 *           uses all F frames as the local context).
 *           n_global == 0 is the local-context-only variant and n_local == 0
 *           the global-context-only variant of the write-up's ablation
 *           paragraph (the key list is then just the other half).
 */
vinf_status vinf_dual_domain_attn(const void* q, const void* k, const void* v, void* o, int F, int H,
                                  int W, int C, int head_dim, int n_local, int n_global, float scale,
                                  vinf_dtype dt, vinf_stream stream);

/*
 * Query, key and value tokens of the attention (dual-domain attention
 * paragraph: the query token comes from frame t, and the keys and values are
 * computed from the tokens of its frame set).  Each is a linear map of every
 * token, with no mixing of frames or locations:
 *
 *   q[f,h,w,co] = bias[0][co] + sum_ci weight[0][co][ci] * x[f,h,w,ci]
 *   k: weight[1], bias[1];  v: weight[2], bias[2]
 *
 * x, q, k, v  [F][H][W][C] in dt; q, k and v must not overlap x, weight,
 *           bias or each other.
 * weight    [3][C_out=C][C_in=C] in dt (a torch Linear weight is [C_out][C_in]).
 * bias      [3][C] float32 or NULL.
 * Limits    bf16: C % 32 == 0 (bf16 MFMA tiles); f32: C % 4 == 0.
 * bf16 runs on the matrix cores (the conv's kernel with one tap and the three
 * maps as three output tiles), fp32 accumulate, rounded to bf16 once.  The
 * attention over the result is vinf_dual_domain_attn(q, k, v, ...).
 */
vinf_status vinf_qkv_project(const void* x, const void* weight, const float* bias, void* q, void* k, void* v,
                             int F, int H, int W, int C, vinf_dtype dt, vinf_stream stream);

/*
 * Dual-domain attention over projected tokens, with the projection inside the
 * attention's work items (dual-domain attention paragraph: the query token
 * comes from frame t, and the keys and values are computed from the tokens
 * of its frame set).  The result is that of
 *
 *   vinf_qkv_project(x, weight, bias, q, k, v, ...)
 *   vinf_dual_domain_attn(q, k, v, o, ..., n_local = 16, n_global = 16, scale)
 *
 * bit for bit (the same bf16 rounding of q, k and v), but q, k and v are
 * never written: each work item (one location, one head, 256 query frames)
 * projects the rows of x its windows and the 16 global frames need, on the
 * matrix cores, straight into the attention's LDS layout.
 *
 * x, o      [F][H][W][C] bf16; o must not overlap x, weight or bias.
 * weight    [3][C_out=C][C_in=C] bf16 (the q, k and v maps).
 * bias      [3][C] float32 or NULL.
 * scale     <= 0 selects 1/sqrt(head_dim).
 * Limits    bf16 only, head_dim == 64, C % 64 == 0, n_local == n_global == 16
 *           (anything else: VINF_ERR_UNSUPPORTED; the two calls above cover
 *           float32 and the ablation key sets).
 */
vinf_status vinf_projected_dual_domain_attn(const void* x, const void* weight, const float* bias, void* o, int F,
                                            int H, int W, int C, int head_dim, int n_local, int n_global, float scale,
                                            vinf_dtype dt, vinf_stream stream);

/*
 * GroupNorm of one clip with statistics over the whole video (the clip-
 * parallelism paragraph: each device holds a clip and its temporal modules
 * exchange context; for GroupNorm the context is the aggregated statistics
 * of the GroupNorm-module paragraph).  Per clip, in this order:
 *
 *   1. vinf_groupnorm_clip_sums(x, NULL, s1)  s1[g] = sum of x over the clip
 *   2. caller: S1 = sum of s1 over all clips (e.g. an fp64 all-reduce)
 *   3. vinf_groupnorm_clip_sums(x, S1, s2)   s2[g] = sum of (x - mean_g)^2,
 *                                             mean_g = S1[g] / N_g
 *   4. caller: S2 = sum of s2 over all clips
 *   5. vinf_groupnorm_clip_apply(x, y, ..., S1, S2)
 *        y = (x - mean_g) / sqrt(S2[g]/N_g + eps) * gamma_c + beta_c
 *
 *   N_g = F_total*H*W*C/groups, F_total = the frames of all clips together.
 *
 * x, y      [F][H][W][C] in dt: this clip's F frames (y == x allowed).
 * mean_sums, sums, sq_sums  [groups] float64 device arrays (8-byte aligned);
 *           mean_sums NULL selects step 1.  sums must not overlap x, the
 *           workspace or mean_sums.
 * gamma, beta, mean_out, rstd_out, eps, workspace: as vinf_groupnorm_global,
 *           with the workspace sized by vinf_groupnorm_workspace_bytes for
 *           this clip's F.
 * vinf_groupnorm_clip_apply with x and y both NULL writes only mean_out and
 *           rstd_out (both required then), e.g. for vinf_temporal_conv3_gn.
 * The sums and statistics use the same kernels and expressions as
 * vinf_groupnorm_global, so a single clip with F_total == F gives the same
 * bits as that call.
 */
vinf_status vinf_groupnorm_clip_sums(const void* x, const double* mean_sums, double* sums, int F, int H, int W,
                                     int C, int groups, int F_total, vinf_dtype dt, void* workspace,
                                     size_t workspace_bytes, vinf_stream stream);
vinf_status vinf_groupnorm_clip_apply(const void* x, void* y, const float* gamma, const float* beta,
                                      const double* sums, const double* sq_sums, float* mean_out,
                                      float* rstd_out, int F, int H, int W, int C, int groups, int F_total,
                                      float eps, vinf_dtype dt, void* workspace, size_t workspace_bytes,
                                      vinf_stream stream);

/*
 * Context a clip needs for the local keys of its queries: the clip holds
 * frames f0 .. f0+Fc-1 of an F_total-frame video; *n_pre / *n_post receive
 * how many frames before f0 and after f0+Fc-1 its local windows reach
 * (8 and 7 for an interior clip of >= 16 frames; up to 15 next to the ends
 * of the video, where windows shift inward; 0 and 0 when n_local == 0).
 * Host only: touches no device state.
 */
vinf_status vinf_dda_clip_halo(int F_total, int f0, int Fc, int n_local, int* n_pre, int* n_post);

/*
 * Dual-domain attention of one clip (the clip-parallel form: the clip's own
 * frames plus the previous clip's and next clip's edge frames as local
 * context and the global context frames gathered from all clips).  Computes
 * vinf_dual_domain_attn of the whole video restricted to query frames
 * f0 .. f0+Fc-1, bit for bit, from:
 *
 * q, o      [Fc][H][W][C] in dt (frames f0 .. f0+Fc-1).
 * k, v      [n_pre + Fc + n_post][H][W][C] in dt: frames f0-n_pre ..
 *           f0+Fc+n_post-1, the clip's rows with the neighbours' rows in
 *           place before and after.  n_pre / n_post must be at least what
 *           vinf_dda_clip_halo reports, and the frames must lie in the video.
 * k_global, v_global  [n_global][H][W][C] in dt: frames floor(i*F_total/16),
 *           i = 0..15, of the video's K and V; or both NULL, when k and v
 *           hold all of those frames (e.g. the whole video).
 * Other arguments, limits and errors as vinf_dual_domain_attn.  o must not
 *           overlap any input.
 */
vinf_status vinf_dual_domain_attn_clip(const void* q, const void* k, const void* v, const void* k_global,
                                       const void* v_global, void* o, int F_total, int f0, int Fc, int n_pre,
                                       int n_post, int H, int W, int C, int head_dim, int n_local,
                                       int n_global, float scale, vinf_dtype dt, vinf_stream stream);

/*
 * Reuse of temporal-attention outputs across diffusion steps (the Pyramid
 * Attention Broadcast page, implementation section: the attention output
 * changes markedly between consecutive steps only in the first and last 15%
 * of a schedule; in the middle 70% one step's output is broadcast to the
 * following steps).  Fills recompute[0 .. n_steps-1] with 1 for a step (in
 * sampling order) that computes its attention and 0 for a step that reuses the
 * latest computed output:
 *
 *   edge = floor(15 * n_steps / 100) steps at each end always compute;
 *   in the middle band [edge, n_steps - edge) the steps edge, edge + range,
 *   edge + 2*range, ... compute.
 *
 * range 1 computes every step.  Host only: a reuse step launches nothing, the
 * caller keeps the last output (calls vinf_dual_domain_attn with the same o on
 * computing steps only).  Errors: n_steps < 1, range < 1, recompute NULL.
 */
vinf_status vinf_attn_broadcast_schedule(int n_steps, int range, unsigned char* recompute);

/* Static description of a status code. */
const char* vinf_status_string(vinf_status s);

/* Detail of the calling thread's last failed call ("" if none). */
const char* vinf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VINF_H */

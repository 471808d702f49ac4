/*
 * CPU oracle of the Video-Infinity temporal module -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load
 * this library.  It shares no code with the HIP path.  Every routine is the
 * plain definition of what the temporal module computes, in fp64, following
 * the write-up of "Video-Infinity: Distributed Long Video Generation" (page
 * "新国立祭出视频生成“无限宝石“：2300帧仅需5分钟，提速100倍"):
 *   - oracle_gn_stats / oracle_groupnorm: the GroupNorm-module paragraph
 *     (group means first, aggregated to a global mean; then the standard
 *     deviation computed with that global mean);
 *   - oracle_conv3: the Conv-module paragraph (convolution along frames, the
 *     sequence padded with the neighbouring clip's frames, n = receptive field);
 *   - oracle_dda: the dual-domain attention paragraph and the paragraph that
 *     sets both context sizes to 16 (local neighbour frames + frames sampled
 *     uniformly over the whole video);
 *   - oracle_chain: the three temporal modules in a row (the paragraph that
 *     lists Attention, Conv and GroupNorm as the temporal modules);
 *   - oracle_qkv_project / oracle_qkv_dda: the query, key and value tokens the
 *     dual-domain attention paragraph computes from the layer's tokens (a
 *     linear map each), and the attention over them;
 *   - oracle_broadcast_schedule: the output-reuse schedule of the Pyramid
 *     Attention Broadcast page (implementation section);
 *   - oracle_gn_clip_sums / oracle_dda_clip: the clip-parallel form (the
 *     clip-parallelism paragraph: each device's temporal module maps its clip
 *     plus context from the previous clip, the next clip and a global context
 *     to its output), with the GroupNorm and attention paragraphs above.
 * Readings of points the page leaves open are stated at each function.
 *
 * Tensors are dense channels-last [F][S][C] (S = H*W spatial locations), given
 * as float32 (dt = 0), bf16 bit patterns (dt = 1) or float64 (dt = 2: an
 * unrounded intermediate, such as the exact GroupNorm output); inputs are
 * widened exactly to double.  oracle_chain takes dt 0 or 1 only.  Outputs are double, for a list of spatial locations
 * `locs` (n_locs entries), laid out [F][n_locs][C].  Temporal modules act on
 * each spatial location independently, so a location subset is exact.
 *
 * Return value: 0 on success, nonzero on a bad argument.
 * nthreads <= 0 uses every online core, at most 16.
 */
#ifndef VINF_ORACLE_H
#define VINF_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Global per-group statistics over all F*S voxels of the group's channels.
 * mean[g] = sum x / N_g;  var[g] = sum (x - mean[g])^2 / N_g (biased);
 * rstd[g] = 1 / sqrt(var[g] + eps).  Any of mean/var/rstd may be NULL. */
int oracle_gn_stats(const void* x, int dt, int64_t F, int64_t S, int64_t C, int64_t G, double eps,
                    double* mean, double* var, double* rstd, int nthreads);

/* y = (x - mean_g) * rstd_g * gamma_c + beta_c at the given locations.
 * gamma/beta may be NULL (1 and 0).  mean/rstd outputs may be NULL. */
int oracle_groupnorm(const void* x, int dt, int64_t F, int64_t S, int64_t C, int64_t G, double eps,
                     const double* gamma, const double* beta, const int64_t* locs, int64_t n_locs,
                     double* y, double* mean, double* rstd, int nthreads);

/* One clip's share of the GroupNorm sums: sums[g] = sum of x over the clip's
 * F*S voxels and group g's channels (mean == NULL, first pass), or of
 * (x - mean[g])^2 (second pass, mean = the global means).  Summed over all
 * clips and divided by the whole video's N_g they give mean_g and var_g. */
int oracle_gn_clip_sums(const void* x, int dt, int64_t F, int64_t S, int64_t C, int64_t G, const double* mean,
                        double* sums, int nthreads);

/* y[f,s,co] = bias[co] + sum_{k=0..2} sum_ci w[k][co][ci] * xt[f+k-1, s, ci],
 * xt[-1] = ctx_pre (or 0 if NULL), xt[F] = ctx_post (or 0 if NULL).
 * w is [3][C][C] in dt; ctx_* are [S][C] in dt; bias is [C] double or NULL. */
int oracle_conv3(const void* x, const void* ctx_pre, const void* ctx_post, const void* w,
                 const double* bias, int dt, int64_t F, int64_t S, int64_t C, const int64_t* locs,
                 int64_t n_locs, double* y, int nthreads);

/* Key frames of query frame t: local frames st .. st+min(L,F)-1 with
 * st = clamp(t - L/2, 0, max(F-L, 0)), then global frames floor(i*F/Gk),
 * i = 0..Gk-1.  Writes min(L,F)+Gk frame indices to keys (a multiset: a frame
 * in both lists appears twice).  Returns the count. */
int oracle_dda_keys(int64_t F, int64_t t, int n_local, int n_global, int64_t* keys);

/* o[t,s,h*dh+d] = sum_j e^{s_j - m} v[j,s,h*dh+d] / sum_j e^{s_j - m}, j over
 * the key multiset of t, s_j = scale * q[t,s,h] . k[j,s,h], m = max_j s_j.
 * Heads are contiguous head_dim-channel slices; C % head_dim == 0. */
int oracle_dda(const void* q, const void* k, const void* v, int dt, int64_t F, int64_t S, int64_t C,
               int head_dim, int n_local, int n_global, double scale, const int64_t* locs,
               int64_t n_locs, double* o, int nthreads);

/* Attention of one clip of an F_total-frame video (the clip-parallel form of
 * the temporal module: a clip's frames plus context taken from the others).
 * Query frames f0 .. f0+Fc-1; q and o are [Fc][S][C] / [Fc][n_locs][C].
 * k and v are [n_ext][S][C] holding frames kf0 .. kf0+n_ext-1.  k_glob and
 * v_glob are [n_global][S][C] holding frames floor(i*F_total/n_global), or
 * both NULL: the global rows are then read from k and v.  The key multiset is
 * oracle_dda_keys(F_total, t, ...).  Returns 3 when a key frame read from k/v
 * is not among their frames. */
int oracle_dda_clip(const void* q, const void* k, const void* v, const void* k_glob, const void* v_glob, int dt,
                    int64_t F_total, int64_t f0, int64_t Fc, int64_t kf0, int64_t n_ext, int64_t S, int64_t C,
                    int head_dim, int n_local, int n_global, double scale, const int64_t* locs, int64_t n_locs,
                    double* o, int nthreads);

/* GroupNorm (identity affine) -> round to dt -> conv3 (zero padded, no bias)
 * -> round to dt -> dual-domain attention with Q = K = V = the conv output.
 * round_gn == 0 skips the first rounding: the conv reads the exact GroupNorm
 * output (GroupNorm folded into the conv, no GroupNorm tensor in between).
 * gn_out / conv_out ([F][n_locs][C], the values the next module reads) and
 * gn_exact / conv_exact (the same before rounding) may be NULL. */
int oracle_chain(const void* x, const void* w, int dt, int64_t F, int64_t S, int64_t C, int64_t G,
                 double eps, int head_dim, int n_local, int n_global, double scale, int round_gn,
                 const int64_t* locs, int64_t n_locs, double* out, double* gn_out, double* conv_out,
                 double* gn_exact, double* conv_exact, double* mean, double* rstd, int nthreads);

/* Q, K and V tokens (the dual-domain attention paragraph: the query token of
 * frame t, keys and values computed from the tokens of its frame set):
 * out[p][f][s][co] = bias[p][co] + sum_ci w[p][co][ci] * x[f][s][ci] for
 * p = 0, 1, 2 (Q, K, V).  w is [3][C][C] in dt, bias [3][C] double or NULL;
 * out is [3][F][n_locs][C]. */
int oracle_qkv_project(const void* x, const void* w, const double* bias, int dt, int64_t F, int64_t S, int64_t C,
                       const int64_t* locs, int64_t n_locs, double* out, int nthreads);

/* oracle_qkv_project -> round Q, K and V to dt -> dual-domain attention.
 * qkv_out ([3][F][n_locs][C], the rounded values the attention reads) may be
 * NULL.  dt 0 or 1 only. */
int oracle_qkv_dda(const void* x, const void* w, const double* bias, int dt, int64_t F, int64_t S, int64_t C,
                   int head_dim, int n_local, int n_global, double scale, const int64_t* locs, int64_t n_locs,
                   double* out, double* qkv_out, int nthreads);

/* Which diffusion steps compute their temporal attention and which reuse the
 * latest computed output (the Pyramid Attention Broadcast page, implementation
 * section): every step in the first and last floor(15% * n_steps) steps
 * computes; in the middle band the first step and every range-th step after it
 * compute.  recompute[n_steps] receives 1 / 0. */
int oracle_broadcast_schedule(int n_steps, int range, unsigned char* recompute);

/* Round a double to the nearest value representable in dt (ties to even). */
double oracle_round_to(double v, int dt);

#ifdef __cplusplus
}
#endif
#endif

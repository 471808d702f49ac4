/*
 * CPU oracle of the Video-Infinity temporal module -- TEST INFRASTRUCTURE ONLY
 * (see oracle.h for scope, layout and the passages each routine follows).
 *
 * Plain fp64 loops.  Threads only split independent work (voxel ranges for
 * the GroupNorm sums, spatial locations for the conv and the attention);
 * per-thread fp64 partial sums are combined in thread order.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---- helpers ---------------------------------------------------------- */

static double load(const void* p, int dt, int64_t i) {
    if (dt == 2) return ((const double*)p)[i];
    if (dt == 0) return (double)((const float*)p)[i];
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double oracle_round_to(double v, int dt) {
    if (dt == 2) return v;
    if (dt == 0) return (double)(float)v;
    /* bf16 keeps 8 significant bits: v = m * 2^e with 0.5 <= |m| < 1, so the
     * nearest bf16 is nearbyint(m * 2^8) * 2^(e-8) (ties to even under the
     * default rounding mode).  Only the normal range is needed here. */
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    double m = frexp(v, &e);
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

static int resolve_threads(int nthreads) {
    if (nthreads <= 0) { /* default: every online core, at most 16 */
        nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
        if (nthreads > 16) nthreads = 16;
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    return nthreads;
}

typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end, int tid);
typedef struct {
    range_fn fn;
    void* ctx;
    int64_t begin, end;
    int tid;
} range_job;

static void* range_trampoline(void* p) {
    range_job* j = (range_job*)p;
    j->fn(j->ctx, j->begin, j->end, j->tid);
    return NULL;
}

/* Split [0, n) into nthreads contiguous ranges; thread t gets range t. */
static void parallel_ranges(int64_t n, int nthreads, range_fn fn, void* ctx) {
    pthread_t th[256];
    range_job jobs[256];
    int made[256];
    int64_t chunk = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        int64_t b = chunk * t, e = b + chunk;
        if (b > n) b = n;
        if (e > n) e = n;
        jobs[t] = (range_job){fn, ctx, b, e, t};
        made[t] = t < nthreads - 1 && pthread_create(&th[t], NULL, range_trampoline, &jobs[t]) == 0;
        if (!made[t]) fn(ctx, b, e, t);
    }
    for (int t = 0; t < nthreads; ++t)
        if (made[t]) pthread_join(th[t], NULL);
}

/* ---- GroupNorm with global statistics --------------------------------- */
/* Group g owns the contiguous channels [g*C/G, (g+1)*C/G).  First pass: the
 * mean of each group over every voxel of the whole video.  Second pass: the
 * mean squared deviation from that global mean (population variance, divided
 * by N_g).  eps is added inside the square root. */

typedef struct {
    const void* x;
    int dt;
    int64_t C, G, cg;
    const double* mean; /* NULL in the first pass */
    double* partial;    /* [nthreads][G] */
} gn_ctx;

static void gn_pass(void* vctx, int64_t r0, int64_t r1, int tid) {
    gn_ctx* c = (gn_ctx*)vctx;
    double* acc = c->partial + (int64_t)tid * c->G;
    for (int64_t g = 0; g < c->G; ++g) acc[g] = 0.0;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t ch = 0; ch < c->C; ++ch) {
            int64_t g = ch / c->cg;
            double v = load(c->x, c->dt, r * c->C + ch);
            if (c->mean) {
                double d = v - c->mean[g];
                acc[g] += d * d;
            } else {
                acc[g] += v;
            }
        }
    }
}

int oracle_gn_stats(const void* x, int dt, int64_t F, int64_t S, int64_t C, int64_t G, double eps,
                    double* mean, double* var, double* rstd, int nthreads) {
    if (!x || dt < 0 || dt > 2 || F < 1 || S < 1 || C < 1 || G < 1 || C % G) return 1;
    nthreads = resolve_threads(nthreads);
    int64_t rows = F * S, cg = C / G;
    double n_g = (double)rows * (double)cg;
    double* partial = (double*)calloc((size_t)nthreads * (size_t)G, sizeof(double));
    double* mu = (double*)calloc((size_t)G, sizeof(double));
    if (!partial || !mu) {
        free(partial);
        free(mu);
        return 2;
    }
    gn_ctx c = {x, dt, C, G, cg, NULL, partial};
    parallel_ranges(rows, nthreads, gn_pass, &c);
    for (int64_t g = 0; g < G; ++g) {
        double s = 0.0;
        for (int t = 0; t < nthreads; ++t) s += partial[(int64_t)t * G + g];
        mu[g] = s / n_g;
    }
    c.mean = mu;
    parallel_ranges(rows, nthreads, gn_pass, &c);
    for (int64_t g = 0; g < G; ++g) {
        double s = 0.0;
        for (int t = 0; t < nthreads; ++t) s += partial[(int64_t)t * G + g];
        double v = s / n_g;
        if (mean) mean[g] = mu[g];
        if (var) var[g] = v;
        if (rstd) rstd[g] = 1.0 / sqrt(v + eps);
    }
    free(partial);
    free(mu);
    return 0;
}

/* One clip's share of the two sums (the per-device step before the
 * aggregation across devices): sums[g] = sum over the clip's voxels of x
 * (mean == NULL) or of (x - mean[g])^2. */
int oracle_gn_clip_sums(const void* x, int dt, int64_t F, int64_t S, int64_t C, int64_t G, const double* mean,
                        double* sums, int nthreads) {
    if (!x || !sums || dt < 0 || dt > 2 || F < 1 || S < 1 || C < 1 || G < 1 || C % G) return 1;
    nthreads = resolve_threads(nthreads);
    double* partial = (double*)calloc((size_t)nthreads * (size_t)G, sizeof(double));
    if (!partial) return 2;
    gn_ctx c = {x, dt, C, G, C / G, mean, partial};
    parallel_ranges(F * S, nthreads, gn_pass, &c);
    for (int64_t g = 0; g < G; ++g) {
        double s = 0.0;
        for (int t = 0; t < nthreads; ++t) s += partial[(int64_t)t * G + g];
        sums[g] = s;
    }
    free(partial);
    return 0;
}

int oracle_groupnorm(const void* x, int dt, int64_t F, int64_t S, int64_t C, int64_t G, double eps,
                     const double* gamma, const double* beta, const int64_t* locs, int64_t n_locs,
                     double* y, double* mean, double* rstd, int nthreads) {
    if (!y || !locs || n_locs < 0) return 1;
    double* mu = (double*)malloc(sizeof(double) * (size_t)G);
    double* rs = (double*)malloc(sizeof(double) * (size_t)G);
    if (!mu || !rs) {
        free(mu);
        free(rs);
        return 2;
    }
    int rc = oracle_gn_stats(x, dt, F, S, C, G, eps, mu, NULL, rs, nthreads);
    if (rc == 0) {
        int64_t cg = C / G;
        for (int64_t f = 0; f < F; ++f)
            for (int64_t li = 0; li < n_locs; ++li) {
                int64_t s = locs[li];
                for (int64_t ch = 0; ch < C; ++ch) {
                    int64_t g = ch / cg;
                    double v = load(x, dt, (f * S + s) * C + ch);
                    double o = (v - mu[g]) * rs[g];
                    if (gamma) o *= gamma[ch];
                    if (beta) o += beta[ch];
                    y[(f * n_locs + li) * C + ch] = o;
                }
            }
        for (int64_t g = 0; g < G; ++g) {
            if (mean) mean[g] = mu[g];
            if (rstd) rstd[g] = rs[g];
        }
    }
    free(mu);
    free(rs);
    return rc;
}

/* ---- Temporal convolution, kernel 3, context padded ------------------- */
/* The frame sequence of one spatial location is extended by one frame on each
 * side (the receptive field of a kernel-3 convolution is one frame per side):
 * the frame before the first is ctx_pre (zeros when absent, i.e. at the start
 * of the whole video) and the frame after the last is ctx_post.  Tap k
 * multiplies frame f+k-1 (cross-correlation order). */

typedef struct {
    const void *x, *pre, *post, *w;
    const double* bias;
    int dt;
    int64_t F, S, C, n_locs;
    const int64_t* locs;
    double* y;
} conv_ctx;

static void conv_locs(void* vctx, int64_t l0, int64_t l1, int tid) {
    (void)tid;
    conv_ctx* c = (conv_ctx*)vctx;
    int64_t F = c->F, S = c->S, C = c->C;
    double* col = (double*)malloc(sizeof(double) * (size_t)((F + 2) * C));
    double* wd = (double*)malloc(sizeof(double) * (size_t)(3 * C * C));
    if (!col || !wd) abort();
    for (int64_t i = 0; i < 3 * C * C; ++i) wd[i] = load(c->w, c->dt, i);
    for (int64_t li = l0; li < l1; ++li) {
        int64_t s = c->locs[li];
        /* col[f+1] holds padded frame f, f = -1 .. F */
        for (int64_t ch = 0; ch < C; ++ch) {
            col[ch] = c->pre ? load(c->pre, c->dt, s * C + ch) : 0.0;
            col[(F + 1) * C + ch] = c->post ? load(c->post, c->dt, s * C + ch) : 0.0;
        }
        for (int64_t f = 0; f < F; ++f)
            for (int64_t ch = 0; ch < C; ++ch) col[(f + 1) * C + ch] = load(c->x, c->dt, (f * S + s) * C + ch);
        for (int64_t f = 0; f < F; ++f)
            for (int64_t co = 0; co < C; ++co) {
                double acc = c->bias ? c->bias[co] : 0.0;
                for (int64_t k = 0; k < 3; ++k) {
                    const double* xr = col + (f + k) * C; /* padded frame (f + k - 1) */
                    const double* wr = wd + (k * C + co) * C;
                    for (int64_t ci = 0; ci < C; ++ci) acc += wr[ci] * xr[ci];
                }
                c->y[(f * c->n_locs + li) * C + co] = acc;
            }
    }
    free(col);
    free(wd);
}

int oracle_conv3(const void* x, const void* ctx_pre, const void* ctx_post, const void* w,
                 const double* bias, int dt, int64_t F, int64_t S, int64_t C, const int64_t* locs,
                 int64_t n_locs, double* y, int nthreads) {
    if (!x || !w || !y || !locs || dt < 0 || dt > 2 || F < 1 || S < 1 || C < 1 || n_locs < 0) return 1;
    for (int64_t i = 0; i < n_locs; ++i)
        if (locs[i] < 0 || locs[i] >= S) return 1;
    nthreads = resolve_threads(nthreads);
    if (nthreads > n_locs) nthreads = n_locs > 0 ? (int)n_locs : 1;
    conv_ctx c = {x, ctx_pre, ctx_post, w, bias, dt, F, S, C, n_locs, locs, y};
    parallel_ranges(n_locs, nthreads, conv_locs, &c);
    return 0;
}

/* ---- Dual-domain attention -------------------------------------------- */
/* Every query frame t attends over a key/value frame set that concatenates a
 * local context (its neighbouring frames) and a global context (frames
 * sampled uniformly over the whole video), each of size 16.  Readings:
 *   local: min(L,F) consecutive frames starting at clamp(t - L/2, 0, F - L),
 *          i.e. L/2 frames before t, t itself and L/2-1 after, shifted inward
 *          at the ends of the video;
 *   global: frames floor(i*F/Gk), i = 0..Gk-1;
 *   the set is the concatenation of both lists (a multiset of min(L,F)+Gk
 *   entries), so a frame in both lists carries two softmax terms;
 *   scores are scale * q.k per head of head_dim contiguous channels, with no
 *   bias or mask; softmax is exact (max-subtracted) in double. */

int oracle_dda_keys(int64_t F, int64_t t, int n_local, int n_global, int64_t* keys) {
    int64_t L = n_local, nl = L < F ? L : F;
    int64_t hi = F - L > 0 ? F - L : 0;
    int64_t st = t - L / 2;
    if (st < 0) st = 0;
    if (st > hi) st = hi;
    int n = 0;
    for (int64_t i = 0; i < nl; ++i) keys[n++] = st + i;
    for (int64_t i = 0; i < n_global; ++i) keys[n++] = (i * F) / n_global;
    return n;
}

/* The video is F frames long; the query frames are f0 .. f0+Fc-1 (q and o
 * row 0 is frame f0); k and v hold the n_ext frames kf0 .. kf0+n_ext-1 (row 0
 * is frame kf0).  The global rows come from kg, vg (row i holds frame
 * floor(i*F/Gk)) or, when those are NULL, from k and v themselves.  The whole
 * video is the case f0 = kf0 = 0, Fc = n_ext = F, kg = vg = NULL. */
typedef struct {
    const void *q, *k, *v, *kg, *vg;
    int dt;
    int64_t F, f0, Fc, kf0, n_ext, S, C, n_locs;
    int dh, L, Gk;
    double scale;
    const int64_t* locs;
    double* o;
} dda_ctx;

/* Element (row of key j, location s, channel ch) of k (want_v = 0) or v. */
static double dda_kv(const dda_ctx* c, int want_v, const int64_t* keys, int nl, int j, int64_t s, int64_t ch) {
    const void* ext = want_v ? c->v : c->k;
    const void* glob = want_v ? c->vg : c->kg;
    int64_t row = (j >= nl && glob) ? (int64_t)(j - nl) : keys[j] - c->kf0;
    const void* base = (j >= nl && glob) ? glob : ext;
    return load(base, c->dt, (row * c->S + s) * c->C + ch);
}

static void dda_locs(void* vctx, int64_t l0, int64_t l1, int tid) {
    (void)tid;
    dda_ctx* c = (dda_ctx*)vctx;
    int64_t S = c->S, C = c->C;
    int nmax = c->L + c->Gk;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)nmax);
    double* sc = (double*)malloc(sizeof(double) * (size_t)nmax);
    double* acc = (double*)malloc(sizeof(double) * (size_t)c->dh);
    if (!keys || !sc || !acc) abort();
    const int nl = (int)(c->L < c->F ? c->L : c->F);
    for (int64_t li = l0; li < l1; ++li) {
        int64_t s = c->locs[li];
        for (int64_t h = 0; h < C / c->dh; ++h) {
            int64_t c0 = h * c->dh;
            for (int64_t i = 0; i < c->Fc; ++i) {
                int64_t t = c->f0 + i;
                int n = oracle_dda_keys(c->F, t, c->L, c->Gk, keys);
                double m = -INFINITY;
                for (int j = 0; j < n; ++j) {
                    double d = 0.0;
                    for (int e = 0; e < c->dh; ++e)
                        d += load(c->q, c->dt, (i * S + s) * C + c0 + e) * dda_kv(c, 0, keys, nl, j, s, c0 + e);
                    sc[j] = c->scale * d;
                    if (sc[j] > m) m = sc[j];
                }
                double den = 0.0;
                for (int e = 0; e < c->dh; ++e) acc[e] = 0.0;
                for (int j = 0; j < n; ++j) {
                    double p = exp(sc[j] - m);
                    den += p;
                    for (int e = 0; e < c->dh; ++e) acc[e] += p * dda_kv(c, 1, keys, nl, j, s, c0 + e);
                }
                for (int e = 0; e < c->dh; ++e) c->o[(i * c->n_locs + li) * C + c0 + e] = acc[e] / den;
            }
        }
    }
    free(keys);
    free(sc);
    free(acc);
}

static int dda_run(dda_ctx* c, int nthreads) {
    if (!c->q || !c->k || !c->v || !c->o || !c->locs || c->dt < 0 || c->dt > 2 || c->F < 1 || c->S < 1 ||
        c->C < 1 || c->dh < 1 || c->C % c->dh || c->L < 0 || c->Gk < 0 || c->L + c->Gk < 1 || c->n_locs < 0 ||
        (!c->kg) != (!c->vg))
        return 1;
    if (c->f0 < 0 || c->Fc < 1 || c->f0 + c->Fc > c->F || c->kf0 < 0 || c->n_ext < 1 || c->kf0 + c->n_ext > c->F)
        return 1;
    for (int64_t i = 0; i < c->n_locs; ++i)
        if (c->locs[i] < 0 || c->locs[i] >= c->S) return 1;
    /* every key row read from k and v must be one of their n_ext frames */
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(c->L + c->Gk));
    if (!keys) return 2;
    const int64_t nl = c->L < c->F ? c->L : c->F;
    int missing = 0;
    for (int64_t t = c->f0; t < c->f0 + c->Fc && !missing; ++t) {
        int n = oracle_dda_keys(c->F, t, c->L, c->Gk, keys);
        for (int j = 0; j < n; ++j) {
            if (j >= nl && c->kg) continue;
            if (keys[j] < c->kf0 || keys[j] >= c->kf0 + c->n_ext) missing = 1;
        }
    }
    free(keys);
    if (missing) return 3;
    if (c->scale <= 0.0) c->scale = 1.0 / sqrt((double)c->dh);
    nthreads = resolve_threads(nthreads);
    if (nthreads > c->n_locs) nthreads = c->n_locs > 0 ? (int)c->n_locs : 1;
    parallel_ranges(c->n_locs, nthreads, dda_locs, c);
    return 0;
}

int oracle_dda(const void* q, const void* k, const void* v, int dt, int64_t F, int64_t S, int64_t C,
               int head_dim, int n_local, int n_global, double scale, const int64_t* locs,
               int64_t n_locs, double* o, int nthreads) {
    dda_ctx c = {q, k, v, NULL, NULL, dt, F, 0, F, 0, F, S, C, n_locs, head_dim, n_local, n_global, scale, locs, o};
    return dda_run(&c, nthreads);
}

int oracle_dda_clip(const void* q, const void* k, const void* v, const void* k_glob, const void* v_glob, int dt,
                    int64_t F_total, int64_t f0, int64_t Fc, int64_t kf0, int64_t n_ext, int64_t S, int64_t C,
                    int head_dim, int n_local, int n_global, double scale, const int64_t* locs, int64_t n_locs,
                    double* o, int nthreads) {
    dda_ctx c = {q, k, v, k_glob, v_glob, dt, F_total, f0, Fc, kf0, n_ext, S, C, n_locs,
                 head_dim, n_local, n_global, scale, locs, o};
    return dda_run(&c, nthreads);
}

/* ---- Query, key and value tokens ------------------------------------- */
/* The attention takes the query token from frame t and computes the key and
 * value tokens from the tokens of its frame set.  The plain reading is the
 * usual attention layer's three linear maps of each token, with no mixing of
 * frames or locations: out[p][f][s][co] = bias[p][co] + sum_ci
 * w[p][co][ci] * x[f][s][ci], p = 0, 1, 2 for Q, K, V. */

typedef struct {
    const void *x, *w;
    const double* bias;
    int dt;
    int64_t F, S, C, n_locs;
    const int64_t* locs;
    double* out;
} proj_ctx;

static void proj_locs(void* vctx, int64_t l0, int64_t l1, int tid) {
    (void)tid;
    proj_ctx* c = (proj_ctx*)vctx;
    int64_t F = c->F, S = c->S, C = c->C, nl = c->n_locs;
    double* tok = (double*)malloc(sizeof(double) * (size_t)C);
    double* wd = (double*)malloc(sizeof(double) * (size_t)(3 * C * C));
    if (!tok || !wd) abort();
    for (int64_t i = 0; i < 3 * C * C; ++i) wd[i] = load(c->w, c->dt, i);
    for (int64_t li = l0; li < l1; ++li) {
        int64_t s = c->locs[li];
        for (int64_t f = 0; f < F; ++f) {
            for (int64_t ci = 0; ci < C; ++ci) tok[ci] = load(c->x, c->dt, (f * S + s) * C + ci);
            for (int64_t p = 0; p < 3; ++p)
                for (int64_t co = 0; co < C; ++co) {
                    const double* wr = wd + (p * C + co) * C;
                    double acc = c->bias ? c->bias[p * C + co] : 0.0;
                    for (int64_t ci = 0; ci < C; ++ci) acc += wr[ci] * tok[ci];
                    c->out[((p * F + f) * nl + li) * C + co] = acc;
                }
        }
    }
    free(tok);
    free(wd);
}

int oracle_qkv_project(const void* x, const void* w, const double* bias, int dt, int64_t F, int64_t S, int64_t C,
                       const int64_t* locs, int64_t n_locs, double* out, int nthreads) {
    if (!x || !w || !out || !locs || dt < 0 || dt > 2 || F < 1 || S < 1 || C < 1 || n_locs < 0) return 1;
    for (int64_t i = 0; i < n_locs; ++i)
        if (locs[i] < 0 || locs[i] >= S) return 1;
    nthreads = resolve_threads(nthreads);
    if (nthreads > n_locs) nthreads = n_locs > 0 ? (int)n_locs : 1;
    proj_ctx c = {x, w, bias, dt, F, S, C, n_locs, locs, out};
    parallel_ranges(n_locs, nthreads, proj_locs, &c);
    return 0;
}

/* Store the rounded values v[0..n) in dt (exact: each is a dt value). */
static void store_rounded(double* v, size_t n, int dt, void* t) {
    for (size_t i = 0; i < n; ++i) {
        v[i] = oracle_round_to(v[i], dt);
        if (dt == 0) {
            ((float*)t)[i] = (float)v[i];
        } else {
            float f = (float)v[i];
            uint32_t u;
            memcpy(&u, &f, 4);
            ((uint16_t*)t)[i] = (uint16_t)(u >> 16);
        }
    }
}

/* Projection, then the attention over the projected tokens.  Q, K and V are
 * tensors of the I/O type, so each is rounded to dt before the attention
 * reads it.  The location subset stays exact (neither step mixes spatial
 * locations). */
int oracle_qkv_dda(const void* x, const void* w, const double* bias, int dt, int64_t F, int64_t S, int64_t C,
                   int head_dim, int n_local, int n_global, double scale, const int64_t* locs, int64_t n_locs,
                   double* out, double* qkv_out, int nthreads) {
    if (!out || n_locs < 1 || (dt != 0 && dt != 1)) return 1;
    size_t n = (size_t)(F * n_locs * C);
    double* pr = (double*)malloc(sizeof(double) * 3 * n);
    char* t = (char*)malloc((dt == 0 ? 4 : 2) * 3 * n);
    int64_t* seq = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_locs);
    if (!pr || !t || !seq) {
        free(pr);
        free(t);
        free(seq);
        return 2;
    }
    int rc = oracle_qkv_project(x, w, bias, dt, F, S, C, locs, n_locs, pr, nthreads);
    if (rc == 0) {
        const size_t tb = (dt == 0 ? 4 : 2) * n;
        for (int p = 0; p < 3; ++p) store_rounded(pr + p * n, n, dt, t + p * tb);
        if (qkv_out) memcpy(qkv_out, pr, sizeof(double) * 3 * n);
        for (int64_t i = 0; i < n_locs; ++i) seq[i] = i;
        rc = oracle_dda(t, t + tb, t + 2 * tb, dt, F, n_locs, C, head_dim, n_local, n_global, scale, seq, n_locs,
                        out, nthreads);
    }
    free(pr);
    free(t);
    free(seq);
    return rc;
}

/* ---- The three modules in a row --------------------------------------- */
/* Each module's output is a tensor of the I/O type, so intermediates are
 * rounded to dt before they feed the next module.  With round_gn == 0 the
 * GroupNorm output is not a tensor of its own (GroupNorm folded into the
 * conv): the conv then reads the exact GroupNorm values and only the conv
 * output is rounded.  The location subset stays exact: conv and attention
 * never mix spatial locations, and the GroupNorm statistics are taken over
 * the whole tensor. */

int oracle_chain(const void* x, const void* w, int dt, int64_t F, int64_t S, int64_t C, int64_t G,
                 double eps, int head_dim, int n_local, int n_global, double scale, int round_gn,
                 const int64_t* locs, int64_t n_locs, double* out, double* gn_out, double* conv_out,
                 double* gn_exact, double* conv_exact, double* mean, double* rstd, int nthreads) {
    if (!out || !w || n_locs < 1 || (dt != 0 && dt != 1)) return 1; /* intermediates are rounded to dt */
    size_t n = (size_t)(F * n_locs * C);
    double* a = (double*)malloc(sizeof(double) * n);
    double* b = (double*)malloc(sizeof(double) * n);
    void* ta = malloc((dt == 0 ? 4 : 2) * n);
    int64_t* seq = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_locs);
    double* w64 = round_gn ? NULL : (double*)malloc(sizeof(double) * (size_t)(3 * C * C));
    if (!a || !b || !ta || !seq || (!round_gn && !w64)) {
        free(a);
        free(b);
        free(ta);
        free(seq);
        free(w64);
        return 2;
    }
    int rc = oracle_groupnorm(x, dt, F, S, C, G, eps, NULL, NULL, locs, n_locs, a, mean, rstd, nthreads);
    /* The sampled columns become a dense [F][n_locs][C] tensor in dt. */
    for (int64_t i = 0; i < n_locs; ++i) seq[i] = i;
    if (rc == 0 && !round_gn) {
        /* the conv reads the exact GroupNorm values, and the weights widened alike */
        if (gn_exact) memcpy(gn_exact, a, sizeof(double) * n);
        if (gn_out) memcpy(gn_out, a, sizeof(double) * n);
        for (int64_t i = 0; i < 3 * C * C; ++i) w64[i] = load(w, dt, i);
        rc = oracle_conv3(a, NULL, NULL, w64, NULL, 2, F, n_locs, C, seq, n_locs, b, nthreads);
    } else if (rc == 0) {
        if (gn_exact) memcpy(gn_exact, a, sizeof(double) * n);
        for (size_t i = 0; i < n; ++i) {
            a[i] = oracle_round_to(a[i], dt);
            if (dt == 0) {
                ((float*)ta)[i] = (float)a[i];
            } else {
                float f = (float)a[i];
                uint32_t u;
                memcpy(&u, &f, 4);
                ((uint16_t*)ta)[i] = (uint16_t)(u >> 16); /* exact: a[i] is a bf16 value */
            }
        }
        if (gn_out) memcpy(gn_out, a, sizeof(double) * n);
        rc = oracle_conv3(ta, NULL, NULL, w, NULL, dt, F, n_locs, C, seq, n_locs, b, nthreads);
    }
    if (rc == 0) {
        if (conv_exact) memcpy(conv_exact, b, sizeof(double) * n);
        for (size_t i = 0; i < n; ++i) {
            b[i] = oracle_round_to(b[i], dt);
            if (dt == 0) {
                ((float*)ta)[i] = (float)b[i];
            } else {
                float f = (float)b[i];
                uint32_t u;
                memcpy(&u, &f, 4);
                ((uint16_t*)ta)[i] = (uint16_t)(u >> 16);
            }
        }
        if (conv_out) memcpy(conv_out, b, sizeof(double) * n);
        rc = oracle_dda(ta, ta, ta, dt, F, n_locs, C, head_dim, n_local, n_global, scale, seq, n_locs, out,
                        nthreads);
    }
    free(a);
    free(b);
    free(ta);
    free(seq);
    free(w64);
    return rc;
}

/* ---- Reuse of temporal-attention outputs across diffusion steps ------- */
/* The attention difference between consecutive diffusion steps is large in
 * the first and last 15% of the steps and small in the middle 70%; in that
 * middle band one step's attention output is broadcast to the following steps
 * of a range.  Readings: the edge is floor(15% of n_steps) steps at each end;
 * the middle band is [edge, n_steps - edge); inside it the steps edge,
 * edge + range, edge + 2*range, ... compute and the others reuse the latest
 * computed output.  recompute[i] = 1 for a step that computes. */
int oracle_broadcast_schedule(int n_steps, int range, unsigned char* recompute) {
    if (n_steps < 1 || range < 1 || !recompute) return 1;
    int edge = (15 * n_steps) / 100;
    for (int i = 0; i < n_steps; ++i) {
        int in_middle = i >= edge && i < n_steps - edge;
        recompute[i] = (unsigned char)(in_middle ? ((i - edge) % range == 0) : 1);
    }
    return 0;
}

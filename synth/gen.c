/*
 * Seeded synthetic inputs, shared by the HIP path's tests/bench and the oracle.
 *
 * This file holds no arithmetic of the temporal module: it only turns
 * (seed, element index) into a number.  Element e of a tensor is
 *
 *     u1 = U(splitmix64(seed, 2e)),  u2 = U(splitmix64(seed, 2e+1))
 *     z  = sqrt(-2 ln u1) * cos(2 pi u2)                 (Box-Muller, one branch)
 *     v  = scale * z + frame_slope * floor(e / frame_elems)
 *
 * evaluated in double, rounded to float (round-to-nearest-even), and for bf16
 * output rounded once more from float to bf16 (round-to-nearest-even).
 *
 * splitmix64(seed, i) is the output function of Steele, Lea and Flood's
 * SplitMix64 ("Fast splittable pseudorandom number generators", OOPSLA 2014)
 * applied to the state seed + (i+1)*0x9E3779B97F4A7C15, i.e. the i-th output of
 * a SplitMix64 stream started at `seed`.  Because every element is a pure
 * function of its index, the result does not depend on the thread count.
 * U(x) = ((x >> 11) + 1) * 2^-53 lies in (0, 1], so ln u1 is finite.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>
#include <unistd.h>

static inline uint64_t sm64(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline double unit_open0(uint64_t x) { return (double)((x >> 11) + 1) * 0x1.0p-53; }

static inline float gen_value(uint64_t seed, uint64_t e, double scale, uint64_t frame_elems,
                              double frame_slope) {
    double u1 = unit_open0(sm64(seed, 2 * e));
    double u2 = unit_open0(sm64(seed, 2 * e + 1));
    double z = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
    double v = scale * z;
    if (frame_elems) v += frame_slope * (double)(e / frame_elems);
    return (float)v;
}

/* float -> bf16 bits, round to nearest even (NaN kept quiet). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef struct {
    uint64_t seed, begin, end, frame_elems;
    double scale, frame_slope;
    int dtype; /* 0 = f32, 1 = bf16 */
    void* out;
} job_t;

static void* worker(void* p) {
    job_t* j = (job_t*)p;
    if (j->dtype == 0) {
        float* o = (float*)j->out;
        for (uint64_t e = j->begin; e < j->end; ++e)
            o[e] = gen_value(j->seed, e, j->scale, j->frame_elems, j->frame_slope);
    } else {
        uint16_t* o = (uint16_t*)j->out;
        for (uint64_t e = j->begin; e < j->end; ++e)
            o[e] = f32_to_bf16_rne(gen_value(j->seed, e, j->scale, j->frame_elems, j->frame_slope));
    }
    return NULL;
}

/* Fill out[0..n) (float or bf16 bits).  nthreads <= 0 uses every online core, at most 16. */
int synth_normal(void* out, uint64_t n, int dtype, uint64_t seed, double scale, uint64_t frame_elems,
                 double frame_slope, int nthreads) {
    if (!out || (dtype != 0 && dtype != 1)) return 1;
    if (nthreads <= 0) { /* default: every online core, at most 16 */
        nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
        if (nthreads > 16) nthreads = 16;
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((uint64_t)nthreads > n / 65536 + 1) nthreads = (int)(n / 65536 + 1);
    pthread_t th[256];
    int made[256];
    job_t jobs[256];
    uint64_t chunk = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t b = chunk * t, e = b + chunk;
        if (b > n) b = n;
        if (e > n) e = n;
        jobs[t] = (job_t){seed, b, e, frame_elems, scale, frame_slope, dtype, out};
        made[t] = t < nthreads - 1 && pthread_create(&th[t], NULL, worker, &jobs[t]) == 0;
        if (!made[t]) worker(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (made[t]) pthread_join(th[t], NULL);
    return 0;
}

/* Exposed for the generator's own tests. */
uint64_t synth_splitmix64(uint64_t seed, uint64_t i) { return sm64(seed, i); }
uint16_t synth_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

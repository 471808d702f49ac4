// Internal helpers shared by the libvinf HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vinf.h"

namespace vinf {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 <-> fp32.  A dword holds two bf16: element 0 in the low half.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round two floats to bf16 (nearest even; v_cvt_pk_bf16_f32) and pack them.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// acc + a.x*b.x + a.y*b.y over bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                           acc, false);
}

// Hardware workgroup id -> logical id such that consecutive logical ids land
// on the same XCD (the dispatcher deals workgroups to the 8 XCDs round-robin).
// Only a permutation when n % 8 == 0; otherwise the identity.
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t b, uint32_t n) {
    if (n & 7u) return b;
    return (b & 7u) * (n >> 3) + (b >> 3);
}

}  // namespace vinf

// ---- host side ------------------------------------------------------------

namespace vinf_host {

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
vinf_status fail(vinf_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// hipGetLastError() after a launch, mapped to VINF_ERR_HIP with `what`.
vinf_status check_launch(const char* what);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Do byte ranges [a, a+na) and [b, b+nb) intersect?
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

inline size_t dtype_bytes(vinf_dtype dt) { return dt == VINF_BF16 ? 2 : 4; }

// Launchers implemented next to their kernels (arguments already validated).
// y == NULL: statistics only (the two sweeps; mean_out and rstd_out required).
vinf_status launch_groupnorm(const void* x, void* y, const float* gamma, const float* beta, float* mean_out,
                             float* rstd_out, int64_t rows, int C, int groups, float eps, vinf_dtype dt,
                             void* workspace, hipStream_t stream);
size_t groupnorm_workspace(int64_t rows, int C, int groups, vinf_dtype dt);
// The same with the library's static scratch array as the workspace (sizes
// needing more than VINF_NOALLOC_SCRATCH_BYTES are rejected).
vinf_status launch_groupnorm_noalloc(const void* x, void* y, const float* gamma, const float* beta, float* mean_out,
                                     float* rstd_out, int64_t rows, int C, int groups, float eps, vinf_dtype dt,
                                     hipStream_t stream);
// One clip's fp64 group sums (first pass: mean_sums null; second pass: about
// the means mean_sums[g] / n_total).
vinf_status launch_groupnorm_clip_sums(const void* x, const double* mean_sums, double* sums, int64_t rows, int C,
                                       int groups, double n_total, vinf_dtype dt, void* workspace,
                                       hipStream_t stream);
// Normalise one clip with the statistics of the aggregated sums (x == NULL:
// statistics only).
vinf_status launch_groupnorm_clip_apply(const void* x, void* y, const float* gamma, const float* beta,
                                        const double* sums, const double* sq_sums, float* mean_out, float* rstd_out,
                                        int64_t rows, int C, int groups, double n_total, float eps, vinf_dtype dt,
                                        void* workspace, hipStream_t stream);

vinf_status launch_conv3(const void* x, const void* ctx_pre, const void* ctx_post, const void* weight,
                         const float* bias, void* y, int F, int S, int C, vinf_dtype dt, hipStream_t stream);
// The conv of GroupNorm(x) with the given statistics, the normalisation
// applied to the conv's input tiles (workspace: conv3_gn_workspace bytes).
size_t conv3_gn_workspace(int C, vinf_dtype dt);
vinf_status launch_conv3_gn(const void* x, const void* ctx_pre, const void* ctx_post, const void* weight,
                            const float* bias, const float* mean, const float* rstd, const float* gamma,
                            const float* beta, int groups, void* y, int F, int S, int C, vinf_dtype dt,
                            void* workspace, hipStream_t stream);
// Q, K and V = the three C x C maps of w ([3][C][C]) applied to every token of
// x (bf16: the conv's MFMA kernel with one tap; fp32: one element per thread).
vinf_status launch_qkv_project(const void* x, const void* w, const float* bias, void* q, void* k, void* v, int F,
                               int S, int C, vinf_dtype dt, hipStream_t st);

// Attention over the projected tokens of x (bf16): the Q/K/V maps of
// weight [3][C][C] (+ bias [3][C] or null) computed per work item, never
// written out; the full key set (16 local + 16 global).
vinf_status launch_dda_projected(const void* x, const void* w, const float* bias, void* o, int F, int S, int C,
                                 float scale, hipStream_t st);

// Attention of query frames f0 .. f0+nq-1 of an F-frame video; k/v hold
// frames kf0 .. kend-1; kg/vg the global rows or null (read from k/v).
vinf_status launch_dda(const void* q, const void* k, const void* v, const void* kg, const void* vg, void* o,
                       int F, int f0, int nq, int kf0, int kend, int S, int C, int n_local, int n_global,
                       float scale, vinf_dtype dt, hipStream_t stream);

}  // namespace vinf_host

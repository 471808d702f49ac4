// Dual-domain temporal attention, gfx950.
//
// Method (Video-Infinity write-up, dual-domain attention paragraph and the
// paragraph fixing both context sizes at 16): every query frame t of a spatial
// location attends over a key/value frame set made of its 16 neighbouring
// frames (local context) followed by 16 frames sampled uniformly over the
// whole video (global context).  Readings: the local window starts at
// clamp(t-8, 0, F-16); the global frames are floor(i*F/16); the two lists are
// concatenated, so a frame in both carries two softmax terms.
//
// bf16 kernel (dda_bf16).  One workgroup = 4 wave64s = one (location, head)
// strip x 256 consecutive query frames, one query per lane.
//   * Staging: the strip's K rows for every local key of the 256 queries
//     (<= 271 frames, 128 B each) and the 16 global K rows go to LDS; the V
//     rows go to LDS re-packed as frame pairs, each dword holding
//     (v[f][d], v[f+1][d]), so that the weighted sum over keys runs on
//     v_dot2c_f32_bf16 with the softmax weights packed as bf16 pairs.  LDS
//     rows are XOR-swizzled per 16-byte chunk so that lanes reading
//     neighbouring frames hit distinct banks.  Every HBM load is a full
//     128-byte row (one cache line) of one frame.
//   * Scores: q stays in 32 VGPRs as bf16 pairs; 32 keys x 32 v_dot2c each.
//     The lane holds all 32 scores, so the softmax is lane-local: one max,
//     exp2 with log2(e)*scale folded in, no cross-lane traffic.
//   * Weighted sum: 9 local pair rows (the window's parity decides which
//     pair holds its first frame; the unused slot gets weight 0) and 8 global
//     pair rows, 64 v_dot2c each, into 64 fp32 accumulators.  The normaliser
//     is the sum of the same bf16-rounded weights, so the output is an exact
//     convex combination of the V rows up to fp32 rounding.
//   * Output: fp32 -> bf16 (nearest even), 128-byte row per lane.
// fp32 kernel (dda_f32): one query per thread, fp32 FMA, keys read through
// the cache; used for float32 I/O.
#include <math.h>

#include "common.h"

namespace vinf {

constexpr int DDA_D = 64;          // head dim
constexpr int DDA_L = 16;          // local keys
constexpr int DDA_G = 16;          // global keys
constexpr int DDA_TQ = 256;        // queries per workgroup
constexpr int DDA_KROWS = DDA_TQ + DDA_L;            // 272 local K rows
constexpr int DDA_VPAIRS = (DDA_TQ + 19) / 2 + 1;    // 138 local V pair rows
constexpr int DDA_LDS_KL = 0;
constexpr int DDA_LDS_VP = DDA_LDS_KL + DDA_KROWS * 128;
constexpr int DDA_LDS_KG = DDA_LDS_VP + DDA_VPAIRS * 256;
constexpr int DDA_LDS_VG = DDA_LDS_KG + DDA_G * 128;
constexpr int DDA_LDS_BYTES = DDA_LDS_VG + (DDA_G / 2) * 256;

__device__ __forceinline__ int dda_start(int t, int F) {
    int hi = F - DDA_L > 0 ? F - DDA_L : 0;
    int st = t - DDA_L / 2;
    return st < 0 ? 0 : (st > hi ? hi : st);
}

// Byte offset of 16-byte chunk c of K row r (8 chunks per row).
__device__ __forceinline__ int kl_off(int r, int c) { return DDA_LDS_KL + r * 128 + ((c ^ (r & 7)) << 4); }
// Byte offset of 16-byte chunk c of V pair row p (16 chunks per row).
__device__ __forceinline__ int vp_off(int p, int c) { return DDA_LDS_VP + p * 256 + ((c ^ (p & 7)) << 4); }

__device__ __forceinline__ u32x4_t gload(const uint16_t* base, int64_t elem) {
    return *reinterpret_cast<const u32x4_t*>(base + elem);
}

// Interleave two rows' dwords: (a.lo, b.lo) and (a.hi, b.hi).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__global__ void __launch_bounds__(256) dda_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, uint16_t* __restrict__ o, int F,
                                                   int S, int C, int nstrips, float sl2e) {
    __shared__ __attribute__((aligned(16))) char lds[DDA_LDS_BYTES];
    const uint32_t lb = xcd_swizzle(blockIdx.x, gridDim.x);
    const int strip = (int)(lb % (uint32_t)nstrips);
    const int fblk = (int)(lb / (uint32_t)nstrips);
    const int heads = C / DDA_D;
    const int s = strip / heads, h = strip % heads;
    const int64_t rs = (int64_t)S * C;                     // elements between frames
    const int64_t col = (int64_t)s * C + h * DDA_D;        // strip's offset inside a frame
    const int t0 = fblk * DDA_TQ;
    const int tlast = min(t0 + DDA_TQ, F) - 1;
    const int lo = dda_start(t0, F);
    const int khi = dda_start(tlast, F) + DDA_L;           // stage K frames [lo, khi)
    const int plo = lo & ~1;
    const int np = (dda_start(tlast, F) + DDA_L + 2 - plo + 1) >> 1;  // V pairs cover [plo, plo+2np)
    const int tid = threadIdx.x;

    // ---- stage local K rows ----
    const int nk = (khi - lo) * 8;
#pragma unroll
    for (int it = 0; it < (DDA_KROWS * 8 + 255) / 256; ++it) {
        int i = tid + it * 256;
        if (i < nk) {
            int r = i >> 3, c = i & 7, f = lo + r;
            u32x4_t u = {0u, 0u, 0u, 0u};
            if (f < F) u = gload(k, f * rs + col + c * 8);
            *reinterpret_cast<u32x4_t*>(lds + kl_off(r, c)) = u;
        }
    }
    // ---- stage local V as frame pairs ----
    const int nv = np * 8;
#pragma unroll
    for (int it = 0; it < (DDA_VPAIRS * 8 + 255) / 256; ++it) {
        int i = tid + it * 256;
        if (i < nv) {
            int p = i >> 3, oc = i & 7, fa = plo + 2 * p, fb = fa + 1;
            u32x4_t a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (fa < F) a = gload(v, fa * rs + col + oc * 8);
            if (fb < F) b = gload(v, fb * rs + col + oc * 8);
            u32x4_t w0 = {pair_lo(a[0], b[0]), pair_hi(a[0], b[0]), pair_lo(a[1], b[1]), pair_hi(a[1], b[1])};
            u32x4_t w1 = {pair_lo(a[2], b[2]), pair_hi(a[2], b[2]), pair_lo(a[3], b[3]), pair_hi(a[3], b[3])};
            *reinterpret_cast<u32x4_t*>(lds + vp_off(p, 2 * oc)) = w0;
            *reinterpret_cast<u32x4_t*>(lds + vp_off(p, 2 * oc + 1)) = w1;
        }
    }
    // ---- stage global K rows and V pairs ----
    if (tid < DDA_G * 8) {
        int i = tid >> 3, c = tid & 7;
        int f = (int)(((int64_t)i * F) / DDA_G);
        *reinterpret_cast<u32x4_t*>(lds + DDA_LDS_KG + i * 128 + c * 16) = gload(k, f * rs + col + c * 8);
    } else if (tid < DDA_G * 8 + (DDA_G / 2) * 8) {
        int j = tid - DDA_G * 8;
        int p = j >> 3, oc = j & 7;
        int fa = (int)(((int64_t)(2 * p) * F) / DDA_G), fb = (int)(((int64_t)(2 * p + 1) * F) / DDA_G);
        u32x4_t a = gload(v, fa * rs + col + oc * 8), b = gload(v, fb * rs + col + oc * 8);
        u32x4_t w0 = {pair_lo(a[0], b[0]), pair_hi(a[0], b[0]), pair_lo(a[1], b[1]), pair_hi(a[1], b[1])};
        u32x4_t w1 = {pair_lo(a[2], b[2]), pair_hi(a[2], b[2]), pair_lo(a[3], b[3]), pair_hi(a[3], b[3])};
        *reinterpret_cast<u32x4_t*>(lds + DDA_LDS_VG + p * 256 + (2 * oc) * 16) = w0;
        *reinterpret_cast<u32x4_t*>(lds + DDA_LDS_VG + p * 256 + (2 * oc + 1) * 16) = w1;
    }
    __syncthreads();

    const int t = t0 + tid;
    if (t >= F) return;
    const int nl = F < DDA_L ? F : DDA_L;
    const int st = dda_start(t, F);

    // q row as 32 bf16 pairs
    uint32_t qv[32];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u32x4_t u = gload(q, t * rs + col + c * 8);
        qv[4 * c] = u[0];
        qv[4 * c + 1] = u[1];
        qv[4 * c + 2] = u[2];
        qv[4 * c + 3] = u[3];
    }

    // ---- scores ----
    float sc[DDA_L + DDA_G];
#pragma unroll
    for (int j = 0; j < DDA_L + DDA_G; ++j) sc[j] = 0.f;
    const int kr0 = st - lo;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int i = 0; i < DDA_L; ++i) {
            u32x4_t u = *reinterpret_cast<const u32x4_t*>(lds + kl_off(kr0 + i, c));
            float a = sc[i];
            a = dot2_bf16(qv[4 * c], u[0], a);
            a = dot2_bf16(qv[4 * c + 1], u[1], a);
            a = dot2_bf16(qv[4 * c + 2], u[2], a);
            a = dot2_bf16(qv[4 * c + 3], u[3], a);
            sc[i] = a;
        }
#pragma unroll
        for (int i = 0; i < DDA_G; ++i) {
            u32x4_t u = *reinterpret_cast<const u32x4_t*>(lds + DDA_LDS_KG + i * 128 + c * 16);
            float a = sc[DDA_L + i];
            a = dot2_bf16(qv[4 * c], u[0], a);
            a = dot2_bf16(qv[4 * c + 1], u[1], a);
            a = dot2_bf16(qv[4 * c + 2], u[2], a);
            a = dot2_bf16(qv[4 * c + 3], u[3], a);
            sc[DDA_L + i] = a;
        }
    }

    // ---- lane-local softmax (base 2, scale folded in) ----
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < DDA_L + DDA_G; ++j) {
        sc[j] = (j < DDA_L && j >= nl) ? -INFINITY : sc[j] * sl2e;
        m = fmaxf(m, sc[j]);
    }
#pragma unroll
    for (int j = 0; j < DDA_L + DDA_G; ++j) sc[j] = __builtin_amdgcn_exp2f(sc[j] - m);

    // weights as bf16 pairs matching the V pair rows
    const int par = st & 1;
    uint32_t wl[9], wg[8];
#pragma unroll
    for (int j = 0; j < 9; ++j) {
        float a_even = j < 8 ? sc[2 * j] : 0.f;          // par == 0: frames (st+2j, st+2j+1)
        float b_even = j < 8 ? sc[2 * j + 1] : 0.f;
        float a_odd = j > 0 ? sc[2 * j - 1] : 0.f;       // par == 1: frames (st+2j-1, st+2j)
        float b_odd = j < 8 ? sc[2 * j] : 0.f;
        wl[j] = par ? pack_bf16x2(a_odd, b_odd) : pack_bf16x2(a_even, b_even);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) wg[i] = pack_bf16x2(sc[DDA_L + 2 * i], sc[DDA_L + 2 * i + 1]);
    const uint32_t ones = 0x3f803f80u;  // (1.0, 1.0) in bf16
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < 9; ++j) den = dot2_bf16(wl[j], ones, den);
#pragma unroll
    for (int i = 0; i < 8; ++i) den = dot2_bf16(wg[i], ones, den);

    // ---- weighted sum of V ----
    float acc[DDA_D];
#pragma unroll
    for (int d = 0; d < DDA_D; ++d) acc[d] = 0.f;
    const int pb = (st - plo) >> 1;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            u32x4_t u = *reinterpret_cast<const u32x4_t*>(lds + vp_off(pb + j, c));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * c + e] = dot2_bf16(wl[j], u[e], acc[4 * c + e]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            u32x4_t u = *reinterpret_cast<const u32x4_t*>(lds + DDA_LDS_VG + i * 256 + c * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * c + e] = dot2_bf16(wg[i], u[e], acc[4 * c + e]);
        }
    }

    const float inv = 1.f / den;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc[8 * c + 2 * e] * inv, acc[8 * c + 2 * e + 1] * inv);
        *reinterpret_cast<u32x4_t*>(o + t * rs + col + c * 8) = w;
    }
}

// float32 I/O: one query per thread, keys read through the cache.
__global__ void __launch_bounds__(64) dda_f32(const float* __restrict__ q, const float* __restrict__ k,
                                              const float* __restrict__ v, float* __restrict__ o, int F, int S,
                                              int C, float sl2e) {
    const int heads = C / DDA_D;
    const int64_t qi = (int64_t)blockIdx.x * 64 + threadIdx.x;  // (t, s, h) flattened
    if (qi >= (int64_t)F * S * heads) return;
    const int h = (int)(qi % heads);
    const int s = (int)((qi / heads) % S);
    const int t = (int)(qi / ((int64_t)heads * S));
    const int64_t rs = (int64_t)S * C, col = (int64_t)s * C + h * DDA_D;
    const int nl = F < DDA_L ? F : DDA_L;
    const int st = dda_start(t, F);
    int keys[DDA_L + DDA_G];
    float sc[DDA_L + DDA_G];
    const int n = nl + DDA_G;
    for (int j = 0; j < DDA_L + DDA_G; ++j) {
        keys[j] = j < nl ? st + j : (j < n ? (int)(((int64_t)(j - nl) * F) / DDA_G) : 0);
    }
    const float* qr = q + t * rs + col;
    float m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        const float* kr = k + keys[j] * rs + col;
        float a = 0.f;
        for (int d = 0; d < DDA_D; ++d) a = fmaf(qr[d], kr[d], a);
        sc[j] = a * sl2e;
        m = fmaxf(m, sc[j]);
    }
    float acc[DDA_D];
    for (int d = 0; d < DDA_D; ++d) acc[d] = 0.f;
    float den = 0.f;
    for (int j = 0; j < n; ++j) {
        float p = __builtin_amdgcn_exp2f(sc[j] - m);
        den += p;
        const float* vr = v + keys[j] * rs + col;
        for (int d = 0; d < DDA_D; ++d) acc[d] = fmaf(p, vr[d], acc[d]);
    }
    float inv = 1.f / den;
    float* orow = o + t * rs + col;
    for (int d = 0; d < DDA_D; ++d) orow[d] = acc[d] * inv;
}

}  // namespace vinf

namespace vinf_host {
using namespace vinf;

vinf_status launch_dda(const void* q, const void* k, const void* v, void* o, int F, int S, int C, float scale,
                       vinf_dtype dt, hipStream_t st) {
    const float sl2e = scale * 1.4426950408889634f;
    const int heads = C / DDA_D;
    if (dt == VINF_BF16) {
        const int nstrips = S * heads;
        const int nfb = (F + DDA_TQ - 1) / DDA_TQ;
        const int64_t blocks = (int64_t)nstrips * nfb;
        if (blocks > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "dual_domain_attn: grid too large");
        hipLaunchKernelGGL(dda_bf16, dim3((uint32_t)blocks), dim3(256), 0, st,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), F, S, C, nstrips, sl2e);
    } else {
        const int64_t nq = (int64_t)F * S * heads;
        const int64_t blocks = (nq + 63) / 64;
        if (blocks > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "dual_domain_attn: grid too large");
        hipLaunchKernelGGL(dda_f32, dim3((uint32_t)blocks), dim3(64), 0, st, static_cast<const float*>(q),
                           static_cast<const float*>(k), static_cast<const float*>(v), static_cast<float*>(o), F, S,
                           C, sl2e);
    }
    return check_launch("dual_domain_attn");
}

}  // namespace vinf_host

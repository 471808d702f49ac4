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
// bf16 kernel (dda_bf16).  Work item = one (location, head) strip x 256
// consecutive query frames, one query per lane.
//   * Staging: the strip's K rows for every local key of the 256 queries
//     (<= 271 frames, 128 B each) and the 16 global K rows go to LDS; the V
//     rows go to LDS re-packed as frame pairs, each dword holding
//     (v[f][d], v[f+1][d]), so that the weighted sum over keys runs on
//     v_dot2c_f32_bf16 with the softmax weights packed as bf16 pairs.  LDS
//     rows are padded by 16 bytes (K rows 144 B, V pair rows 272 B) so that
//     16 lanes reading neighbouring frames hit distinct banks, and every LDS
//     read is a per-lane base plus an immediate offset (no address VALU).
//     Every HBM load is a full 128-byte row (one cache line) of one frame.
//   * Scores: q stays in 32 VGPRs as bf16 pairs; 32 keys x 32 v_dot2c each.
//     The lane holds all 32 scores, so the softmax is lane-local: one max,
//     exp2 with log2(e)*scale folded in, no cross-lane traffic.
//   * Weighted sum: 9 local pair rows (the window's parity decides which
//     pair holds its first frame; the unused slot gets weight 0) and 8 global
//     pair rows, 64 v_dot2c each, into 64 fp32 accumulators.  The normaliser
//     is the sum of the same bf16-rounded weights, so the output is an exact
//     convex combination of the V rows up to fp32 rounding.
//   * Output: fp32 -> bf16 (nearest even), 128-byte row per lane.  The 4
//     lanes of a quad (4 consecutive frames) transpose each half of their
//     eight 16-byte chunks through two ds_swizzle exchanges (lane distances
//     2, 1), so each store instruction writes 64 contiguous bytes of 16
//     frames rather than 16 bytes of 64.  Lanes past the last query
//     therefore stay in the quad (computing the last query again) and only
//     skip their stores.
//   * Frame ranges (DdaGeo): the queries' frames and the frames the K/V
//     buffers hold are given separately, and the 16 global rows may come from
//     buffers of their own, so one clip of a longer video with its
//     neighbours' context frames runs the same code; the whole video is the
//     case where both ranges are the video and the global rows are read in
//     place.
//   * Key sets: the bf16 kernel is templated on the local and global keys
//     present (16 or 0 each): the full method, local context only, global
//     context only.
//   * Remainders: when the query count leaves r = nq % 256 queries per strip
//     (a clip of 288 frames: 32), M strips share one item (M = 4 for r <= 36,
//     2 for r <= 104), each in its own slice of the buffer with 4/M waves, so
//     a short remainder does not cost a whole item per strip.
//   * Pipelining: one persistent 512-thread workgroup per CU owns two LDS
//     buffers (2 x 80 KB).  Its two 256-thread halves alternate: while one
//     half stages its next work item (HBM -> LDS, plus its q rows into
//     registers), the other computes from its own buffer; a workgroup barrier
//     ends each phase.  HBM traffic and the VALU-bound compute overlap
//     instead of alternating.
// fp32 kernel (dda_f32): one query per thread, fp32 FMA, keys read through
// the cache; used for float32 I/O.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"

namespace vinf {

constexpr int DDA_D = 64;          // head dim
constexpr int DDA_L = 16;          // local keys
constexpr int DDA_G = 16;          // global keys
constexpr int DDA_TQ = 256;        // queries per work item (one per thread of a half workgroup)
constexpr int DDA_KSTR = 144;      // padded K row (bytes)
constexpr int DDA_VSTR = 272;      // padded V pair row (bytes)

// LDS slice of one strip for up to R consecutive queries: 16 global K rows
// (128 B), 8 global V pair rows (256 B), then the R + 15 local K rows and
// (R + 18) / 2 local V pair rows their windows cover.
template <int R>
struct DdaSlice {
    static constexpr int KROWS = R + DDA_L - 1;
    static constexpr int VPAIRS = (R + 18) / 2;
    static constexpr int KG = 0;
    static constexpr int VG = KG + DDA_G * 128;
    static constexpr int KL = VG + (DDA_G / 2) * 256;
    static constexpr int VP = KL + KROWS * DDA_KSTR;
    static constexpr int BYTES = VP + VPAIRS * DDA_VSTR;
};
using DdaFull = DdaSlice<DDA_TQ>;
constexpr int DDA_LDS_BYTES = DdaFull::BYTES;  // one half workgroup's buffer
static_assert(2 * DDA_LDS_BYTES <= 160 * 1024, "two buffers per CU");

// Remainder items: when a clip's query count leaves r = nq % 256 queries per
// strip, M strips share one item (4 / M waves each, up to DdaRemR<M> queries
// per strip), each in its own slice of the half's buffer.
template <int M>
constexpr int DdaRemR = M == 4 ? 36 : (M == 2 ? 104 : DDA_TQ);
static_assert(4 * DdaSlice<DdaRemR<4>>::BYTES <= DDA_LDS_BYTES, "4 remainder slices");
static_assert(2 * DdaSlice<DdaRemR<2>>::BYTES <= DDA_LDS_BYTES, "2 remainder slices");

__device__ __forceinline__ int dda_start(int t, int F) {
    int hi = F - DDA_L > 0 ? F - DDA_L : 0;
    int st = t - DDA_L / 2;
    return st < 0 ? 0 : (st > hi ? hi : st);
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Frames and buffers of one call.  The video has F frames; the queries are
// frames f0 .. f0+nq-1 (q and o row 0 is frame f0); k and v hold frames
// kf0 .. kend-1 (row 0 is frame kf0).  kg and vg hold the global rows (row i
// is frame floor(i*F/16)) or are null when k and v hold those frames.  The
// whole video on its own is f0 = kf0 = 0, nq = kend = F, kg = vg = null.
// Work items: nfull = nstrips * nchunks items of (strip, 256 query frames
// from f0 + 256*chunk), then the remainder items (packed kernels only).
struct DdaGeo {
    const void* kg;
    const void* vg;
    int F, f0, nq, kf0, kend;
    int S, C, nstrips, nchunks, nfull, nitems;
    float sl2e;
};

struct DdaItem {
    int strip, t0;
};

// Stage one strip's rows for queries t0 .. t0+R-1 into its slice `buf`
// (NT threads, lt = 0..NT-1) and load the q row of query t0 + lt into qv.
// NL / NG: local / global keys present (16 or 0).
template <int NL, int NG, int R, int NT>
__device__ __forceinline__ void dda_stage(char* __restrict__ buf, const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                          const DdaGeo& g, int64_t rs, int heads, DdaItem it, int lt,
                                          uint32_t (&qv)[32]) {
    using SL = DdaSlice<R>;
    constexpr int RSTEP = NT / 8;  // rows one pass of the threads covers (8 chunks per row)
    const int s = it.strip / heads, h = it.strip % heads;
    const int64_t col = (int64_t)s * g.C + h * DDA_D;
    const int t = it.t0 + lt;
    if (t < g.f0 + g.nq) {
        const uint16_t* qrow = q + (int64_t)(t - g.f0) * rs + col;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x4_t u = *reinterpret_cast<const u32x4_t*>(qrow + c * 8);
            qv[4 * c] = u[0];
            qv[4 * c + 1] = u[1];
            qv[4 * c + 2] = u[2];
            qv[4 * c + 3] = u[3];
        }
    } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) qv[c] = 0u;  // a lane past the last query computes a throw-away copy
    }
    if constexpr (NL > 0) {
        const int tlast = min(it.t0 + R, g.f0 + g.nq) - 1;
        const int lo = dda_start(it.t0, g.F);
        const int stl = dda_start(tlast, g.F);
        const int nkr = stl + DDA_L - lo;             // K rows [lo, lo+nkr), <= R + 15
        const int plo = lo & ~1;
        const int np = (stl + DDA_L + 2 - plo) >> 1;  // V pairs cover [plo, plo+2np), <= (R + 18) / 2
        // Frames outside [kf0, kend) are not in k/v: their rows are zero-filled
        // (only frames past the video's last frame, or the unused half of a
        // pair row, which carry no weight, fall outside).
        // local K rows: this thread's chunk c = lt&7 of rows lt>>3 + RSTEP*i
        {
            constexpr int NI = (SL::KROWS + RSTEP - 1) / RSTEP;
            const int c = lt & 7, r0 = lt >> 3;
            const uint16_t* src = k + col + (int64_t)(lo + r0 - g.kf0) * rs + c * 8;
            char* dst = buf + SL::KL + r0 * DDA_KSTR + c * 16;
            u32x4_t u[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int r = r0 + RSTEP * i;
                u[i] = u32x4_t{0u, 0u, 0u, 0u};
                if (r < nkr && lo + r < g.kend)
                    u[i] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)(RSTEP * i) * rs);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (r0 + RSTEP * i < nkr) *reinterpret_cast<u32x4_t*>(dst + RSTEP * i * DDA_KSTR) = u[i];
        }
        // local V as frame pairs: this thread's 8-dim group oc = lt&7 of pairs lt>>3 + RSTEP*i
        {
            constexpr int NI = (SL::VPAIRS + RSTEP - 1) / RSTEP;
            const int oc = lt & 7, p0 = lt >> 3;
            const uint16_t* src = v + col + (int64_t)(plo + 2 * p0 - g.kf0) * rs + oc * 8;
            char* dst = buf + SL::VP + p0 * DDA_VSTR + oc * 32;
            u32x4_t a[NI], b[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int p = p0 + RSTEP * i, fa = plo + 2 * p;
                a[i] = u32x4_t{0u, 0u, 0u, 0u};
                b[i] = u32x4_t{0u, 0u, 0u, 0u};
                if (p < np && fa >= g.kf0 && fa < g.kend)
                    a[i] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)(2 * RSTEP * i) * rs);
                if (p < np && fa + 1 < g.kend)
                    b[i] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)(2 * RSTEP * i + 1) * rs);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                if (p0 + RSTEP * i < np) {
                    u32x4_t w0 = {perm_lo(a[i][0], b[i][0]), perm_hi(a[i][0], b[i][0]), perm_lo(a[i][1], b[i][1]),
                                  perm_hi(a[i][1], b[i][1])};
                    u32x4_t w1 = {perm_lo(a[i][2], b[i][2]), perm_hi(a[i][2], b[i][2]), perm_lo(a[i][3], b[i][3]),
                                  perm_hi(a[i][3], b[i][3])};
                    *reinterpret_cast<u32x4_t*>(dst + RSTEP * i * DDA_VSTR) = w0;
                    *reinterpret_cast<u32x4_t*>(dst + RSTEP * i * DDA_VSTR + 16) = w1;
                }
            }
        }
    }
    if constexpr (NG > 0) {
        // 192 tasks: global K row chunks (tasks 0..127) and V pair chunks (128..191)
        const uint16_t* kgb = g.kg ? static_cast<const uint16_t*>(g.kg) : k;
        const uint16_t* vgb = g.vg ? static_cast<const uint16_t*>(g.vg) : v;
        auto grow = [&](int i) -> int64_t {  // row of global frame i in kgb / vgb
            return g.kg ? (int64_t)i : (int64_t)(((int64_t)i * g.F) / DDA_G) - g.kf0;
        };
#pragma unroll
        for (int task = lt; task < DDA_G * 8 + (DDA_G / 2) * 8; task += NT) {
            if (task < DDA_G * 8) {
                const int i = task >> 3, c = task & 7;
                *reinterpret_cast<u32x4_t*>(buf + SL::KG + i * 128 + c * 16) =
                    *reinterpret_cast<const u32x4_t*>(kgb + col + grow(i) * rs + c * 8);
            } else {
                const int j = task - DDA_G * 8;
                const int p = j >> 3, oc = j & 7;
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(vgb + col + grow(2 * p) * rs + oc * 8);
                const u32x4_t b = *reinterpret_cast<const u32x4_t*>(vgb + col + grow(2 * p + 1) * rs + oc * 8);
                u32x4_t w0 = {perm_lo(a[0], b[0]), perm_hi(a[0], b[0]), perm_lo(a[1], b[1]), perm_hi(a[1], b[1])};
                u32x4_t w1 = {perm_lo(a[2], b[2]), perm_hi(a[2], b[2]), perm_lo(a[3], b[3]), perm_hi(a[3], b[3])};
                char* dst = buf + SL::VG + p * 256 + oc * 32;
                *reinterpret_cast<u32x4_t*>(dst) = w0;
                *reinterpret_cast<u32x4_t*>(dst + 16) = w1;
            }
        }
    }
}

// Compute query t0 + lt of a strip staged in slice `buf` (layout DdaSlice<R>).
template <int NL, int NG, int R>
__device__ __forceinline__ void dda_compute(const char* __restrict__ buf, uint16_t* __restrict__ o,
                                            const DdaGeo& g, int64_t rs, int heads, DdaItem it, int lt,
                                            const uint32_t (&qv)[32]) {
    using SL = DdaSlice<R>;
    constexpr int NK = NL + NG;                 // keys
    constexpr int NLP = NL > 0 ? 9 : 0;         // local V pair rows
    constexpr int NP = NLP + (NG > 0 ? 8 : 0);  // V pair rows
    // Lanes past the last query stay in (the output transpose below moves
    // data between the 8 lanes of a group) and compute the last query's
    // windows; their own results are not stored.
    const int tend = g.f0 + g.nq;
    const int t = min(it.t0 + lt, tend - 1);
    const int s = it.strip / heads, h = it.strip % heads;
    const int64_t col = (int64_t)s * g.C + h * DDA_D;
    const int F = g.F;
    const int lo = dda_start(it.t0, F);
    const int plo = lo & ~1;
    const int nl = F < DDA_L ? F : DDA_L;
    const int st = dda_start(t, F);

    // ---- scores: one K row (8 x 16 B) per key; the next row's reads are
    // issued before the current row's dot products ----
    float sc[NK];
    const char* krow = buf + SL::KL + (st - lo) * DDA_KSTR;
    auto key_row = [&](int i) -> const char* {
        return i < NL ? krow + i * DDA_KSTR : buf + SL::KG + (i - NL) * 128;
    };
    u32x4_t kb[2][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) kb[0][c] = *reinterpret_cast<const u32x4_t*>(key_row(0) + c * 16);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        if (i + 1 < NK) {
#pragma unroll
            for (int c = 0; c < 8; ++c) kb[(i + 1) & 1][c] = *reinterpret_cast<const u32x4_t*>(key_row(i + 1) + c * 16);
        }
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4_t u = kb[i & 1][c];
            a = dot2_bf16(qv[4 * c], u[0], a);
            a = dot2_bf16(qv[4 * c + 1], u[1], a);
            a = dot2_bf16(qv[4 * c + 2], u[2], a);
            a = dot2_bf16(qv[4 * c + 3], u[3], a);
        }
        sc[i] = a;
    }

    // ---- lane-local softmax (base 2, scale folded in) ----
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        sc[j] = (j < NL && j >= nl) ? -INFINITY : sc[j] * g.sl2e;
        m = fmaxf(m, sc[j]);
    }
#pragma unroll
    for (int j = 0; j < NK; ++j) sc[j] = __builtin_amdgcn_exp2f(sc[j] - m);

    // weights as bf16 pairs matching the V pair rows: NLP local, then 8 global
    uint32_t w[NP];
    if constexpr (NL > 0) {
        const int par = st & 1;
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            float a_even = j < 8 ? sc[2 * j] : 0.f;          // par == 0: frames (st+2j, st+2j+1)
            float b_even = j < 8 ? sc[2 * j + 1] : 0.f;
            float a_odd = j > 0 ? sc[2 * j - 1] : 0.f;       // par == 1: frames (st+2j-1, st+2j)
            float b_odd = j < 8 ? sc[2 * j] : 0.f;
            w[j] = par ? pack_bf16x2(a_odd, b_odd) : pack_bf16x2(a_even, b_even);
        }
    }
    if constexpr (NG > 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[NLP + i] = pack_bf16x2(sc[NL + 2 * i], sc[NL + 2 * i + 1]);
    }
    const uint32_t ones = 0x3f803f80u;  // (1.0, 1.0) in bf16
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < NP; ++j) den = dot2_bf16(w[j], ones, den);

    // ---- weighted sum of V over the NP pair rows, next row's reads issued
    // before the current row's dot products ----
    float acc[DDA_D];
#pragma unroll
    for (int d = 0; d < DDA_D; ++d) acc[d] = 0.f;
    const char* vrow = buf + SL::VP + ((st - plo) >> 1) * DDA_VSTR;
    auto val_row = [&](int j) -> const char* {
        return j < NLP ? vrow + j * DDA_VSTR : buf + SL::VG + (j - NLP) * 256;
    };
    // half rows (32 dims, 8 x 16 B) double-buffered: step 2j + hh reads
    // dims 32*hh.. of pair row j
    u32x4_t vb[2][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) vb[0][c] = *reinterpret_cast<const u32x4_t*>(val_row(0) + c * 16);
#pragma unroll
    for (int step = 0; step < 2 * NP; ++step) {
        const int j = step >> 1, hh = step & 1;
        if (step + 1 < 2 * NP) {
            const int jn = (step + 1) >> 1, hn = (step + 1) & 1;
#pragma unroll
            for (int c = 0; c < 8; ++c)
                vb[(step + 1) & 1][c] = *reinterpret_cast<const u32x4_t*>(val_row(jn) + hn * 128 + c * 16);
        }
        const uint32_t wj = w[j];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[32 * hh + 4 * c + e] = dot2_bf16(wj, vb[step & 1][c][e], acc[32 * hh + 4 * c + e]);
        }
    }

    // ---- output: the 4 lanes of a quad (4 consecutive frames) transpose
    // each half of their 8 x 16-byte chunks (xor-butterfly over lane
    // distances 2, 1), so that a store writes 64 contiguous bytes (half a
    // head row) of each of 16 frames instead of 16 bytes of each of 64 ----
    const float inv = 1.f / den;
    uint32_t ov[8][4];  // ov[c]: channels 8c .. 8c+7, bf16 pairs
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[c][e] = pack_bf16x2(acc[8 * c + 2 * e] * inv, acc[8 * c + 2 * e + 1] * inv);
    const int lb = lt & 3;
    // One butterfly stage over lane distance j within each quad: the lower
    // lane takes the partner's chunk c0 into slot c0+j, the upper lane the
    // partner's chunk c0+j into slot c0 (ds_swizzle reads the partner).
    auto stage = [&](auto dist) {
        constexpr int j = decltype(dist)::value;
        constexpr int pattern = 0x1f | (j << 10);  // ds_swizzle bit mode: lane ^ j
        const bool upper = (lb & j) != 0;
#pragma unroll
        for (int c0 = 0; c0 < 8; ++c0) {
            if (c0 & j) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t send = upper ? ov[c0][e] : ov[c0 + j][e];
                const uint32_t got = (uint32_t)__builtin_amdgcn_ds_swizzle((int)send, pattern);
                if (upper)
                    ov[c0][e] = got;
                else
                    ov[c0 + j][e] = got;
            }
        }
    };
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 1>{});
    // lane 4a+b now holds chunks b and b+4 of frames 4a .. 4a+3 (slot k:
    // frame 4a + k%4, chunk b + 4*(k/4))
    const int tg = it.t0 + (lt & ~3);
#pragma unroll
    for (int kf = 0; kf < 8; ++kf) {
        const int tf = tg + (kf & 3);
        if (tf < tend)
            *reinterpret_cast<u32x4_t*>(o + (int64_t)(tf - g.f0) * rs + col + (lb + 4 * (kf >> 2)) * 8) =
                u32x4_t{ov[kf][0], ov[kf][1], ov[kf][2], ov[kf][3]};
    }
}

// One work item of a half workgroup (256 threads, lt = 0..255): stage it
// (STAGE) or compute it.  Items below g.nfull are one strip x 256 queries;
// the rest are remainder items of M strips (s0 .. s0+M-1) x the last
// nq - 256*nchunks queries, strip j in slice j of the buffer, threads
// 256/M*j .. 256/M*(j+1)-1 (waves 4/M*j ..) on it.
template <int NL, int NG, int M, bool STAGE>
__device__ __forceinline__ void dda_item_run(char* __restrict__ buf, const uint16_t* __restrict__ q,
                                             const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                             uint16_t* __restrict__ o, const DdaGeo& g, int64_t rs, int heads,
                                             int idx, int lt, uint32_t (&qv)[32]) {
    if (M == 1 || idx < g.nfull) {
        const DdaItem it{idx % g.nstrips, g.f0 + (idx / g.nstrips) * DDA_TQ};
        if constexpr (STAGE)
            dda_stage<NL, NG, DDA_TQ, 256>(buf, q, k, v, g, rs, heads, it, lt, qv);
        else
            dda_compute<NL, NG, DDA_TQ>(buf, o, g, rs, heads, it, lt, qv);
    } else {
        constexpr int R = DdaRemR<M>, NT = 256 / M;
        const int j = lt / NT, ls = lt % NT;
        const DdaItem it{(idx - g.nfull) * M + j, g.f0 + g.nchunks * DDA_TQ};
        if (it.strip >= g.nstrips) return;  // the last remainder item may hold fewer strips
        char* slice = buf + j * DdaSlice<R>::BYTES;
        if constexpr (STAGE)
            dda_stage<NL, NG, R, NT>(slice, q, k, v, g, rs, heads, it, ls, qv);
        else
            dda_compute<NL, NG, R>(slice, o, g, rs, heads, it, ls, qv);
    }
}

// Persistent, two-phase pipelined kernel: workgroup w takes items
// w, w + G, w + 2G, ... (G = gridDim.x); its half g (threads 256g..256g+255)
// takes the items with odd (g = 1) or even (g = 0) position in that list.
// Phase p: half 0 stages its item p/2 (p even) or computes item (p-1)/2 (p
// odd); half 1 stages item (p-1)/2 (p odd) or computes item (p-2)/2 (p even,
// p >= 2).  Every thread runs every phase and barrier.
template <int NL, int NG, int M>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
dda_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
         uint16_t* __restrict__ o, DdaGeo g) {
    __shared__ __attribute__((aligned(16))) char lds[2 * DDA_LDS_BYTES];
    const int heads = g.C / DDA_D;
    const int64_t rs = (int64_t)g.S * g.C;
    const int half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8), lt = threadIdx.x & 255;
    char* buf = lds + half * DDA_LDS_BYTES;
    const int G = gridDim.x, w = blockIdx.x;
    const int mine = w < g.nitems ? (g.nitems - w + G - 1) / G : 0;  // items of this workgroup
    const int jh = (mine - half + 1) / 2;                             // items of this half
    const int j0 = (mine + 1) / 2, j1 = mine / 2;
    const int phases = max(2 * j0, 2 * j1 + 1);
    uint32_t qv[32];
    for (int p = 0; p < phases; ++p) {
        const int rel = p - half;                 // half 0: rel = p, half 1: rel = p - 1
        if (rel >= 0) {
            const int j = rel >> 1;
            if (j < jh) {
                const int idx = w + (2 * j + half) * G;
                if ((rel & 1) == 0)
                    dda_item_run<NL, NG, M, true>(buf, q, k, v, o, g, rs, heads, idx, lt, qv);
                else
                    dda_item_run<NL, NG, M, false>(buf, q, k, v, o, g, rs, heads, idx, lt, qv);
            }
        }
        __syncthreads();
    }
}

// float32 I/O: one query per thread, keys read through the cache.
// n_local, n_global: 16 or 0.
__global__ void __launch_bounds__(64) dda_f32(const float* __restrict__ q, const float* __restrict__ k,
                                              const float* __restrict__ v, float* __restrict__ o, DdaGeo g,
                                              int n_local, int n_global) {
    const int heads = g.C / DDA_D;
    const int64_t qi = (int64_t)blockIdx.x * 64 + threadIdx.x;  // (t - f0, s, h) flattened
    if (qi >= (int64_t)g.nq * g.S * heads) return;
    const int h = (int)(qi % heads);
    const int s = (int)((qi / heads) % g.S);
    const int i = (int)(qi / ((int64_t)heads * g.S));
    const int t = g.f0 + i, F = g.F;
    const int64_t rs = (int64_t)g.S * g.C, col = (int64_t)s * g.C + h * DDA_D;
    const int nl = F < n_local ? F : n_local;
    const int st = dda_start(t, F);
    const float* kgb = g.kg ? static_cast<const float*>(g.kg) : k;
    const float* vgb = g.vg ? static_cast<const float*>(g.vg) : v;
    // row offset (elements) of key j in k / v (local) or kgb / vgb (global)
    auto row = [&](int j) -> int64_t {
        const int gi = j - nl;
        return j < nl ? (int64_t)(st + j - g.kf0) * rs
                      : (g.kg ? (int64_t)gi * rs : (((int64_t)gi * F) / DDA_G - g.kf0) * rs);
    };
    float sc[DDA_L + DDA_G];
    const int n = nl + n_global;
    const float* qr = q + (int64_t)i * rs + col;
    float m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        const float* kr = (j < nl ? k : kgb) + row(j) + col;
        float a = 0.f;
        for (int d = 0; d < DDA_D; ++d) a = fmaf(qr[d], kr[d], a);
        sc[j] = a * g.sl2e;
        m = fmaxf(m, sc[j]);
    }
    float acc[DDA_D];
    for (int d = 0; d < DDA_D; ++d) acc[d] = 0.f;
    float den = 0.f;
    for (int j = 0; j < n; ++j) {
        float p = __builtin_amdgcn_exp2f(sc[j] - m);
        den += p;
        const float* vr = (j < nl ? v : vgb) + row(j) + col;
        for (int d = 0; d < DDA_D; ++d) acc[d] = fmaf(p, vr[d], acc[d]);
    }
    float inv = 1.f / den;
    float* orow = o + (int64_t)i * rs + col;
    for (int d = 0; d < DDA_D; ++d) orow[d] = acc[d] * inv;
}

}  // namespace vinf

namespace vinf_host {
using namespace vinf;

vinf_status launch_dda(const void* q, const void* k, const void* v, const void* kg, const void* vg, void* o,
                       int F, int f0, int nq, int kf0, int kend, int S, int C, int n_local, int n_global,
                       float scale, vinf_dtype dt, hipStream_t st) {
    const int heads = C / DDA_D;
    if ((int64_t)S * heads > 0x7fffffff)
        return fail(VINF_ERR_UNSUPPORTED, "dual_domain_attn: more than 2^31 (location, head) strips");
    DdaGeo g;
    g.kg = kg;
    g.vg = vg;
    g.F = F;
    g.f0 = f0;
    g.nq = nq;
    g.kf0 = kf0;
    g.kend = kend;
    g.S = S;
    g.C = C;
    g.nstrips = S * heads;
    g.nchunks = g.nfull = g.nitems = 0;
    g.sl2e = scale * 1.4426950408889634f;
    if (dt == VINF_BF16) {
        // Remainder packing: r = nq % 256 leftover queries per strip go M strips
        // to an item when they fit M slices (M = 1: one partial item per strip).
        const int r = nq % DDA_TQ;
        const int M = (r > 0 && r <= DdaRemR<4>) ? 4 : ((r > 0 && r <= DdaRemR<2>) ? 2 : 1);
        const int64_t nchunks = M == 1 ? (nq + DDA_TQ - 1) / DDA_TQ : nq / DDA_TQ;
        const int64_t nfull = (int64_t)g.nstrips * nchunks;
        const int64_t items = nfull + (M == 1 ? 0 : ((int64_t)g.nstrips + M - 1) / M);
        if (items > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "dual_domain_attn: too many work items");
        g.nchunks = (int)nchunks;
        g.nfull = (int)nfull;
        g.nitems = (int)items;
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            return fail(VINF_ERR_HIP, "dual_domain_attn: cannot query the device");
        // one persistent workgroup per CU, each with at least two items
        const dim3 grid((uint32_t)std::min<int64_t>(cus, (items + 1) / 2)), block(512);
        const uint16_t *qb = static_cast<const uint16_t*>(q), *kb = static_cast<const uint16_t*>(k),
                       *vb = static_cast<const uint16_t*>(v);
        uint16_t* ob = static_cast<uint16_t*>(o);
        auto run = [&](auto nl, auto ng) {
            constexpr int NL = decltype(nl)::value, NG = decltype(ng)::value;
            if (M == 4)
                hipLaunchKernelGGL((dda_bf16<NL, NG, 4>), grid, block, 0, st, qb, kb, vb, ob, g);
            else if (M == 2)
                hipLaunchKernelGGL((dda_bf16<NL, NG, 2>), grid, block, 0, st, qb, kb, vb, ob, g);
            else
                hipLaunchKernelGGL((dda_bf16<NL, NG, 1>), grid, block, 0, st, qb, kb, vb, ob, g);
        };
        using K16 = std::integral_constant<int, DDA_L>;
        using K0 = std::integral_constant<int, 0>;
        if (n_local > 0 && n_global > 0)
            run(K16{}, K16{});
        else if (n_local > 0)
            run(K16{}, K0{});
        else
            run(K0{}, K16{});
    } else {
        const int64_t nqs = (int64_t)nq * S * heads;
        const int64_t blocks = (nqs + 63) / 64;
        if (blocks > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "dual_domain_attn: grid too large");
        hipLaunchKernelGGL(dda_f32, dim3((uint32_t)blocks), dim3(64), 0, st, static_cast<const float*>(q),
                           static_cast<const float*>(k), static_cast<const float*>(v), static_cast<float*>(o), g,
                           n_local, n_global);
    }
    return check_launch("dual_domain_attn");
}

}  // namespace vinf_host

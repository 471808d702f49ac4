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
//     A whole-strip item stages without a branch: buffer loads whose range
//     ends at the last frame in k/v read rows outside it as zero (frames
//     whose 290 strides fit 32 bits; larger frames guard each load).
//   * Scores: q stays in 32 VGPRs as bf16 pairs; 32 keys x 32 v_dot2c each.
//     The lane holds all 32 scores, so the softmax is lane-local: one max,
//     exp2 with log2(e)*scale folded in, no cross-lane traffic.  A K row's
//     eight 16-byte reads are issued a row ahead and waited for once (one
//     s_waitcnt per row, not per read: with one computing wave per SIMD
//     every instruction of that wave costs an issue slot); the weighted sum
//     does the same per half pair row.
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
//   * Item order: items are numbered strip-major (a strip's frame chunks in
//     a row) and every workgroup takes a contiguous range, so consecutive
//     items of a workgroup are neighbouring chunks of one strip whose shared
//     window frames come from L2; when q, k and v are one tensor and the
//     key set is full, workgroups take chunk-major items round-robin
//     instead (measured faster there).
//   * Pipelining: one persistent 512-thread workgroup per CU owns two LDS
//     buffers (2 x 80 KB).  Its two 256-thread halves alternate: while one
//     half stages its next work item (HBM -> LDS, plus its q rows into
//     registers; a whole-strip item issues all its loads before its first
//     LDS write), the other computes from its own buffer; a workgroup barrier
//     ends each phase.  HBM traffic and the VALU-bound compute overlap
//     instead of alternating.  The computing waves run at raised wave
//     priority (s_setprio), so they issue first on their SIMDs.
// Projected kernel (dda_proj_bf16): the Q/K/V projection inside the
// attention's work items (see its comment below).
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
// from f0 + 256*chunk), numbered strip * nchunks + chunk in dda_bf16 and
// chunk * nstrips + strip in the projected kernel, then the remainder items
// (packed kernels only).
struct DdaGeo {
    const void* kg;
    const void* vg;
    int F, f0, nq, kf0, kend;
    int S, C, nstrips, nchunks, nfull, nitems;
    int chunk_major;  // dda_bf16 item order (below)
    float sl2e;
};

struct DdaItem {
    int strip, t0;
    int s, h;  // location and head of the strip (strip = s * heads + h)
};

__device__ __forceinline__ DdaItem dda_item(int strip, int t0, int heads) {
    return DdaItem{strip, t0, strip / heads, strip % heads};
}

// V rows f, f+1 (16 bytes each, 8 dims) -> two 16-byte pair chunks
// (v[f][d], v[f+1][d]) in LDS at dst.
__device__ __forceinline__ void dda_put_pairs(char* dst, const u32x4_t& a, const u32x4_t& b) {
    const u32x4_t w0 = {perm_lo(a[0], b[0]), perm_hi(a[0], b[0]), perm_lo(a[1], b[1]), perm_hi(a[1], b[1])};
    const u32x4_t w1 = {perm_lo(a[2], b[2]), perm_hi(a[2], b[2]), perm_lo(a[3], b[3]), perm_hi(a[3], b[3])};
    *reinterpret_cast<u32x4_t*>(dst) = w0;
    *reinterpret_cast<u32x4_t*>(dst + 16) = w1;
}

// Stage one strip's rows for queries t0 .. t0+R-1 into its slice `buf`
// (NT threads, lt = 0..NT-1) and load the q row of query t0 + lt into qv.
// NL / NG: local / global keys present (16 or 0).  A thread moves 16-byte
// chunks: chunk lt&7 of local K rows lt>>3 + (NT/8)*i, the same of V pair
// rows, and global-row tasks lt + NT*n.  A full item (R = 256) issues every
// load before its first LDS write, so its stage costs one memory round trip;
// the smaller remainder slices write each row kind before loading the next
// (fewer registers live at once).  Whole-strip items use this stage only for
// frames too large for dda_stage_b32's 32-bit offsets.
template <int NL, int NG, int R, int NT, bool QROWS = R == DDA_TQ>
__device__ __forceinline__ void dda_stage(char* __restrict__ buf, const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                          const DdaGeo& g, int64_t rs, int heads, DdaItem it, int lt,
                                          uint32_t (&qv)[32]) {
    using SL = DdaSlice<R>;
    constexpr bool ALL_FIRST = R == DDA_TQ;
    constexpr int RSTEP = NT / 8;  // rows one pass of the threads covers (8 chunks per row)
    constexpr int NIK = NL > 0 ? (SL::KROWS + RSTEP - 1) / RSTEP : 1;
    constexpr int NIV = NL > 0 ? (SL::VPAIRS + RSTEP - 1) / RSTEP : 1;
    constexpr int NGTASK = DDA_G * 8 + (DDA_G / 2) * 8;  // global K row chunks, then V pair chunks
    constexpr int NGT = NG > 0 ? (NGTASK + NT - 1) / NT : 1;
    const int s = it.s, h = it.h;
    const int64_t col = (int64_t)s * g.C + h * DDA_D;
    const int t = it.t0 + lt;
    const int c8 = lt & 7, r0 = lt >> 3;
    // QROWS (whole-strip items): the q rows of a wave's 64 queries are loaded
    // as whole 128-byte rows (8 lanes a row, 8 rows an instruction: an eighth
    // of the cache-line requests of one row per lane) and each lane gets its
    // own row through LDS, in rows of the K region that only this wave writes
    // later (its K chunks are rows r0 + RSTEP*i: 8 rows of every 32).  Lanes
    // past the last query take the last query's row (their results are dropped).
    static_assert(!QROWS || (ALL_FIRST && NT == 256), "whole q rows: whole-strip items");
    u32x4_t qw[QROWS ? 8 : 1];
    auto qtemp = [&](int rq) { return buf + SL::KL + ((lt & ~63) / 8 + RSTEP * (rq >> 3) + (rq & 7)) * DDA_KSTR; };
    if constexpr (QROWS) {
        const int tw = it.t0 + (lt & ~63), last = g.f0 + g.nq - 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tr = min(tw + 8 * i + ((lt & 63) >> 3), last);
            qw[i] = *reinterpret_cast<const u32x4_t*>(q + (int64_t)(tr - g.f0) * rs + col + c8 * 8);
        }
    } else if (t < g.f0 + g.nq) {
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
    // Frames outside [kf0, kend) are not in k/v: their rows are zero-filled
    // (only frames past the video's last frame, or the unused half of a pair
    // row, which carry no weight, fall outside).
    int nkr = 0, np = 0;
    u32x4_t ku[NIK], va[NIV], vb[NIV];
    auto store_k = [&]() {
        char* dst = buf + SL::KL + r0 * DDA_KSTR + c8 * 16;
#pragma unroll
        for (int i = 0; i < NIK; ++i)
            if (r0 + RSTEP * i < nkr) *reinterpret_cast<u32x4_t*>(dst + RSTEP * i * DDA_KSTR) = ku[i];
    };
    auto q_handover = [&]() {
        // row 8i + lane/8 of the wave's 64, chunk lane%8, then the lane's own row
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4_t*>(qtemp(8 * i + ((lt & 63) >> 3)) + c8 * 16) = qw[i];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4_t u = *reinterpret_cast<const u32x4_t*>(qtemp(lt & 63) + c * 16);
            qv[4 * c] = u[0];
            qv[4 * c + 1] = u[1];
            qv[4 * c + 2] = u[2];
            qv[4 * c + 3] = u[3];
        }
    };
    auto store_v = [&]() {
        char* dst = buf + SL::VP + r0 * DDA_VSTR + c8 * 32;
#pragma unroll
        for (int i = 0; i < NIV; ++i)
            if (r0 + RSTEP * i < np) dda_put_pairs(dst + RSTEP * i * DDA_VSTR, va[i], vb[i]);
    };
    if constexpr (NL > 0) {
        const int tlast = min(it.t0 + R, g.f0 + g.nq) - 1;
        const int lo = dda_start(it.t0, g.F);
        const int stl = dda_start(tlast, g.F);
        nkr = stl + DDA_L - lo;                       // K rows [lo, lo+nkr), <= R + 15
        const int plo = lo & ~1;
        np = (stl + DDA_L + 2 - plo) >> 1;            // V pairs cover [plo, plo+2np), <= (R + 18) / 2
        const uint16_t* ks = k + col + (int64_t)(lo + r0 - g.kf0) * rs + c8 * 8;
#pragma unroll
        for (int i = 0; i < NIK; ++i) {
            const int r = r0 + RSTEP * i;
            ku[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (r < nkr && lo + r < g.kend) ku[i] = *reinterpret_cast<const u32x4_t*>(ks + (int64_t)(RSTEP * i) * rs);
        }
        if constexpr (!ALL_FIRST) store_k();
        const uint16_t* vs = v + col + (int64_t)(plo + 2 * r0 - g.kf0) * rs + c8 * 8;
#pragma unroll
        for (int i = 0; i < NIV; ++i) {
            const int p = r0 + RSTEP * i, fa = plo + 2 * p;
            va[i] = u32x4_t{0u, 0u, 0u, 0u};
            vb[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (p < np && fa >= g.kf0 && fa < g.kend)
                va[i] = *reinterpret_cast<const u32x4_t*>(vs + (int64_t)(2 * RSTEP * i) * rs);
            if (p < np && fa + 1 < g.kend)
                vb[i] = *reinterpret_cast<const u32x4_t*>(vs + (int64_t)(2 * RSTEP * i + 1) * rs);
        }
        if constexpr (!ALL_FIRST) store_v();
    }
    if constexpr (NG > 0) {
        const uint16_t* kgb = g.kg ? static_cast<const uint16_t*>(g.kg) : k;
        const uint16_t* vgb = g.vg ? static_cast<const uint16_t*>(g.vg) : v;
        auto grow = [&](int i) -> int64_t {  // row of global frame i in kgb / vgb
            return g.kg ? (int64_t)i : (int64_t)(((int64_t)i * g.F) / DDA_G) - g.kf0;
        };
        u32x4_t ga[NGT], gb[NGT];
#pragma unroll
        for (int n = 0; n < NGT; ++n) {
            const int task = lt + NT * n;
            if (task < DDA_G * 8) {
                ga[n] = *reinterpret_cast<const u32x4_t*>(kgb + col + grow(task >> 3) * rs + (task & 7) * 8);
            } else if (task < NGTASK) {
                const int p = (task - DDA_G * 8) >> 3, oc = task & 7;
                ga[n] = *reinterpret_cast<const u32x4_t*>(vgb + col + grow(2 * p) * rs + oc * 8);
                gb[n] = *reinterpret_cast<const u32x4_t*>(vgb + col + grow(2 * p + 1) * rs + oc * 8);
            }
        }
        if constexpr (QROWS) q_handover();
        if constexpr (ALL_FIRST && NL > 0) {
            store_k();
            store_v();
        }
#pragma unroll
        for (int n = 0; n < NGT; ++n) {
            const int task = lt + NT * n;
            if (task < DDA_G * 8)
                *reinterpret_cast<u32x4_t*>(buf + SL::KG + (task >> 3) * 128 + (task & 7) * 16) = ga[n];
            else if (task < NGTASK)
                dda_put_pairs(buf + SL::VG + ((task - DDA_G * 8) >> 3) * 256 + (task & 7) * 32, ga[n], gb[n]);
        }
    } else if constexpr (ALL_FIRST) {
        if constexpr (QROWS) q_handover();
        if constexpr (NL > 0) {
            store_k();
            store_v();
        }
    }
}

// Loads at byte offsets outside [0, bytes) of a buffer resource read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dda_rsrc(const uint16_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)bytes, 0x00020000);
}

// Frame strides for which a whole-strip stage can address its rows with
// 32-bit buffer offsets (dda_stage_b32): 290 of them below 4 GiB.
constexpr int64_t DDA_B32_MAX_RS = (int64_t)((1ull << 32) / (290ull * 2ull));

// The stage of a whole-strip item (R = 256 queries, 256 threads) without a
// branch.  The item's K rows (from its first window frame lo) and V rows
// (from max(lo & ~1, kf0)) are each one buffer resource whose range ends at
// kend, so a frame outside [kf0, kend) reads as zero (the row before kf0 has
// a negative offset, which wraps past the range); every load and store is
// unconditional.  Rows past the slice (K rows >= KROWS, pairs >= VPAIRS) load
// and store the slice's last row again: the same value to the same place.
// Rows past the windows' frames (>= nkr, pairs >= np) are staged but never
// read.  Lanes past the last query load the last query's row.  Loads are all
// issued before the first LDS write, as in dda_stage.
template <int NL, int NG, bool QROWS>
__device__ __forceinline__ void dda_stage_b32(char* __restrict__ buf, const uint16_t* __restrict__ q,
                                              const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                              const DdaGeo& g, int64_t rs, int heads, DdaItem it, int lt,
                                              uint32_t (&qv)[32]) {
    using SL = DdaFull;
    constexpr int RSTEP = 32;  // rows one pass of the 256 threads covers (8 chunks per row)
    constexpr int NIK = (SL::KROWS + RSTEP - 1) / RSTEP;
    constexpr int NIV = (SL::VPAIRS + RSTEP - 1) / RSTEP;
    static_assert((NIK - 1) * RSTEP + RSTEP - 1 >= SL::KROWS - 1 && (NIK - 1) * RSTEP <= SL::KROWS - 1, "K passes");
    static_assert((NIV - 1) * RSTEP + RSTEP - 1 >= SL::VPAIRS - 1 && (NIV - 1) * RSTEP <= SL::VPAIRS - 1, "V passes");
    const int s = it.s, h = it.h;
    const int64_t col = (int64_t)s * g.C + h * DDA_D;
    const int c8 = lt & 7, r0 = lt >> 3;
    const int last = g.f0 + g.nq - 1;
    const uint32_t fb = (uint32_t)rs * 2u;  // frame stride in bytes
    u32x4_t qw[QROWS ? 8 : 1];
    if constexpr (QROWS) {
        // 8 lanes a row, 8 rows an instruction; handed over through LDS below
        const int tw = it.t0 + (lt & ~63);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tr = min(tw + 8 * i + ((lt & 63) >> 3), last);
            qw[i] = *reinterpret_cast<const u32x4_t*>(q + (int64_t)(tr - g.f0) * rs + col + c8 * 8);
        }
    } else {
        const uint16_t* qrow = q + (int64_t)(min(it.t0 + lt, last) - g.f0) * rs + col;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4_t u = *reinterpret_cast<const u32x4_t*>(qrow + c * 8);
            qv[4 * c] = u[0];
            qv[4 * c + 1] = u[1];
            qv[4 * c + 2] = u[2];
            qv[4 * c + 3] = u[3];
        }
    }
    u32x4_t ku[NL > 0 ? NIK : 1], va[NL > 0 ? NIV : 1], vb[NL > 0 ? NIV : 1];
    if constexpr (NL > 0) {
        const int lo = dda_start(it.t0, g.F);
        const int plo = lo & ~1, vf = max(plo, g.kf0);
        const __amdgpu_buffer_rsrc_t kr =
            dda_rsrc(k + col + (int64_t)(lo - g.kf0) * rs, (uint32_t)min(g.kend - lo, SL::KROWS) * fb);
        const __amdgpu_buffer_rsrc_t vr =
            dda_rsrc(v + col + (int64_t)(vf - g.kf0) * rs, (uint32_t)min(g.kend - vf, 2 * SL::VPAIRS) * fb);
        const uint32_t ko = (uint32_t)r0 * fb + (uint32_t)c8 * 16u;
#pragma unroll
        for (int i = 0; i < NIK; ++i) {
            const uint32_t off = i < NIK - 1 ? ko + (uint32_t)(RSTEP * i) * fb
                                             : (uint32_t)min(r0 + RSTEP * i, SL::KROWS - 1) * fb + (uint32_t)c8 * 16u;
            ku[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, (int)off, 0, 0);
        }
        // pair p holds frames plo + 2p and plo + 2p + 1 (plo - vf is 0 or -1)
        const uint32_t vo = (uint32_t)(plo - vf + 2 * r0) * fb + (uint32_t)c8 * 16u;
#pragma unroll
        for (int i = 0; i < NIV; ++i) {
            const uint32_t off = i < NIV - 1
                                     ? vo + (uint32_t)(2 * RSTEP * i) * fb
                                     : (uint32_t)(plo - vf + 2 * min(r0 + RSTEP * i, SL::VPAIRS - 1)) * fb +
                                           (uint32_t)c8 * 16u;
            va[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, (int)off, 0, 0);
            vb[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, (int)(off + fb), 0, 0);
        }
    }
    constexpr int NGTASK = DDA_G * 8 + (DDA_G / 2) * 8;  // global K row chunks, then V pair chunks
    static_assert(NGTASK <= 256, "one global task per thread");
    u32x4_t ga = u32x4_t{0u, 0u, 0u, 0u}, gb = ga;
    if constexpr (NG > 0) {
        const uint16_t* kgb = g.kg ? static_cast<const uint16_t*>(g.kg) : k;
        const uint16_t* vgb = g.vg ? static_cast<const uint16_t*>(g.vg) : v;
        auto grow = [&](int i) -> int64_t {  // row of global frame i in kgb / vgb
            return g.kg ? (int64_t)i : (int64_t)(((int64_t)i * g.F) / DDA_G) - g.kf0;
        };
        // wave-uniform: waves 0-1 the K rows, wave 2 the V pairs, wave 3 none
        if (lt < DDA_G * 8) {
            ga = *reinterpret_cast<const u32x4_t*>(kgb + col + grow(lt >> 3) * rs + c8 * 8);
        } else if (lt < NGTASK) {
            const int p = (lt - DDA_G * 8) >> 3;
            ga = *reinterpret_cast<const u32x4_t*>(vgb + col + grow(2 * p) * rs + c8 * 8);
            gb = *reinterpret_cast<const u32x4_t*>(vgb + col + grow(2 * p + 1) * rs + c8 * 8);
        }
    }
    if constexpr (QROWS) {
        // row 8i + lane/8 of the wave's 64, chunk lane%8, then the lane's own
        // row, in K rows that only this wave writes later (its K chunks are
        // rows r0 + 32i: 8 rows of every 32)
        auto qtemp = [&](int rq) { return buf + SL::KL + ((lt & ~63) / 8 + RSTEP * (rq >> 3) + (rq & 7)) * DDA_KSTR; };
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4_t*>(qtemp(8 * i + ((lt & 63) >> 3)) + c8 * 16) = qw[i];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4_t u = *reinterpret_cast<const u32x4_t*>(qtemp(lt & 63) + c * 16);
            qv[4 * c] = u[0];
            qv[4 * c + 1] = u[1];
            qv[4 * c + 2] = u[2];
            qv[4 * c + 3] = u[3];
        }
    }
    if constexpr (NL > 0) {
        char* kd = buf + SL::KL + r0 * DDA_KSTR + c8 * 16;
#pragma unroll
        for (int i = 0; i < NIK - 1; ++i) *reinterpret_cast<u32x4_t*>(kd + RSTEP * i * DDA_KSTR) = ku[i];
        *reinterpret_cast<u32x4_t*>(buf + SL::KL + min(r0 + RSTEP * (NIK - 1), SL::KROWS - 1) * DDA_KSTR + c8 * 16) =
            ku[NIK - 1];
        char* vd = buf + SL::VP + r0 * DDA_VSTR + c8 * 32;
#pragma unroll
        for (int i = 0; i < NIV - 1; ++i) dda_put_pairs(vd + RSTEP * i * DDA_VSTR, va[i], vb[i]);
        dda_put_pairs(buf + SL::VP + min(r0 + RSTEP * (NIV - 1), SL::VPAIRS - 1) * DDA_VSTR + c8 * 32, va[NIV - 1],
                      vb[NIV - 1]);
    }
    if constexpr (NG > 0) {
        if (lt < DDA_G * 8)
            *reinterpret_cast<u32x4_t*>(buf + SL::KG + (lt >> 3) * 128 + c8 * 16) = ga;
        else if (lt < NGTASK)
            dda_put_pairs(buf + SL::VG + ((lt - DDA_G * 8) >> 3) * 256 + c8 * 32, ga, gb);
    }
}

// a.x*b.x + a.y*b.y for bf16 pairs, fp32 (the three-operand v_dot2_f32_bf16
// with a zero addend: a chain starts without a zeroed accumulator).
__device__ __forceinline__ float dot2_zero(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Wait until at most n LDS reads of this wave are outstanding (s_waitcnt
// lgkmcnt(n), n <= 15).  The scheduling barriers keep the reads issued before
// it above it and the dot products after it below it.
__device__ __forceinline__ void lds_wait(int n) {
    __builtin_amdgcn_sched_barrier(0);
    switch (n) {
#define VINF_LGKM_CASE(k) \
    case k: __builtin_amdgcn_s_waitcnt(0xC07F | ((k) << 8)); break;
        VINF_LGKM_CASE(0) VINF_LGKM_CASE(1) VINF_LGKM_CASE(2) VINF_LGKM_CASE(3)
        VINF_LGKM_CASE(4) VINF_LGKM_CASE(5) VINF_LGKM_CASE(6) VINF_LGKM_CASE(7)
        VINF_LGKM_CASE(8) VINF_LGKM_CASE(9) VINF_LGKM_CASE(10) VINF_LGKM_CASE(11)
        VINF_LGKM_CASE(12) VINF_LGKM_CASE(13) VINF_LGKM_CASE(14) VINF_LGKM_CASE(15)
#undef VINF_LGKM_CASE
        default: __builtin_amdgcn_s_waitcnt(0xC07F | (15 << 8)); break;
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Compute query t0 + lt of a strip staged in slice `buf` (layout DdaSlice<R>).
// SHORT: the video may have fewer frames than the local window.
template <int NL, int NG, int R, bool SHORT = true>
__device__ __forceinline__ void dda_compute(const char* __restrict__ buf, uint16_t* __restrict__ o,
                                            const DdaGeo& g, int64_t rs, int heads, DdaItem it, int lt,
                                            const uint32_t (&qv)[32]) {
    using SL = DdaSlice<R>;
    constexpr int NK = NL + NG;                 // keys
    constexpr int NLP = NL > 0 ? 9 : 0;         // local V pair rows
    constexpr int NP = NLP + (NG > 0 ? 8 : 0);  // V pair rows
    // Lanes past the last query stay in (the output transpose below moves
    // data between the 4 lanes of a quad) and compute the last query's
    // windows; their own results are not stored.
    const int tend = g.f0 + g.nq;
    const int t = min(it.t0 + lt, tend - 1);
    const int s = it.s, h = it.h;
    const int64_t col = (int64_t)s * g.C + h * DDA_D;
    const int F = g.F;
    const int lo = dda_start(it.t0, F);
    const int plo = lo & ~1;
    const int nl = F < DDA_L ? F : DDA_L;
    const int st = dda_start(t, F);

    // ---- scores: one K row (8 x 16 B) per key; the next row's reads are
    // issued before the current row's dot products, and one wait per row
    // covers all eight (a wait per 16-byte read costs an issue slot each) ----
    float sc[NK];
    const char* krow = buf + SL::KL + (st - lo) * DDA_KSTR;
    auto key_row = [&](int i) -> const char* {
        return i < NL ? krow + i * DDA_KSTR : buf + SL::KG + (i - NL) * 128;
    };
    u32x4_t kb[2][8];
    uint32_t klast = 0;  // last dword of the previous K row
#pragma unroll
    for (int c = 0; c < 8; ++c) kb[0][c] = *reinterpret_cast<const u32x4_t*>(key_row(0) + c * 16);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        if (i + 1 < NK) {
#pragma unroll
            for (int c = 0; c < 8; ++c) kb[(i + 1) & 1][c] = *reinterpret_cast<const u32x4_t*>(key_row(i + 1) + c * 16);
        }
        lds_wait(i + 1 < NK ? 8 : 0);  // row i has landed; row i+1's 8 reads may be in flight
        float a = dot2_zero(qv[0], kb[i & 1][0][0]);
        // the previous row's last product goes between this zero-addend
        // dot2 and the first use of its result (which would otherwise wait
        // one cycle); each score still sums its products in order
        if (i > 0) sc[i - 1] = dot2_bf16(qv[31], klast, sc[i - 1]);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4_t u = kb[i & 1][c];
            if (c > 0) a = dot2_bf16(qv[4 * c], u[0], a);
            a = dot2_bf16(qv[4 * c + 1], u[1], a);
            a = dot2_bf16(qv[4 * c + 2], u[2], a);
            if (c < 7) a = dot2_bf16(qv[4 * c + 3], u[3], a);
        }
        klast = kb[i & 1][7][3];
        sc[i] = a;
    }
    sc[NK - 1] = dot2_bf16(qv[31], klast, sc[NK - 1]);

    // The weighted sum's first half pair row is read now, so that the
    // softmax below covers its latency (the scheduling barrier keeps the
    // reads here).
    const char* vrow0 = NLP > 0 ? buf + SL::VP + ((st - plo) >> 1) * DDA_VSTR : buf + SL::VG;
    u32x4_t vfirst[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) vfirst[c] = *reinterpret_cast<const u32x4_t*>(vrow0 + c * 16);
    __builtin_amdgcn_sched_barrier(0);

    // ---- lane-local softmax (base 2, scale folded in) ----
    // (the maximum is taken before the scaling: sl2e > 0 keeps the order)
    // A video shorter than the window has nl < 16 local keys: the rest are
    // masked out (SHORT; a whole-strip item has 256 query frames, so 16).
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        if (SHORT) sc[j] = (j < NL && j >= nl) ? -INFINITY : sc[j];
        m = fmaxf(m, sc[j]);
    }
    const float msl = -(m * g.sl2e);
#pragma unroll
    for (int j = 0; j < NK; ++j) sc[j] = __builtin_amdgcn_exp2f(fmaf(sc[j], g.sl2e, msl));

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
    float acc[DDA_D];  // set by pair row 0
    const char* vrow = buf + SL::VP + ((st - plo) >> 1) * DDA_VSTR;
    auto val_row = [&](int j) -> const char* {
        return j < NLP ? vrow + j * DDA_VSTR : buf + SL::VG + (j - NLP) * 256;
    };
    // half rows (32 dims, 8 x 16 B) double-buffered: step 2j + hh reads
    // dims 32*hh.. of pair row j; one wait per step
    u32x4_t vb[2][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) vb[0][c] = vfirst[c];  // val_row(0), read before the softmax
#pragma unroll
    for (int step = 0; step < 2 * NP; ++step) {
        const int j = step >> 1, hh = step & 1;
        if (step + 1 < 2 * NP) {
            const int jn = (step + 1) >> 1, hn = (step + 1) & 1;
#pragma unroll
            for (int c = 0; c < 8; ++c)
                vb[(step + 1) & 1][c] = *reinterpret_cast<const u32x4_t*>(val_row(jn) + hn * 128 + c * 16);
        }
        lds_wait(step + 1 < 2 * NP ? 8 : 0);
        const uint32_t wj = w[j];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float& r = acc[32 * hh + 4 * c + e];
                r = j == 0 ? dot2_zero(wj, vb[step & 1][c][e]) : dot2_bf16(wj, vb[step & 1][c][e], r);
            }
        }
    }

    // ---- output: the 4 lanes of a quad (4 consecutive frames) transpose
    // each half of their 8 x 16-byte chunks (xor-butterfly over lane
    // distances 2, 1), so that a store writes 64 contiguous bytes (half a
    // head row) of each of 16 frames instead of 16 bytes of each of 64 ----
    // hardware reciprocal (1 ulp); den >= 1, as the largest weight is exactly 1
    const float inv = __builtin_amdgcn_rcpf(den);
    uint32_t ov[8][4];  // ov[c]: channels 8c .. 8c+7, bf16 pairs
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[c][e] = pack_bf16x2(acc[8 * c + 2 * e] * inv, acc[8 * c + 2 * e + 1] * inv);
    const int lb = lt & 3;
    // One butterfly stage over lane distance j within each quad: the lower
    // lane takes the partner's chunk c0 into slot c0+j, the upper lane the
    // partner's chunk c0+j into slot c0 (ds_swizzle reads the partner).
    // The 16 exchanges of a stage are issued back to back (all sends first,
    // a scheduling barrier, all swizzles), so their latencies overlap.
    auto stage = [&](auto dist) {
        constexpr int j = decltype(dist)::value;
        constexpr int pattern = 0x1f | (j << 10);  // ds_swizzle bit mode: lane ^ j
        const bool upper = (lb & j) != 0;
        uint32_t x[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const int c0 = ((n >> 2) / j) * 2 * j + (n >> 2) % j, e = n & 3;  // the 4 slots c0 with c0 & j == 0
            x[n] = upper ? ov[c0][e] : ov[c0 + j][e];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < 16; ++n) x[n] = (uint32_t)__builtin_amdgcn_ds_swizzle((int)x[n], pattern);
        lds_wait(0);  // one wait for the 16 exchanges, not one per use
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const int c0 = ((n >> 2) / j) * 2 * j + (n >> 2) % j, e = n & 3;
            ov[c0][e] = upper ? x[n] : ov[c0][e];          // value selects: every index stays static
            ov[c0 + j][e] = upper ? ov[c0 + j][e] : x[n];
        }
    };
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 1>{});
    // lane 4a+b now holds chunks b and b+4 of frames 4a .. 4a+3 (slot k:
    // frame 4a + k%4, chunk b + 4*(k/4))
    const int tg = it.t0 + (lt & ~3);
    if (tg + 3 < tend) {
        // every frame of the quad is a query (all but the queries' last
        // quad): 8 stores from one address, no branch per store
        uint16_t* ob = o + (int64_t)(tg - g.f0) * rs + col + lb * 8;
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            uint16_t* p = ob + (int64_t)kq * rs;
            *reinterpret_cast<u32x4_t*>(p) = u32x4_t{ov[kq][0], ov[kq][1], ov[kq][2], ov[kq][3]};
            *reinterpret_cast<u32x4_t*>(p + 32) = u32x4_t{ov[kq + 4][0], ov[kq + 4][1], ov[kq + 4][2], ov[kq + 4][3]};
        }
    } else {
#pragma unroll
        for (int kf = 0; kf < 8; ++kf) {
            const int tf = tg + (kf & 3);
            if (tf < tend)
                *reinterpret_cast<u32x4_t*>(o + (int64_t)(tf - g.f0) * rs + col + (lb + 4 * (kf >> 2)) * 8) =
                    u32x4_t{ov[kf][0], ov[kf][1], ov[kf][2], ov[kf][3]};
        }
    }
}

// The compute of an item at raised wave priority.  Each SIMD holds one wave
// of each half; when both have an instruction ready, the computing wave (the
// phase's critical path) issues first and the staging wave fills its gaps.
// Measured at F=1024, 64x40x320, one box, three alternating pairs of whole
// runs: chain attention 1.57-1.62 against 1.60-1.65 ms, distinct Q/K/V within
// 1%.  (A wave's priority is a hint to the CU's instruction arbiter; the
// stream's priority is untouched.)
template <int NL, int NG, int R, bool SHORT>
__device__ __forceinline__ void dda_compute_prio(const char* __restrict__ buf, uint16_t* __restrict__ o,
                                                 const DdaGeo& g, int64_t rs, int heads, DdaItem it, int lt,
                                                 uint32_t (&qv)[32]) {
    __builtin_amdgcn_s_setprio(1);
    dda_compute<NL, NG, R, SHORT>(buf, o, g, rs, heads, it, lt, qv);
    __builtin_amdgcn_s_setprio(0);
}

// One work item of a half workgroup (256 threads, lt = 0..255): stage it
// (STAGE) or compute it.  Items below g.nfull are one strip x 256 queries;
// the rest are remainder items of M strips (s0 .. s0+M-1) x the last
// nq - 256*nchunks queries, strip j in slice j of the buffer, threads
// 256/M*j .. 256/M*(j+1)-1 (waves 4/M*j ..) on it.
template <int NL, int NG, int M, bool B32, bool STAGE>
__device__ __forceinline__ void dda_item_run(char* __restrict__ buf, const uint16_t* __restrict__ q,
                                             const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                             uint16_t* __restrict__ o, const DdaGeo& g, int64_t rs, int heads,
                                             int idx, int lt, uint32_t (&qv)[32], DdaItem& cur) {
    // The stage works out the item's coordinates (integer divisions) and
    // the compute of the same item, a phase later, reuses them.
    if (M == 1 || idx < g.nfull) {
        if constexpr (STAGE) {
            // item idx of the strip-major list (a strip's frame chunks in a
            // row) or of the chunk-major one
            const int strip = g.chunk_major ? idx % g.nstrips : idx / g.nchunks;
            const int chunk = g.chunk_major ? idx / g.nstrips : idx % g.nchunks;
            cur = dda_item(strip, g.f0 + chunk * DDA_TQ, heads);
        }
        const DdaItem it = cur;
        // Whole q rows through LDS (QROWS): measured faster for the one-sided
        // key sets (local only 1.13 -> 1.04-1.07 ms, global only 0.90 -> 0.87-0.89
        // at F=1024, 64x40x320) but 3% slower for the full key set with
        // Q = K = V (the extra LDS traffic of the stage competes with the
        // compute half), and it makes the clip kernels (M > 1) spill.
        constexpr bool QROWS = M == 1 && (NL == 0 || NG == 0);
        if constexpr (STAGE && B32)
            dda_stage_b32<NL, NG, QROWS>(buf, q, k, v, g, rs, heads, it, lt, qv);
        else if constexpr (STAGE)
            dda_stage<NL, NG, DDA_TQ, 256, QROWS>(buf, q, k, v, g, rs, heads, it, lt, qv);
        else
            dda_compute_prio<NL, NG, DDA_TQ, false>(buf, o, g, rs, heads, it, lt, qv);
    } else {
        constexpr int R = DdaRemR<M>, NT = 256 / M;
        const int j = lt / NT, ls = lt % NT;
        if constexpr (STAGE) cur = dda_item((idx - g.nfull) * M + j, g.f0 + g.nchunks * DDA_TQ, heads);
        const DdaItem it = cur;
        if (it.strip >= g.nstrips) return;  // the last remainder item may hold fewer strips
        char* slice = buf + j * DdaSlice<R>::BYTES;
        if constexpr (STAGE)
            dda_stage<NL, NG, R, NT>(slice, q, k, v, g, rs, heads, it, ls, qv);
        else
            dda_compute_prio<NL, NG, R, true>(slice, o, g, rs, heads, it, ls, qv);
    }
}

// Persistent, two-phase pipelined kernel: workgroup w takes a contiguous
// range of the item list (G = gridDim.x workgroups share it evenly); its half
// g (threads 256g..256g+255) takes the items with odd (g = 1) or even (g = 0)
// position in that range.
// Phase p: half 0 stages its item p/2 (p even) or computes item (p-1)/2 (p
// odd); half 1 stages item (p-1)/2 (p odd) or computes item (p-2)/2 (p even,
// p >= 2).  Every thread runs every phase and barrier.
template <int NL, int NG, int M, bool B32>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
dda_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
         uint16_t* __restrict__ o, DdaGeo g) {
    __shared__ __attribute__((aligned(16))) char lds[2 * DDA_LDS_BYTES];
    const int heads = g.C / DDA_D;
    const int64_t rs = (int64_t)g.S * g.C;
    const int half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8), lt = threadIdx.x & 255;
    char* buf = lds + half * DDA_LDS_BYTES;
    const int G = gridDim.x, w = blockIdx.x;
    // Items b0 .. b0+mine-1 of the strip-major list: a contiguous range, so
    // the two halves stage neighbouring frame chunks of a strip in
    // neighbouring phases and the 15 frames their windows share come from L2.
    // With Q = K = V and the full key set (chunk_major) every row is read
    // three times within its own stage anyway, and items w, w + G, w + 2G,
    // ... of the chunk-major list measured faster: the workgroups then stage
    // neighbouring strips.  (The one-sided key sets are slower that way.)
    const int b0 = g.chunk_major ? w : (int)(((int64_t)g.nitems * w) / G);
    const int mine = g.chunk_major ? (w < g.nitems ? (g.nitems - w + G - 1) / G : 0)
                                   : (int)(((int64_t)g.nitems * (w + 1)) / G) - b0;  // items of this workgroup
    const int stride = g.chunk_major ? G : 1;
    const int jh = (mine - half + 1) / 2;                             // items of this half
    const int j0 = (mine + 1) / 2, j1 = mine / 2;
    const int phases = max(2 * j0, 2 * j1 + 1);
    uint32_t qv[32];
    DdaItem cur{0, 0, 0, 0};  // the half's current item, from its stage to its compute
    for (int p = 0; p < phases; ++p) {
        const int rel = p - half;                 // half 0: rel = p, half 1: rel = p - 1
        if (rel >= 0) {
            const int j = rel >> 1;
            if (j < jh) {
                const int idx = b0 + (2 * j + half) * stride;
                if ((rel & 1) == 0)
                    dda_item_run<NL, NG, M, B32, true>(buf, q, k, v, o, g, rs, heads, idx, lt, qv, cur);
                else
                    dda_item_run<NL, NG, M, B32, false>(buf, q, k, v, o, g, rs, heads, idx, lt, qv, cur);
            }
        }
        __syncthreads();
    }
}

// ---- Q/K/V projection fused with the attention ----
//
// The query token comes from frame t, and the keys and values are computed
// from the tokens of its frame set (dual-domain attention paragraph): here
// q, k and v are three C x C linear maps of the input tokens (the reading of
// vinf_qkv_project), computed inside the attention's work item so they never
// reach HBM.  Per item (one location, one head, 256 query frames), one
// 256-thread workgroup:
//   1. projects the item's rows of x, the <= 271 frames its local windows
//      cover and the 16 global frames, onto the head's 64 q, 64 k and 64 v
//      channels: a 288 x 192 x C product on v_mfma_f32_16x16x32_bf16, the
//      weight fragment as the A operand and the accumulators started from the
//      bias, with the same K order as vinf_qkv_project's kernel, so every
//      value rounds to the same bf16;
//   2. writes the results straight into the attention's LDS layout: K rows,
//      V frame pairs, the global rows, and the q rows in the freed staging
//      area;
//   3. runs the attention's compute on them (dda_compute).
// x and weight slices (32 channels) are staged through registers, their
// loads issued two slices ahead, double buffered in LDS with one barrier per
// slice; 4 waves, each 9 row tiles x 6 column tiles (216 accumulators).
constexpr int PJ_ROWS = 288;                            // 18 row tiles: <= 271 local + 16 global
constexpr int PJ_COLS = 3 * DDA_D;                      // 12 column tiles: q, k, v of the head
constexpr int PJ_XS = PJ_ROWS * 64;                     // one 32-channel slice of the rows
constexpr int PJ_WS = PJ_COLS * 64;                     // one 32-channel slice of the weight rows
constexpr int PJ_STAGE = PJ_XS + PJ_WS;
constexpr int PJ_LDS = DDA_LDS_BYTES + 2 * PJ_STAGE;    // the attention slice, then two stages (or the q rows)
static_assert(DDA_TQ * 128 <= 2 * PJ_STAGE, "the q rows fit in the staging area");
static_assert(PJ_LDS <= 160 * 1024, "LDS of one CU");
static_assert(DdaFull::KROWS + DDA_G <= PJ_ROWS, "the projected rows");
constexpr int PJ_XT = (PJ_ROWS * 4 + 255) / 256;        // x chunks per thread and slice
constexpr int PJ_WT = PJ_COLS * 4 / 256;                // weight chunks per thread and slice

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
dda_proj_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias,
              uint16_t* __restrict__ o, DdaGeo g) {
    __shared__ __attribute__((aligned(16))) char lds[PJ_LDS];
    using SL = DdaFull;
    const int heads = g.C / DDA_D;
    const int64_t rs = (int64_t)g.S * g.C;
    const int lt = threadIdx.x, lane = lt & 63;
    const int wv = __builtin_amdgcn_readfirstlane(lt >> 6);
    const int wm = wv & 1, wn = wv >> 1;            // row tiles 9wm .. 9wm+8, column tiles 6wn .. 6wn+5
    // Persistent: workgroup b runs on XCD b % 8 (the dispatcher deals them
    // round-robin), and the eight XCDs take contiguous eighths of the item
    // list, so the items running at once on an XCD are neighbours: the heads
    // of one location, which read the same rows of x, share that XCD's L2.
    const int G = gridDim.x, b = blockIdx.x;
    const int per_xcd = (g.nitems + 7) / 8;
    auto item_of = [&](int k) -> int {
        if (G & 7) {
            const int i = b + k * G;
            return i < g.nitems ? i : -1;
        }
        const int kk = (b >> 3) + k * (G >> 3);
        const int i = (b & 7) * per_xcd + kk;
        return kk < per_xcd && i < g.nitems ? i : -1;
    };
    // x and the weight as buffers: byte offsets are 32-bit (the launcher
    // rejects an x of 4 GiB or more)
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), (short)0, (int)0xffffffffu, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(w), (short)0, (int)0xffffffffu, 0x00020000);
    for (int k = 0;; ++k) {
        const int idx = item_of(k);
        if (idx < 0) break;
        const DdaItem it = dda_item(idx % g.nstrips, (idx / g.nstrips) * DDA_TQ, heads);
        const int s = it.s, h = it.h;
        const int F = g.F;
        const int lo = dda_start(it.t0, F);
        const int tlast = min(it.t0 + DDA_TQ, F) - 1;
        const int nkr = dda_start(tlast, F) + DDA_L - lo;  // local rows: frames lo .. lo+nkr-1
        const int plo = lo & ~1;
        char* const stage = lds + DDA_LDS_BYTES;
        // frame of projected row r: a local frame, a global frame, or none (-1)
        auto frame_of = [&](int r) -> int {
            if (r < nkr) return lo + r;
            if (r < nkr + DDA_G) return (int)(((int64_t)(r - nkr) * F) / DDA_G);
            return -1;
        };

        // The V pair rows are filled half by half below; a half with no projected
        // frame (before lo, past the last) carries weight 0 and must read as 0.
        for (int i = lt; i < (DDA_G / 2) * 256 / 16; i += 256)
            *reinterpret_cast<u32x4_t*>(lds + SL::VG + i * 16) = u32x4_t{0u, 0u, 0u, 0u};
        for (int i = lt; i < SL::VPAIRS * DDA_VSTR / 16; i += 256)
            *reinterpret_cast<u32x4_t*>(lds + SL::VP + i * 16) = u32x4_t{0u, 0u, 0u, 0u};

        // accumulators: row tile 9wm + mi, column tile 6wn + ni; lane l holds
        // columns 4 (l / 16) .. +3 of the tile's row l % 16, started from the bias
        const int lr = lane & 15, lc = lane >> 4;
        f32x4_t acc[9][6];
#pragma unroll
        for (int ni = 0; ni < 6; ++ni) {
            const int c0 = (6 * wn + ni) * 16 + 4 * lc, p = c0 / DDA_D;
            f32x4_t b = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (bias) {
                const float* bp = bias + p * g.C + h * DDA_D + (c0 % DDA_D);
                b = f32x4_t{bp[0], bp[1], bp[2], bp[3]};
            }
#pragma unroll
            for (int mi = 0; mi < 9; ++mi) acc[mi][ni] = b;
        }
        // Staging of slice kc: thread task i -> row i / 4, 16-byte chunk i % 4, at
        // LDS slot chunk ^ ((row >> 1) & 3) of the row's 64 bytes, so that the
        // fragment reads (16 rows, one chunk per lane group) are conflict-free.
        // Each thread's chunk offsets are formed once per item; a slice is the
        // buffer loads' scalar offset.  Every lane loads (rows without a frame
        // read frame 0, and their value is dropped when written), so the loads
        // are straight-line code and each wait before the writes counts only
        // the older register stage's loads.
        uint32_t xo[PJ_XT], wo[PJ_WT], xin = 0;
#pragma unroll
        for (int j = 0; j < PJ_XT; ++j) {
            const int task = lt + 256 * j;
            const int f = frame_of(task >> 2);
            const bool ok = f >= 0 && f < F;
            xo[j] = (uint32_t)((((int64_t)(ok ? f : 0) * g.S + s) * g.C + (task & 3) * 8) * 2);
            xin |= (ok ? 1u : 0u) << j;
        }
#pragma unroll
        for (int j = 0; j < PJ_WT; ++j) {
            const int task = lt + 256 * j;
            const int n = task >> 2, p = n / DDA_D;   // column n: output p (q, k, v), channel n % 64 of the head
            wo[j] = (uint32_t)((((int64_t)p * g.C + h * DDA_D + (n % DDA_D)) * g.C + (task & 3) * 8) * 2);
        }
        auto load = [&](int kc, u32x4_t (&xr)[PJ_XT], u32x4_t (&wr)[PJ_WT]) {
#pragma unroll
            for (int j = 0; j < PJ_XT; ++j) xr[j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)xo[j], kc * 64, 0);
#pragma unroll
            for (int j = 0; j < PJ_WT; ++j) wr[j] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)wo[j], kc * 64, 0);
        };
        auto put = [&](int b, const u32x4_t (&xr)[PJ_XT], const u32x4_t (&wr)[PJ_WT]) {
            char* xs = stage + b * PJ_STAGE;
            char* ws = xs + PJ_XS;
#pragma unroll
            for (int j = 0; j < PJ_XT; ++j) {
                const int task = lt + 256 * j;
                if (task < PJ_ROWS * 4) {
                    const int r = task >> 2, c = task & 3;
                    const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4_t*>(xs + r * 64 + ((c ^ ((r >> 1) & 3)) << 4)) = (xin >> j) & 1u ? xr[j] : z;
                }
            }
#pragma unroll
            for (int j = 0; j < PJ_WT; ++j) {
                const int task = lt + 256 * j;
                const int r = task >> 2, c = task & 3;
                *reinterpret_cast<u32x4_t*>(ws + r * 64 + ((c ^ ((r >> 1) & 3)) << 4)) = wr[j];
            }
        };
        const int rd_off = lr * 64 + ((lc ^ ((lr >> 1) & 3)) << 4);
        const int nk = g.C / 32;  // even (C % 64 == 0)
        // Two register stages: slice kc: issue slice kc+2's loads (into stage kc &
        // 1, free since slice kc went to LDS; the last two slices reload slice
        // nk-1, unused, so there is no branch around the loads), multiply from LDS
        // buffer kc & 1, write slice kc+1 (loaded a slice ago) to the other
        // buffer, barrier.
        u32x4_t xr[2][PJ_XT], wr[2][PJ_WT];
        auto step = [&](int kc, auto par) {
            constexpr int P = decltype(par)::value;
            load(min(kc + 2, nk - 1), xr[P], wr[P]);
            const char* xs = stage + P * PJ_STAGE;
            const char* ws = xs + PJ_XS;
            bf16x8_t xf[9], wf[6];
#pragma unroll
            for (int mi = 0; mi < 9; ++mi) xf[mi] = *reinterpret_cast<const bf16x8_t*>(xs + (9 * wm + mi) * 16 * 64 + rd_off);
#pragma unroll
            for (int ni = 0; ni < 6; ++ni) wf[ni] = *reinterpret_cast<const bf16x8_t*>(ws + (6 * wn + ni) * 16 * 64 + rd_off);
#pragma unroll
            for (int ni = 0; ni < 6; ++ni)
#pragma unroll
                for (int mi = 0; mi < 9; ++mi)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[ni], xf[mi], acc[mi][ni], 0, 0, 0);
            if (kc + 1 < nk) put(1 - P, xr[1 - P], wr[1 - P]);
            __syncthreads();
        };
        load(0, xr[0], wr[0]);
        load(min(1, nk - 1), xr[1], wr[1]);
        put(0, xr[0], wr[0]);
        __syncthreads();
        for (int kc = 0; kc < nk; kc += 2) {
            step(kc, std::integral_constant<int, 0>{});
            step(kc + 1, std::integral_constant<int, 1>{});
        }

        // Results into the attention's layout (the staging area is free now: the
        // loop ended with a barrier, which also ordered the zero fill above).
        // Frames outside the video become zeros, as the unfused attention reads
        // them.
        char* const qrows = stage;
#pragma unroll
        for (int mi = 0; mi < 9; ++mi) {
            const int r = (9 * wm + mi) * 16 + lr;
            const int f = frame_of(r);
            const bool in = f >= 0 && f < F;
#pragma unroll
            for (int ni = 0; ni < 6; ++ni) {
                const int c0 = (6 * wn + ni) * 16 + 4 * lc, p = c0 / DDA_D, j0 = c0 % DDA_D;
                const f32x4_t a = acc[mi][ni];
                const uint32_t u0 = in ? pack_bf16x2(a[0], a[1]) : 0u, u1 = in ? pack_bf16x2(a[2], a[3]) : 0u;
                if (r < nkr) {
                    if (p == 0) {
                        if (in && f >= it.t0 && f < it.t0 + DDA_TQ)
                            *reinterpret_cast<uint2*>(qrows + (f - it.t0) * 128 + j0 * 2) = uint2{u0, u1};
                    } else if (p == 1) {
                        *reinterpret_cast<uint2*>(lds + SL::KL + r * DDA_KSTR + j0 * 2) = uint2{u0, u1};
                    } else {
                        char* vp = lds + SL::VP + ((f - plo) >> 1) * DDA_VSTR + j0 * 4 + ((f - plo) & 1) * 2;
                        *reinterpret_cast<uint16_t*>(vp) = (uint16_t)u0;
                        *reinterpret_cast<uint16_t*>(vp + 4) = (uint16_t)(u0 >> 16);
                        *reinterpret_cast<uint16_t*>(vp + 8) = (uint16_t)u1;
                        *reinterpret_cast<uint16_t*>(vp + 12) = (uint16_t)(u1 >> 16);
                    }
                } else if (r < nkr + DDA_G) {
                    const int i = r - nkr;
                    if (p == 1) {
                        *reinterpret_cast<uint2*>(lds + SL::KG + i * 128 + j0 * 2) = uint2{u0, u1};
                    } else if (p == 2) {
                        char* vp = lds + SL::VG + (i >> 1) * 256 + j0 * 4 + (i & 1) * 2;
                        *reinterpret_cast<uint16_t*>(vp) = (uint16_t)u0;
                        *reinterpret_cast<uint16_t*>(vp + 4) = (uint16_t)(u0 >> 16);
                        *reinterpret_cast<uint16_t*>(vp + 8) = (uint16_t)u1;
                        *reinterpret_cast<uint16_t*>(vp + 12) = (uint16_t)(u1 >> 16);
                    }
                }
            }
        }
        __syncthreads();
        uint32_t qv[32];
        if (it.t0 + lt < F) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const u32x4_t u = *reinterpret_cast<const u32x4_t*>(qrows + lt * 128 + c * 16);
                qv[4 * c] = u[0];
                qv[4 * c + 1] = u[1];
                qv[4 * c + 2] = u[2];
                qv[4 * c + 3] = u[3];
            }
        } else {
#pragma unroll
            for (int c = 0; c < 32; ++c) qv[c] = 0u;  // a lane past the last query computes a throw-away copy
        }
        dda_compute<DDA_L, DDA_G, DDA_TQ>(lds, o, g, rs, heads, it, lt, qv);
        __syncthreads();  // the next item's zero fill and staging overwrite this item's LDS
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

vinf_status launch_dda_projected(const void* x, const void* w, const float* bias, void* o, int F, int S, int C,
                                 float scale, hipStream_t st) {
    const int heads = C / DDA_D;
    DdaGeo g;
    g.kg = g.vg = nullptr;
    g.F = F;
    g.f0 = 0;
    g.nq = F;
    g.kf0 = 0;
    g.kend = F;
    g.S = S;
    g.C = C;
    g.sl2e = scale * 1.4426950408889634f;
    const int64_t nstrips = (int64_t)S * heads, nchunks = (F + DDA_TQ - 1) / DDA_TQ;
    if (nstrips * nchunks > 0x7fffffff)
        return fail(VINF_ERR_UNSUPPORTED, "projected_dual_domain_attn: more than 2^31 work items");
    g.nstrips = (int)nstrips;
    g.nchunks = (int)nchunks;
    g.nfull = g.nitems = (int)(nstrips * nchunks);
    g.chunk_major = 0;
    if ((uint64_t)F * S * C * 2 > 0xffffffffull)
        return fail(VINF_ERR_UNSUPPORTED, "projected_dual_domain_attn: x of 4 GiB or more (32-bit buffer offsets)");
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return fail(VINF_ERR_HIP, "projected_dual_domain_attn: cannot query the device");
    // one persistent workgroup per CU, a multiple of 8 of them when there are
    // enough items (the kernel's XCD-contiguous item order needs it)
    int grid = (int)std::min<int64_t>(cus, g.nitems);
    if (grid >= 8) grid &= ~7;
    hipLaunchKernelGGL(dda_proj_bf16, dim3((uint32_t)grid), dim3(256), 0, st, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(w), bias, static_cast<uint16_t*>(o), g);
    return check_launch("projected_dual_domain_attn");
}

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
    g.chunk_major = q == k && k == v && n_local > 0 && n_global > 0;
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
        // whole-strip stages with 32-bit buffer offsets unless a frame is too large
        const bool b32 = (int64_t)S * C <= DDA_B32_MAX_RS;
        auto run2 = [&](auto nl, auto ng, auto b) {
            constexpr int NL = decltype(nl)::value, NG = decltype(ng)::value;
            constexpr bool B = decltype(b)::value;
            if (M == 4)
                hipLaunchKernelGGL((dda_bf16<NL, NG, 4, B>), grid, block, 0, st, qb, kb, vb, ob, g);
            else if (M == 2)
                hipLaunchKernelGGL((dda_bf16<NL, NG, 2, B>), grid, block, 0, st, qb, kb, vb, ob, g);
            else
                hipLaunchKernelGGL((dda_bf16<NL, NG, 1, B>), grid, block, 0, st, qb, kb, vb, ob, g);
        };
        auto run = [&](auto nl, auto ng) {
            if (b32)
                run2(nl, ng, std::true_type{});
            else
                run2(nl, ng, std::false_type{});
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

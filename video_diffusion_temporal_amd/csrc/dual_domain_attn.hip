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
// bf16 kernel (dda_bf16).  A strip is one (location, head) column of 64
// channels; four consecutive strips are 512 contiguous bytes of every frame.
// A persistent 512-thread workgroup per CU walks units = (4 strips, a run of
// query frames) in chunks of 32 query frames.  Both contractions run on MFMA:
//   * Scores, transposed: S^T = K * Q^T on v_mfma_f32_16x16x32_bf16, one wave
//     per (strip, 16 queries).  The 16 queries t0..t0+15 need local keys from
//     one 32-frame window starting at b0 = (window start of t0) rounded down
//     to 8, so two 16-key tiles plus the 16-key global tile cover them; keys
//     outside a query's own window are masked.  In the result a lane holds 4
//     keys of one query, so the softmax needs two cross-lane steps only.
//   * Weighted sum, transposed: O^T = V^T * P^T.  The lane's own softmax
//     weights are already the B operand (the two local tiles are one K = 32
//     step with the keys in a lane-matched order; the global tile is a
//     16x16x16 step), and V^T comes from a transposed copy of V in LDS.  The
//     normaliser is the sum of the bf16-rounded weights, so the output is a
//     convex combination of V rows up to fp32 rounding; bf16 output.
//   * Staging: K rows go to an LDS ring (128 frames x 4 strips, 16-byte
//     chunks XOR-swizzled by frame), V to a transposed ring [strip][dim][frame]
//     (rows padded to 272 B).  Every step stages 32 new frames; loads are
//     issued two steps ahead into registers and written to LDS one step
//     ahead, q rows one step ahead straight into MFMA operand registers, and
//     the 16 global K/V rows of a unit into registers when the unit opens
//     (a staging-only step).  Nothing waits on a load issued in the same
//     step, so HBM sees a steady stream of 512-byte frame rows.
// fp32 kernel (dda_f32): one query per thread, fp32 FMA, keys read through
// the cache; used for float32 I/O.
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "common.h"

namespace vinf {

constexpr int DDA_D = 64;                 // head dim
constexpr int DDA_L = 16;                 // local keys
constexpr int DDA_G = 16;                 // global keys
constexpr int DDA_CQ = 32;                // query frames per chunk (and frames staged per step)
constexpr int DDA_NS = 4;                 // strips per workgroup
constexpr int DDA_RING = 128;             // frames held per strip: 4 steps of 32
constexpr int DDA_KSTRIP = DDA_RING * 128;                 // K ring bytes per strip
constexpr int DDA_VPITCH = 2 * DDA_RING + 16;              // transposed V row (one dim), padded
constexpr int DDA_VSTRIP = DDA_D * DDA_VPITCH;             // V ring bytes per strip
constexpr int DDA_VOFF = DDA_NS * DDA_KSTRIP;              // V ring offset
constexpr int DDA_LDS = DDA_VOFF + DDA_NS * DDA_VSTRIP;    // 135168 B
static_assert(DDA_LDS <= 160 * 1024, "LDS budget");

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct DdaGeo {
    int F;        // frames
    int nstrips;  // locations * heads
    int nseg;     // query runs per strip group
    int ts;       // query frames per run (multiple of 32)
    int nunits;   // strip groups * nseg
    int nl;       // local keys present: min(F, 16)
    int stmax;    // largest window start: max(F - 16, 0)
    int64_t rs;   // elements per frame (H*W*C)
    float sl2e;   // scale * log2(e)
};

__device__ __forceinline__ int dda_st(int t, int stmax) {
    const int s = t - DDA_L / 2;
    return s < 0 ? 0 : (s > stmax ? stmax : s);
}

// (v[f][d], v[f+1][d]) from dwords a = (v[f][d], v[f][d+1]), b = (v[f+1][d], v[f+1][d+1]); _hi gives d+1.
__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Position in this workgroup's sequence of steps.  Each unit opens with a
// staging-only step (c = -1) and then has one step per 32-query chunk.
struct DdaCursor {
    int unit;  // global unit id; >= nunits once the sequence has ended
    int c;     // chunk within the unit, -1 for the opening step
    __device__ __forceinline__ bool live(const DdaGeo& g) const { return unit < g.nunits; }
    __device__ __forceinline__ int fa(const DdaGeo& g) const { return (unit % g.nseg) * g.ts; }
    __device__ __forceinline__ int group(const DdaGeo& g) const { return unit / g.nseg; }
    __device__ __forceinline__ void next(const DdaGeo& g) {
        const int nc = (min(g.ts, g.F - fa(g)) + DDA_CQ - 1) / DDA_CQ;
        if (++c == nc) {
            unit += gridDim.x;
            c = -1;
        }
    }
};

// Frames a step stages: the opening step of a unit starting at query frame fa
// takes [fa-16, fa+16), chunk c takes [fa+32c+16, fa+32c+48).  Step number n
// of the workgroup puts them at ring slots 32n mod 128 onwards.
__device__ __forceinline__ int dda_stage_first(const DdaGeo& g, const DdaCursor& cs) {
    return cs.fa(g) + (cs.c < 0 ? -16 : DDA_CQ * cs.c + 16);
}

// Issue the K or V loads of one step.  Waves 0-3 load V of strip `wave`
// (lane: 4 frames x 8 dims); waves 4-7 load K (lane: 4 frames x 8 dims of
// strip (lane>>3)&3).  Every lane loads from a clamped, valid address (no
// divergent branches around loads); bit j of the result says whether load j
// was a real frame of a real strip, the others are zeroed on commit.
__device__ __forceinline__ int dda_stage_issue(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                               const DdaGeo& g, const DdaCursor& cs, int wave, int lane,
                                               u32x4_t (&r)[4]) {
    const int fs = dda_stage_first(g, cs);
    const int grp = cs.group(g);
    const bool vw = wave < 4;
    const int strip = grp * DDA_NS + (vw ? wave : ((lane >> 3) & 3));
    const int f0 = vw ? fs + 4 * (lane & 7) : fs + 2 * (wave - 4) + (lane >> 5);
    const int fstep = vw ? 1 : 8;
    const uint16_t* base = (vw ? v : k) + (int64_t)min(strip, g.nstrips - 1) * DDA_D + 8 * (vw ? lane >> 3 : lane & 7);
    int okm = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int f = f0 + fstep * j;
        const bool ok = strip < g.nstrips && f >= 0 && f < g.F;
        r[j] = ld16(base + (int64_t)min(max(f, 0), g.F - 1) * g.rs);
        okm |= (int)ok << j;
    }
    return okm;
}

// Write a step's staged registers into the rings (step number n).
__device__ __forceinline__ void dda_stage_commit(char* __restrict__ lds, int n, int wave, int lane,
                                                 const u32x4_t (&rin)[4], int okm) {
    const int slot0 = (DDA_CQ * n) & (DDA_RING - 1);
    u32x4_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = ((okm >> j) & 1) ? rin[j] : u32x4_t{0u, 0u, 0u, 0u};
    if (wave < 4) {
        // lane: frames slot0 + 4*(lane&7) .. +3, dims 8*(lane>>3) .. +7
        char* dst = lds + DDA_VOFF + wave * DDA_VSTRIP + 8 * (lane >> 3) * DDA_VPITCH + 2 * (slot0 + 4 * (lane & 7));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u32x2_t lo = {perm_lo(r[0][e], r[1][e]), perm_lo(r[2][e], r[3][e])};
            u32x2_t hi = {perm_hi(r[0][e], r[1][e]), perm_hi(r[2][e], r[3][e])};
            *reinterpret_cast<u32x2_t*>(dst + (2 * e) * DDA_VPITCH) = lo;
            *reinterpret_cast<u32x2_t*>(dst + (2 * e + 1) * DDA_VPITCH) = hi;
        }
    } else {
        const int s = (lane >> 3) & 3, cc = lane & 7;
        char* base = lds + s * DDA_KSTRIP;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int slot = slot0 + 2 * (wave - 4) + (lane >> 5) + 8 * j;
            *reinterpret_cast<u32x4_t*>(base + slot * 128 + ((cc ^ ((slot >> 1) & 7)) << 4)) = r[j];
        }
    }
}

// q rows of the wave's 16 queries as the B operand of the score MFMAs:
// lane (q = lane&15, g = lane>>4) holds dims 8g..8g+7 and 32+8g..32+8g+7.
// Loaded for every step (clamped to a valid row) so the code stays
// branch-free; a step without a chunk never reads them.
__device__ __forceinline__ void dda_q_issue(const uint16_t* __restrict__ q, const DdaGeo& g, const DdaCursor& cs,
                                            int wave, int lane, u32x4_t (&qf)[2]) {
    const int strip = min(cs.group(g) * DDA_NS + (wave & 3), g.nstrips - 1);
    const int t0 = cs.fa(g) + DDA_CQ * max(cs.c, 0) + 16 * (wave >> 2);
    const int tq = min(t0 + (lane & 15), g.F - 1);
    const uint16_t* p = q + (int64_t)tq * g.rs + (int64_t)strip * DDA_D + 8 * (lane >> 4);
    qf[0] = ld16(p);
    qf[1] = ld16(p + 32);
}

// Global rows of the wave's strip: K as the A operand of the global score tile
// (lane: key lane&15, dims 8g.. and 32+8g..), V^T as the A operand of the
// 16x16x16 weighted-sum step (lane: dim 16n + (lane&15), keys 4g..4g+3).
__device__ __forceinline__ void dda_glob_issue(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                               const DdaGeo& g, const DdaCursor& cs, int wave, int lane,
                                               u32x4_t (&kg)[2], uint32_t (&vraw)[16]) {
    const int strip = min(cs.group(g) * DDA_NS + (wave & 3), g.nstrips - 1);
    const int r = lane & 15, gq = lane >> 4;
    const int64_t col = (int64_t)strip * DDA_D;
    const int64_t gf = ((int64_t)r * g.F) / DDA_G;
    const uint16_t* p = k + gf * g.rs + col + 8 * gq;
    kg[0] = *reinterpret_cast<const u32x4_t*>(p);
    kg[1] = *reinterpret_cast<const u32x4_t*>(p + 32);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t f = ((int64_t)(4 * gq + j) * g.F) / DDA_G;
            vraw[4 * n + j] = v[f * g.rs + col + 16 * n + r];  // packed when the unit opens
        }
    }
}

__device__ __forceinline__ f32x4_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                     c, 0, 0, 0);
}

// One wave's 16 queries of chunk cs (workgroup step number z).
__device__ __forceinline__ void dda_chunk(const char* __restrict__ lds, uint16_t* __restrict__ o, const DdaGeo& g,
                                          const DdaCursor& cs, int z, int wave, int lane, const u32x4_t (&qf)[2],
                                          const u32x4_t (&kg)[2], const u32x2_t (&vg)[4]) {
    const int si = wave & 3;
    const int strip = cs.group(g) * DDA_NS + si;
    const int fa = cs.fa(g);
    const int t0 = fa + DDA_CQ * cs.c + 16 * (wave >> 2);
    if (strip >= g.nstrips || t0 >= g.F) return;
    const int r = lane & 15, gq = lane >> 4;
    // ring slot of frame f: (f + k0) mod 128 (steps z-1 and z hold frames fa+32c-16 .. fa+32c+47)
    const int k0 = DDA_CQ * z - 16 - fa - DDA_CQ * cs.c;
    const int b0 = dda_st(t0, g.stmax) & ~7;

    // scores S^T: lane holds keys 4gq+i of query r (tile 0: b0.., tile 1: b0+16.., tile 2: global)
    const char* kb = lds + si * DDA_KSTRIP;
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, sg = s0;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        const int slot = (b0 + 16 * kt + r + k0) & (DDA_RING - 1);
        const int sw = (slot >> 1) & 7;
        const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(kb + slot * 128 + ((gq ^ sw) << 4));
        const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(kb + slot * 128 + (((gq + 4) ^ sw) << 4));
        f32x4_t& acc = kt ? s1 : s0;
        acc = mfma32(a0, qf[0], acc);
        acc = mfma32(a1, qf[1], acc);
    }
    sg = mfma32(kg[0], qf[0], sg);
    sg = mfma32(kg[1], qf[1], sg);

    // softmax over the query's 16 local keys (window start st) and 16 global keys
    const int tq = min(t0 + r, g.F - 1);
    const int rel = b0 - dda_st(tq, g.stmax);  // key j of tile kt is window position rel + 16kt + 4gq + i
    bool ok0[4], ok1[4];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ok0[i] = (unsigned)(rel + 4 * gq + i) < (unsigned)g.nl;
        ok1[i] = (unsigned)(rel + 16 + 4 * gq + i) < (unsigned)g.nl;
        m = fmaxf(m, ok0[i] ? s0[i] : -INFINITY);
        m = fmaxf(m, ok1[i] ? s1[i] : -INFINITY);
        m = fmaxf(m, sg[i]);
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const float msl = m * g.sl2e;
    float p0[4], p1[4], pg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0[i] = ok0[i] ? __builtin_amdgcn_exp2f(fmaf(s0[i], g.sl2e, -msl)) : 0.f;
        p1[i] = ok1[i] ? __builtin_amdgcn_exp2f(fmaf(s1[i], g.sl2e, -msl)) : 0.f;
        pg[i] = __builtin_amdgcn_exp2f(fmaf(sg[i], g.sl2e, -msl));
    }
    const u32x4_t pl = {pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]), pack_bf16x2(p1[0], p1[1]),
                        pack_bf16x2(p1[2], p1[3])};
    const u32x2_t pgl = {pack_bf16x2(pg[0], pg[1]), pack_bf16x2(pg[2], pg[3])};
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) den += bf_lo(pl[i]) + bf_hi(pl[i]);
    den += bf_lo(pgl[0]) + bf_hi(pgl[0]) + bf_lo(pgl[1]) + bf_hi(pgl[1]);
    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);
    const float inv = 1.f / den;

    // O^T = V^T P^T: lane holds dims 16n + 4gq + i of query r
    const char* vb = lds + DDA_VOFF + si * DDA_VSTRIP + r * DDA_VPITCH;
    const int sa = 2 * ((b0 + 4 * gq + k0) & (DDA_RING - 1));
    const int sb = 2 * ((b0 + 16 + 4 * gq + k0) & (DDA_RING - 1));
    // Lanes past the last frame computed query F-1 (tq is clamped) and store
    // the same values as the lane that owns it.
    uint16_t* orow = o + (int64_t)tq * g.rs + (int64_t)strip * DDA_D + 4 * gq;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const char* vrow = vb + 16 * n * DDA_VPITCH;
        const u32x2_t x = *reinterpret_cast<const u32x2_t*>(vrow + sa);
        const u32x2_t y = *reinterpret_cast<const u32x2_t*>(vrow + sb);
        const u32x4_t a = {x[0], x[1], y[0], y[1]};
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma32(a, pl, acc);
        acc = mfma16(vg[n], pgl, acc);
        const u32x2_t w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + 16 * n) = w;
    }
}

// One step of the pipeline (step number z, register set P = z & 1):
// issue the loads of step z+2 and the q rows of step z+1, write step z+1's
// staged rows into the rings, compute step z, barrier.
template <int P>
__device__ __forceinline__ void dda_step(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ v, uint16_t* __restrict__ o, char* lds,
                                         const DdaGeo& g, int z, const DdaCursor& c0, const DdaCursor& c1,
                                         const DdaCursor& c2, int wave, int lane, u32x4_t (&stg)[2][4],
                                         int (&okm)[2], u32x4_t (&qf)[2][2], u32x4_t (&kg)[2], u32x2_t (&vg)[4],
                                         u32x4_t (&kgn)[2], uint32_t (&vgn)[16]) {
    if (c0.c < 0) {  // a unit opens: its global rows become current
        kg[0] = kgn[0];
        kg[1] = kgn[1];
#pragma unroll
        for (int n = 0; n < 4; ++n) vg[n] = u32x2_t{vgn[4 * n] | (vgn[4 * n + 1] << 16), vgn[4 * n + 2] | (vgn[4 * n + 3] << 16)};
    }
    // Issued unconditionally (a finished sequence loads clamped rows it never
    // commits): a load into a register only on some paths would make the
    // compiler copy the register and wait for the load there.
    okm[P] = dda_stage_issue(k, v, g, c2, wave, lane, stg[P]);
    if (c2.live(g) && c2.c < 0) dda_glob_issue(k, v, g, c2, wave, lane, kgn, vgn);
    dda_q_issue(q, g, c1, wave, lane, qf[P ^ 1]);
    if (c1.live(g)) dda_stage_commit(lds, z + 1, wave, lane, stg[P ^ 1], okm[P ^ 1]);
    if (c0.c >= 0) dda_chunk(lds, o, g, c0, z, wave, lane, qf[P], kg, vg);
    __syncthreads();
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
dda_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
         uint16_t* __restrict__ o, DdaGeo g) {
    __shared__ __attribute__((aligned(16))) char lds[DDA_LDS];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // Masked keys still enter the MFMAs with weight 0, so every ring slot must
    // hold finite values from the start.
    for (int i = threadIdx.x; i < DDA_LDS / 16; i += blockDim.x)
        reinterpret_cast<u32x4_t*>(lds)[i] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();

    DdaCursor c0 = {(int)blockIdx.x, -1};
    if (!c0.live(g)) return;
    DdaCursor c1 = c0, c2;
    c1.next(g);
    c2 = c1;
    c2.next(g);

    u32x4_t stg[2][4], qf[2][2], kg[2], kgn[2];
    u32x2_t vg[4];
    uint32_t vgn[16];
    int okm[2] = {0, 0};
    // prologue: step 0 (a unit's opening step) staged and committed, step 1 issued
    okm[0] = dda_stage_issue(k, v, g, c0, wave, lane, stg[0]);
    dda_glob_issue(k, v, g, c0, wave, lane, kgn, vgn);
    okm[1] = dda_stage_issue(k, v, g, c1, wave, lane, stg[1]);
    dda_stage_commit(lds, 0, wave, lane, stg[0], okm[0]);
    __syncthreads();

    for (int z = 0;; z += 2) {
        dda_step<0>(q, k, v, o, lds, g, z, c0, c1, c2, wave, lane, stg, okm, qf, kg, vg, kgn, vgn);
        c0 = c1;
        c1 = c2;
        c2.next(g);
        if (!c0.live(g)) break;
        dda_step<1>(q, k, v, o, lds, g, z + 1, c0, c1, c2, wave, lane, stg, okm, qf, kg, vg, kgn, vgn);
        c0 = c1;
        c1 = c2;
        c2.next(g);
        if (!c0.live(g)) break;
    }
}

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
    const int st = dda_st(t, F - DDA_L > 0 ? F - DDA_L : 0);
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
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            return fail(VINF_ERR_HIP, "dual_domain_attn: cannot query the device");
        const int64_t nstrips = (int64_t)S * heads;
        const int64_t ngroups = (nstrips + DDA_NS - 1) / DDA_NS;
        const int64_t nchunks = (F + DDA_CQ - 1) / DDA_CQ;
        // Split each strip group's frames into runs so that the busiest CU
        // walks as few steps as possible (a run costs one extra opening step).
        int64_t best_cost = -1, best_run = nchunks;
        for (int64_t nseg = 1; nseg <= nchunks; nseg *= 2) {
            const int64_t run = (nchunks + nseg - 1) / nseg;
            const int64_t units = ngroups * ((nchunks + run - 1) / run);
            const int64_t cost = ((units + cus - 1) / cus) * (run + 1);
            if (best_cost < 0 || cost < best_cost) {
                best_cost = cost;
                best_run = run;
            }
        }
        const int64_t nseg = (nchunks + best_run - 1) / best_run;
        const int64_t nunits = ngroups * nseg;
        if (nstrips > INT_MAX || nunits > INT_MAX - 2 * (int64_t)cus)
            return fail(VINF_ERR_UNSUPPORTED, "dual_domain_attn: too many (location, head) strips");
        DdaGeo g;
        g.F = F;
        g.nstrips = (int)nstrips;
        g.nseg = (int)nseg;
        g.ts = (int)(best_run * DDA_CQ);
        g.nunits = (int)nunits;
        g.nl = std::min(F, DDA_L);
        g.stmax = std::max(F - DDA_L, 0);
        g.rs = (int64_t)S * C;
        g.sl2e = sl2e;
        const int grid = (int)std::min<int64_t>(cus, nunits);
        hipLaunchKernelGGL(dda_bf16, dim3((uint32_t)grid), dim3(512), 0, st, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                           g);
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

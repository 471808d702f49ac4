// Temporal convolution, kernel 3, with context padding, gfx950.
//
// Method (Video-Infinity write-up, Conv-module paragraph): a convolution along
// the frame axis of every spatial location; at a clip edge the sequence is
// padded with the neighbouring clip's edge frames, as many as the receptive
// field (one per side for kernel 3).  On one GPU the whole video is one clip,
// so the pads are ctx_pre / ctx_post when given and zeros otherwise.
//
//   y[f,s,co] = bias[co] + sum_k sum_ci W[k][co][ci] * xt[f+k-1, s, ci]
//
// The same kernel with one tap is the Q/K/V projection (dual-domain attention
// paragraph: the query token is frame t's, and keys and values are computed
// from the tokens of its frame set; read as three linear maps of each token):
//
//   q/k/v[f,s,co] = bias[p][co] + sum_ci W[p][co][ci] * x[f, s, ci],  p = 0, 1, 2
//
// bf16 kernel (conv3_bf16): an implicit GEMM with M = F*S output voxels,
// N = C_out, K = 3*C_in, on v_mfma_f32_16x16x32_bf16.
//   * A tile is 16 frames x 16 locations (256 rows of M) by BN = 16*NF*WN
//     output channels (all 320 with NF = 5, WN = 4).  For each 32-channel
//     slice of C_in, 18 frames x 16 locations of x (the 16 frames plus one
//     halo frame per side) and the three taps' weight rows are staged in LDS;
//     a tap is then a shift of the x operand by one frame (16 LDS rows), so
//     the three taps share one staged tile.
//   * Staging uses buffer_load_dwordx4 ... lds (HBM/L2 -> LDS without
//     VGPRs).  One wave instruction fills one frame's 16 locations; frames
//     outside the video come from ctx_pre / ctx_post or read as zeros
//     (num_records = 0), locations past S read as zeros (out of range).
//   * LDS rows are 64 bytes; 16-byte chunk c of row r sits at slot
//     c ^ ((r >> 1) & 3), which keeps fragment reads (16 consecutive rows,
//     one chunk per lane group) free of bank conflicts (measured with the
//     LDS bank-conflict counter) and makes each lane's slot a constant, so
//     all fragment reads use immediate offsets.
//   * 4 (M) x WN (N) waves; a wave owns 4 frames x 16*NF channels and reads
//     6 x fragments (4 frames + the two tap shifts) and 3*NF weight fragments
//     per slice, the weight fragments LA groups of 4 MFMAs ahead (pinned
//     with scheduling-group hints; the compiler otherwise reads them just
//     before use).  The weight fragment is the MFMA's A operand, so
//     each lane's accumulator holds 4 consecutive output channels of one
//     voxel, and starts from the bias of those channels.  The epilogue
//     rounds and swaps fragment pairs across lane groups
//     (v_permlane32_swap, v_permlane16_swap) so that a lane holds 8
//     consecutive channels and writes 16-byte pieces (64 contiguous bytes of
//     a voxel row per store instruction).
//   * Persistent: one 256*WN-thread workgroup per CU walks a contiguous range of
//     tiles (consecutive frame blocks of the same locations, so halo frames
//     are L2 hits); LDS is double-buffered across slices and tiles with one
//     barrier per slice, and the next slice's loads are in flight while the
//     current one is multiplied.
// Projection (TAPS = 1): the 16 tile frames are staged with no halo and no
// shift, N runs over the 3*C weight rows, and each tile writes to the output
// its channels belong to; KS = 2 slices share a barrier.
// fp32 kernels (conv3_f32, qkv_project_f32): one output element per thread, fp32 FMA.
//
// GroupNorm applied inside the conv (conv3_bf16<.., GN = true>, conv3_f32
// with gn tables): the GroupNorm output g = x*a_c + b_c (a_c = rstd_g*gamma_c,
// b_c = beta_c - mean_g*a_c, formed in fp32 exactly as the GroupNorm apply
// forms them) is what the conv multiplies, but it is never written to HBM.
// In the bf16 kernel each x slice lands in LDS raw (DMA); every wave then
// rewrites the frame blocks its own loads filled, in place, as
// fmaf(x, a_c, b_c) rounded to bf16, before the barrier that publishes the
// slice.  That rewrite is software-pipelined: slice g+1 is normalised while
// slice g's last MFMA groups run (its loads were issued right after slice
// g's barrier, and its buffer is not read before the next one), so the
// vector work fills the matrix pipe's shadow instead of a window where every
// wave waits.  A lane rewrites one 4-byte word (one channel pair) in four
// rows of a block, so it needs one (a, b) pair per block: the coefficients
// come as a table of channel pairs, and one wave stages a slice's 256 bytes
// into LDS two slices ahead.  The first NSTG - NW waves own a second block,
// which they rewrite after the MFMA groups.
// Zero pads stay zero (they are zeros of the normalised tensor); context
// frames are raw neighbouring frames and are normalised like the rest.  The
// result is bit for bit that of the GroupNorm apply followed by the conv.
#include <algorithm>

#include "common.h"

namespace vinf {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

constexpr int CV_TF = 16;                       // frames per tile
constexpr int CV_TP = 16;                       // locations per tile
constexpr int CV_BK = 32;                       // C_in slice

// LDS of one slice: the staged x frames (16 + TAPS - 1 of them: the tile's
// frames plus the halo the taps reach) and TAPS weight slices of BN rows.
// A stage (one barrier) holds KS consecutive slices; two stages alternate.
template <int NF, int WN, int TAPS, int KS>
struct ConvLds {
    static constexpr int BN = 16 * NF * WN;
    static constexpr int NSTG = CV_TF + TAPS - 1;
    static constexpr int A_BYTES = NSTG * CV_TP * 64;
    static constexpr int B_BYTES = TAPS * BN * 64;
    static constexpr int SLOT = A_BYTES + B_BYTES;
    static constexpr int BUF = KS * SLOT;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t cv_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// TAPS = 3: the temporal conv (tap k multiplies frame f+k-1, one output y).
// TAPS = 1: the Q/K/V projection, the same GEMM with no frame shift: N spans
// the 3*C rows of the [3][C][C] weight, and output channel n goes to
// y, y1 or y2 (Q, K, V) by n / C.  The tiles of one location block run at
// the same time on three workgroups of one XCD, so two of the three stagings
// of each x tile come from L2.  With one tap a slice holds a third of the conv's MFMAs, so
// KS = 2 slices share a barrier (more work in flight per load latency).
template <int NF, int WN, int TAPS, int KS, bool GN>
__global__ void __launch_bounds__(256 * WN) __attribute__((amdgpu_waves_per_eu(WN, WN)))
conv3_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ pre, const uint16_t* __restrict__ post,
           const uint16_t* __restrict__ w, const float* __restrict__ bias, const float* __restrict__ gn_ab,
           uint16_t* y, uint16_t* y1, uint16_t* y2, int F, int S, int C, int nfb,
           int nlb, int ntn) {
    static_assert(TAPS == 1 || TAPS == 3, "kernel 3 or a plain projection");
    static_assert(!GN || (TAPS == 3 && KS == 1), "GroupNorm inside only for the conv");
    using L = ConvLds<NF, WN, TAPS, KS>;
    constexpr int BN = L::BN;
    constexpr int NSTG = L::NSTG;               // staged frames
    constexpr int HALO = (TAPS - 1) / 2;        // frames before the tile
    constexpr int NA = TAPS + 3;                // x fragments per wave and slice
    constexpr int NW = 4 * WN;                  // waves: 4 along M x WN along N
    constexpr int B_INSTR = TAPS * BN / 16;     // wave instructions per weight slice (16 rows each)
    // GN: two 256-byte coefficient slots and a 16-byte zero slot follow the buffers.
    __shared__ __attribute__((aligned(1024))) char lds[2 * L::BUF + (GN ? 528 : 0)];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int wm = wv & 3, wn = wv >> 2;          // wave (M, N) position
    const int lr = lane & 15, lc = lane >> 4;
    const int nk = C / CV_BK;
    const int ntiles = nfb * nlb * ntn;
    // The workgroup's tiles: t_first, t_first + t_step, ... below t_stop.
    // Conv: a contiguous range.  Projection (grid a multiple of 8): the tiles
    // go to the 8 XCDs in 8 contiguous ranges, dealt round-robin to the
    // workgroups of an XCD (hardware workgroup b runs on XCD b % 8), so the
    // Q, K and V tiles of a location block run at the same time on one L2 and
    // its x tile comes from HBM once.
    int t_first = (int)(((int64_t)ntiles * blockIdx.x) / gridDim.x), t_step = 1;
    int t_stop = (int)(((int64_t)ntiles * (blockIdx.x + 1)) / gridDim.x);
    if (TAPS == 1 && (gridDim.x & 7) == 0) {
        const int P = gridDim.x >> 3, xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
        const int r0 = (int)(((int64_t)ntiles * xcd) >> 3), r1 = (int)(((int64_t)ntiles * (xcd + 1)) >> 3);
        const int cnt = r1 - r0 > j ? (r1 - r0 - j + P - 1) / P : 0;
        t_first = r0 + j;
        t_step = P;
        t_stop = t_first + cnt * P;
    }
    const uint32_t frame_bytes = (uint32_t)S * (uint32_t)C * 2u;
    const __amdgpu_buffer_rsrc_t wr = cv_rsrc(w, 3u * (uint32_t)C * (uint32_t)C * 2u);

    // Staging lane mapping: lane l of a wave instruction fills LDS slot l of a
    // 1 KB block = row (16*i + l/4), slot l%4, i.e. chunk (l&3) ^ ((l>>3)&3).
    const int st_row = lane >> 2;
    const int st_chunk = (lane & 3) ^ ((lane >> 3) & 3);
    // Fragment reads: row = base + lr (base a multiple of 16), slot = lc ^ ((lr >> 1) & 3).
    const int rd_off = lr * 64 + ((lc ^ ((lr >> 1) & 3)) << 4);

    auto tile_coords = [&](int t, int& f0, int& s0, int& n0) {
        const int nt = t % ntn, m = t / ntn;
        f0 = (m % nfb) * CV_TF;
        s0 = (m / nfb) * CV_TP;
        n0 = nt * BN;
    };

    // Stage cursor: tile ti, slice ki of the next stage to issue, and ti's
    // coordinates (computed once per tile: tile_coords divides).
    int ti = t_first, ki = 0;
    int cf0 = 0, cs0 = 0, cn0 = 0;
    auto cursor_tile = [&]() { tile_coords(ti, cf0, cs0, cn0); };

    // Issue the loads of slices kc0 .. kc0+KS-1 of the cursor tile into
    // buffer b.  The slice is the instructions' scalar offset (kc * 64 bytes);
    // per lane there are two offsets, formed here from an opaque copy of the
    // lane id (kept live through the stages they would cost registers).
    auto issue = [&](int kc0, int b) {
        int el = lane;
        asm volatile("" : "+v"(el));
        const int srow = el >> 2, schunk = (el & 3) ^ ((el >> 3) & 3);
        // x: the lane's location row of a frame, or past the end (zeros)
        const uint32_t xvoff = cs0 + srow < S ? ((uint32_t)(cs0 + srow) * (uint32_t)C + (uint32_t)(schunk * 8)) * 2u
                                              : frame_bytes;
        // weights: the lane's row of a 16-row block
        const uint32_t wlane = ((uint32_t)srow * (uint32_t)C + (uint32_t)(schunk * 8)) * 2u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint32_t soff = (uint32_t)((kc0 + ks) * CV_BK) * 2u;
            char* abuf = lds + b * L::BUF + ks * L::SLOT;
            char* bbuf = abuf + L::A_BYTES;
            for (int i = wv; i < NSTG; i += NW) {                           // one frame per instruction
                const int f = cf0 - HALO + i;
                const void* base = x;
                uint32_t nrec = 0;
                if (f >= 0 && f < F) {
                    base = x + (int64_t)f * S * C;
                    nrec = frame_bytes;
                } else if (f == -1 && pre) {
                    base = pre;
                    nrec = frame_bytes;
                } else if (f == F && post) {
                    base = post;
                    nrec = frame_bytes;
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(cv_rsrc(base, nrec),
                                                         (__attribute__((address_space(3))) void*)(abuf + i * 1024), 16,
                                                         xvoff, soff, 0, 0);
            }
            for (int i = wv; i < B_INSTR; i += NW) {                        // 16 weight rows per instruction
                // rows 16i .. 16i+15 = tap*BN + co0 + 0..15 (16 divides BN)
                const int tap = i / (BN / 16), co0 = 16 * (i - tap * (BN / 16));
                const uint32_t wsoff = (uint32_t)((tap * C + cn0 + co0) * C) * 2u + soff;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)(bbuf + i * 1024),
                                                         16, wlane, wsoff, 0, 0);
            }
        }
    };


    // Accumulators, started from the bias of the lane's channels (4
    // consecutive channels per fragment, the same for every mi) or zeros.
    f32x4_t acc[4][NF];
    auto acc_init = [&](int t) {
        // lane values from an opaque copy of the lane id, so that nothing of
        // this stays live (hoisted) through the MFMA stages
        int el = lane;
        asm volatile("" : "+v"(el));
        const int lc = el >> 4;
        const int n0 = (t % ntn) * BN;
#pragma unroll
        for (int ni = 0; ni < NF; ++ni) {
            f32x4_t b = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (bias) {
                // channel n of the N range (q, k, v rows for the projection) = bias[n]
                const float* bp = bias + n0 + wn * 16 * NF + ni * 16 + 4 * lc;
                b = f32x4_t{bp[0], bp[1], bp[2], bp[3]};
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][ni] = b;
        }
    };
    if (t_first < t_stop) acc_init(t_first);

    // GroupNorm.  gn_ab is a table of channel pairs, 16 bytes each (a_2p,
    // a_2p+1, b_2p, b_2p+1), so a slice's coefficients are 256 contiguous
    // bytes.  The last wave stages them into a coefficient slot two stages
    // ahead (stage s uses slot s & 1), so every wave sees them after the
    // barrier that precedes their use.  Lane (w = lane & 3, c = (lane >> 2) & 3,
    // r = lane >> 4) normalises word w of chunk c in rows r, r+4, r+8, r+12 of a
    // frame block: channel pair 4c + w of the slice, so it needs one pair of
    // (a, b) per block.  Chunk c of row r sits at slot c ^ ((r >> 1) & 3).
    char* const ab_lds = lds + 2 * L::BUF;
    const int gq = ((lane >> 2) & 3) ^ (lane >> 5);
    const int g_even = (lane >> 4) * 64 + (gq << 4) + (lane & 3) * 4;        // rows r and r + 8 (+512)
    const int g_odd = (lane >> 4) * 64 + ((gq ^ 2) << 4) + (lane & 3) * 4;   // rows r + 4 (+256) and r + 12 (+768)
    const int g_pair = (((lane >> 2) & 3) * 4 + (lane & 3)) * 16;
    auto frame_live = [&](int f) { return (f >= 0 && f < F) || (f == -1 && pre != nullptr) || (f == F && post != nullptr); };
    auto ab_issue = [&](int kc, int slot) {
        if constexpr (GN) {
            if (wv == NW - 1)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(cv_rsrc(gn_ab, (uint32_t)C * 8u),
                                                         (__attribute__((address_space(3))) void*)(ab_lds + slot * 256),
                                                         4, (uint32_t)(kc * 256 + lane * 4), 0, 0, 0);
        }
    };
    // One frame block (blk) of a landed slice: read its raw words and the
    // coefficients (the zero slot for a zero pad, which then stays zero) ...
    auto gn_read = [&](const char* blk, bool live, int slot, uint32_t (&u)[4], f32x4_t& co) {
        u[0] = *reinterpret_cast<const uint32_t*>(blk + g_even);
        u[1] = *reinterpret_cast<const uint32_t*>(blk + g_odd + 256);
        u[2] = *reinterpret_cast<const uint32_t*>(blk + g_even + 512);
        u[3] = *reinterpret_cast<const uint32_t*>(blk + g_odd + 768);
        co = *reinterpret_cast<const f32x4_t*>(live ? ab_lds + slot * 256 + g_pair : ab_lds + 512);
    };
    // ... and write back fmaf(x, a_c, b_c) rounded to bf16.
    auto gn_write = [&](char* blk, const uint32_t (&u)[4], f32x4_t co) {
        uint32_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(fmaf(bf_lo(u[j]), co[0], co[2]), fmaf(bf_hi(u[j]), co[1], co[3]));
        *reinterpret_cast<uint32_t*>(blk + g_even) = v[0];
        *reinterpret_cast<uint32_t*>(blk + g_odd + 256) = v[1];
        *reinterpret_cast<uint32_t*>(blk + g_even + 512) = v[2];
        *reinterpret_cast<uint32_t*>(blk + g_odd + 768) = v[3];
    };
    // All frame blocks this wave loaded for a stage of the tile whose first
    // frame is f0 (coefficient slot slot, buffer buf), from block index i0 on.
    auto gn_blocks = [&](int f0, int buf, int slot, int i0) {
        for (int i = i0; i < NSTG; i += NW) {
            char* blk = lds + buf * L::BUF + i * 1024;
            uint32_t u[4];
            f32x4_t co;
            gn_read(blk, frame_live(f0 - HALO + i), slot, u, co);
            gn_write(blk, u, co);
        }
    };

    auto issue_next = [&](int buf) {
        issue(ki, buf);
        ki += KS;
        if (ki >= nk) {
            ki = 0;
            ti += t_step;
            if (ti < t_stop) cursor_tile();
        }
    };
    if (t_first < t_stop) {
        cursor_tile();
        issue_next(0);
        ab_issue(0, 0);    // stage 0
        ab_issue(ki, 1);   // stage 1
    }
    if constexpr (GN) {
        if (tid < 4) reinterpret_cast<uint32_t*>(ab_lds + 512)[tid] = 0u;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();                      // the coefficients of stages 0 and 1 and the zero slot
        if (t_first < t_stop) {
            int f0, s0, n0;
            tile_coords(t_first, f0, s0, n0);
            gn_blocks(f0, 0, 0, wv);
        }
    }
    int g = 0;  // stage counter across tiles (selects the buffer)
    for (int t = t_first; t < t_stop; t += t_step) {
        for (int kc = 0; kc < nk; kc += KS, ++g) {
            // vmcnt(0): this wave's loads of stage g are in LDS (with GN, waited
            // for, and normalised, while stage g-1 was multiplied).
            if constexpr (!GN) __builtin_amdgcn_s_waitcnt(0x0f70);
            __syncthreads();                      // everyone's are; stage g-1 is no longer read
            const int f0_next = cf0;              // first frame of the tile of stage g+1, if there is one
            // Plain conv (KS = 1, no GroupNorm): this stage's x fragments and first weight fragments are
            // read before the next stage's loads are issued, so their latency overlaps that (branchy,
            // scalar) code instead of following it (measured 1.548 against 1.578 ms at F=1024,
            // 64x40x320; with GroupNorm inside it made no difference, 1.612 against 1.609).
            constexpr bool HOIST = KS == 1 && !GN;
            constexpr int NGH = TAPS * NF, LAH = NGH < 3 ? NGH : 3;
            bf16x8v ah[HOIST ? NA : 1], bh[HOIST ? LAH : 1];
            if constexpr (HOIST) {
                const char* abuf0 = lds + (g & 1) * L::BUF;
                const char* bbuf0 = abuf0 + L::A_BYTES;
#pragma unroll
                for (int j = 0; j < NA; ++j)
                    ah[j] = *reinterpret_cast<const bf16x8v*>(abuf0 + (wm * 64 + j * 16) * 64 + rd_off);
#pragma unroll
                for (int q = 0; q < LAH; ++q) {
                    const int tap = q / NF, ni = q - tap * NF;
                    bh[q] = *reinterpret_cast<const bf16x8v*>(bbuf0 + (tap * BN + wn * 16 * NF + ni * 16) * 64 +
                                                              rd_off);
                }
            }
            if (ti < t_stop) issue_next((g + 1) & 1);
            ab_issue(ki, g & 1);                  // GN: the coefficients of stage g+2
            // GN: stage g+1 is normalised in the shadow of stage g's last MFMA
            // groups.  Each wave rewrites the frame blocks its own loads filled,
            // so its own vmcnt wait suffices; the next barrier publishes them.
            // Past the last stage this rewrites a buffer no one reads again.
            char* const nbuf = lds + ((g + 1) & 1) * L::BUF;
            bool n_live = false;
            if constexpr (GN) n_live = frame_live(f0_next - HALO + wv);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const char* abuf = lds + (g & 1) * L::BUF + ks * L::SLOT;
                const char* bbuf = abuf + L::A_BYTES;
                bf16x8v a[NA];
                if constexpr (HOIST) {
#pragma unroll
                    for (int j = 0; j < NA; ++j) a[j] = ah[j];
                } else {
#pragma unroll
                    for (int j = 0; j < NA; ++j)
                        a[j] = *reinterpret_cast<const bf16x8v*>(abuf + (wm * 64 + j * 16) * 64 + rd_off);
                }
                // (tap, ni) groups of 4 MFMAs; weight fragments are read LA groups ahead.
                constexpr int NG = TAPS * NF, LA = NG < 3 ? NG : 3;
                auto bfrag = [&](int gidx) {
                    const int tap = gidx / NF, ni = gidx - tap * NF;
                    return *reinterpret_cast<const bf16x8v*>(bbuf + (tap * BN + wn * 16 * NF + ni * 16) * 64 +
                                                             rd_off);
                };
                bf16x8v bq[LA];
                if constexpr (HOIST) {
#pragma unroll
                    for (int q = 0; q < LA; ++q) bq[q] = bh[q];
                } else {
#pragma unroll
                    for (int q = 0; q < LA; ++q)
                        if (q < NG) bq[q] = bfrag(q);
                }
                // GN: the next stage's block is read after group GA and written after group GA + GL.
                constexpr int GA = NG > 5 ? NG - 5 : 0, GL = NG - 1 - GA < 2 ? NG - 1 - GA : 2;
                uint32_t gu[4];
                f32x4_t gco;
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const int tap = gi / NF, ni = gi - tap * NF;
                    const bf16x8v b = bq[gi % LA];
                    if (gi + LA < NG) bq[gi % LA] = bfrag(gi + LA);
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a[mi + tap], acc[mi][ni], 0, 0, 0);
                    if constexpr (GN) {
                        if (gi == GA) {
                            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of stage g+1
                            gn_read(nbuf + wv * 1024, n_live, (g + 1) & 1, gu, gco);
                        }
                        if (gi == GA + GL) gn_write(nbuf + wv * 1024, gu, gco);
                    }
                }
                // Keep the fragment reads LA groups ahead of their MFMAs.
                if constexpr (!HOIST) __builtin_amdgcn_sched_group_barrier(0x100, NA + LA, 0);
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                    if (gi + LA < NG) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            // GN: a wave's further blocks (NSTG > NW: the first NSTG - NW waves).
            if constexpr (GN && NSTG > NW)
                if (wv + NW < NSTG) gn_blocks(f0_next, (g + 1) & 1, (g + 1) & 1, wv + NW);
        }
        // Epilogue: fragment (mi, ni) holds frame f0 + 4*wm + mi, location
        // s0 + lane%16, channels n0 + wn*16*NF + ni*16 + 4*(lane/16) + 0..3
        // of output n0 / C (BN divides C, so a tile stays in one output).
        int f0, s0, n0;
        tile_coords(t, f0, s0, n0);
        int el = lane;  // opaque lane id: nothing derived from it is hoisted into the stages
        asm volatile("" : "+v"(el));
        const int lr = el & 15, lc = el >> 4;
        const int s = s0 + lr;
        const int po = TAPS == 3 ? 0 : n0 / C;
        uint16_t* yo = TAPS == 3 ? y : (po == 0 ? y : (po == 1 ? y1 : y2));
        // Output channels of fragment pairs (ni, ni+1) go out as 16-byte
        // pieces: lane group g (= lane / 16) holds 4 channels of each fragment;
        // a 32-lane swap and then a 16-lane swap leave group g with channels
        // 8g .. 8g+7 of the pair (g = 0, 1 from fragment ni, g = 2, 3 from
        // ni+1), so each store covers 64 contiguous bytes of a voxel row.
        auto packed = [&](int mi, int ni, int half) {
            return pack_bf16x2(acc[mi][ni][2 * half], acc[mi][ni][2 * half + 1]);
        };
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int f = f0 + 4 * wm + mi;
            int64_t row = ((int64_t)f * S + s) * C - po * C;
#pragma unroll
            for (int np = 0; np + 1 < NF; np += 2) {
                auto lo = __builtin_amdgcn_permlane32_swap(packed(mi, np, 0), packed(mi, np + 1, 0), false, false);
                lo = __builtin_amdgcn_permlane16_swap(lo[0], lo[1], false, false);
                auto hi = __builtin_amdgcn_permlane32_swap(packed(mi, np, 1), packed(mi, np + 1, 1), false, false);
                hi = __builtin_amdgcn_permlane16_swap(hi[0], hi[1], false, false);
                const int nb = n0 + wn * 16 * NF + np * 16 + 8 * lc;
                if (f < F && s < S)
                    *reinterpret_cast<u32x4_t*>(yo + row + nb) = u32x4_t{lo[0], hi[0], lo[1], hi[1]};
                // Projection: each store completes before the next.  Its tiles
                // write as many bytes as they read in five stages; released at
                // once, the writes hold up the next stages' loads (measured:
                // about 10% slower overall than stores one at a time).
                if constexpr (TAPS == 1) __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            }
            if constexpr (NF & 1) {
                const int ni = NF - 1;
                const int n = n0 + wn * 16 * NF + ni * 16 + 4 * lc;
                const uint2 o = {packed(mi, ni, 0), packed(mi, ni, 1)};
                if (f < F && s < S) *reinterpret_cast<uint2*>(yo + row + n) = o;
                if constexpr (TAPS == 1) __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            }
        }
        // The next tile starts from its bias.  These loads go out after the
        // stores and are first needed after the next stage's wait, so nothing
        // waits on them here (a load between stores would make its wait, on a
        // counter that also counts stores, wait for every store before it).
        if (t + t_step < t_stop) acc_init(t + t_step);
    }
}

// float32 I/O: one output element per thread.
// With gn_a / gn_b (GroupNorm applied inside) each input value is first
// fmaf(x, a_ci, b_ci), as the GroupNorm apply writes it.
__global__ void __launch_bounds__(256) conv3_f32(const float* __restrict__ x, const float* __restrict__ pre,
                                                 const float* __restrict__ post, const float* __restrict__ w,
                                                 const float* __restrict__ bias, const float* __restrict__ gn_a,
                                                 const float* __restrict__ gn_b, float* __restrict__ y, int F,
                                                 int S, int C) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)F * S * C) return;
    const int co = (int)(idx % C);
    const int64_t row = idx / C;
    const int s = (int)(row % S);
    const int f = (int)(row / S);
    float acc = bias ? bias[co] : 0.f;
    for (int k = 0; k < 3; ++k) {
        int fs = f + k - 1;
        const float* xr;
        if (fs < 0)
            xr = pre ? pre + (int64_t)s * C : nullptr;
        else if (fs >= F)
            xr = post ? post + (int64_t)s * C : nullptr;
        else
            xr = x + ((int64_t)fs * S + s) * C;
        if (!xr) continue;
        const float* wr = w + ((int64_t)k * C + co) * C;
        if (gn_a)
            for (int ci = 0; ci < C; ++ci) acc = fmaf(wr[ci], fmaf(xr[ci], gn_a[ci], gn_b[ci]), acc);
        else
            for (int ci = 0; ci < C; ++ci) acc = fmaf(wr[ci], xr[ci], acc);
    }
    y[idx] = acc;
}

// float32 I/O Q/K/V projection: one output element per thread, fp32 FMA;
// element idx of the [3][F*S][C] output space goes to q, k or v.
__global__ void __launch_bounds__(256) qkv_project_f32(const float* __restrict__ x, const float* __restrict__ w,
                                                       const float* __restrict__ bias, float* q, float* k, float* v,
                                                       int64_t FS, int C) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= 3 * FS * C) return;
    const int co = (int)(idx % C);
    const int64_t row = (idx / C) % FS;
    const int p = (int)(idx / (FS * C));
    const float* xr = x + row * C;
    const float* wr = w + ((int64_t)p * C + co) * C;
    float acc = bias ? bias[p * C + co] : 0.f;
    for (int ci = 0; ci < C; ++ci) acc = fmaf(wr[ci], xr[ci], acc);
    (p == 0 ? q : (p == 1 ? k : v))[row * C + co] = acc;
}

// The GroupNorm coefficients per channel, in fp32 exactly as the GroupNorm
// apply forms them: a_c = rstd_g * gamma_c, b_c = beta_c - mean_g * a_c.
// pairs = 0: two tables a[C], b[C] (the fp32 kernel).  pairs = 1: one table
// of channel pairs (a_2p, a_2p+1, b_2p, b_2p+1) in a (the bf16 kernel).
__global__ void __launch_bounds__(256) conv3_gn_coeffs(const float* __restrict__ mean, const float* __restrict__ rstd,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, int C, int cpg, int pairs,
                                                       float* __restrict__ a, float* __restrict__ b) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    const int g = c / cpg;
    const float ga = gamma ? gamma[c] : 1.f;
    const float be = beta ? beta[c] : 0.f;
    const float ac = rstd[g] * ga;
    const float bc = be - mean[g] * ac;
    if (pairs) {
        a[(c >> 1) * 4 + (c & 1)] = ac;
        a[(c >> 1) * 4 + 2 + (c & 1)] = bc;
    } else {
        a[c] = ac;
        b[c] = bc;
    }
}

}  // namespace vinf

namespace vinf_host {
using namespace vinf;

// TAPS = 3: the conv into y.  TAPS = 1: the projection into y, y1, y2, KS
// slices per barrier (C / 32 must be a multiple of KS).
template <int NF, int WN, int TAPS = 3, int KS = 1>
static vinf_status launch_bf16(const void* x, const void* pre, const void* post, const void* w, const float* bias,
                               const float* gn_ab, void* y, int F, int S, int C, hipStream_t st,
                               void* y1 = nullptr, void* y2 = nullptr, bool check_only = false) {
    constexpr int NOUT = TAPS == 3 ? 1 : 3;
    const int nfb = (F + CV_TF - 1) / CV_TF, nlb = (S + CV_TP - 1) / CV_TP,
              ntn = NOUT * C / ConvLds<NF, WN, TAPS, KS>::BN;
    const int64_t tiles = (int64_t)nfb * nlb * ntn;
    if (tiles > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "temporal_conv3: too many tiles");
    if ((uint64_t)S * C * 2 >= 0x80000000ull || (uint64_t)3 * C * C * 2 >= 0x80000000ull)
        return fail(VINF_ERR_UNSUPPORTED, "temporal_conv3: one frame or the weights exceed 2 GiB");
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return fail(VINF_ERR_HIP, "temporal_conv3: cannot query the device");
    if (check_only) return VINF_OK;
    const int grid = (int)std::min<int64_t>(cus, tiles);
    const uint16_t *xb = static_cast<const uint16_t*>(x), *pb = static_cast<const uint16_t*>(pre),
                   *qb = static_cast<const uint16_t*>(post), *wb = static_cast<const uint16_t*>(w);
    uint16_t* yb = static_cast<uint16_t*>(y);
    uint16_t* y1b = y1 ? static_cast<uint16_t*>(y1) : yb;
    uint16_t* y2b = y2 ? static_cast<uint16_t*>(y2) : yb;
    if constexpr (TAPS == 3) {
        if (gn_ab) {
            hipLaunchKernelGGL((conv3_bf16<NF, WN, 3, 1, true>), dim3(grid), dim3(256 * WN), 0, st, xb, pb, qb, wb, bias,
                               gn_ab, yb, y1b, y2b, F, S, C, nfb, nlb, ntn);
            return VINF_OK;
        }
    }
    hipLaunchKernelGGL((conv3_bf16<NF, WN, TAPS, KS, false>), dim3(grid), dim3(256 * WN), 0, st, xb, pb, qb, wb, bias,
                       gn_ab, yb, y1b, y2b, F, S, C, nfb, nlb, ntn);
    return VINF_OK;
}

// The conv, with the GroupNorm coefficients or without (null): bf16 reads the
// channel-pair table in gn_a, fp32 the two tables gn_a / gn_b.  check_only:
// run the host-side size checks and launch nothing.
static vinf_status run_conv3(const void* x, const void* ctx_pre, const void* ctx_post, const void* weight,
                             const float* bias, const float* gn_a, const float* gn_b, void* y, int F, int S, int C,
                             vinf_dtype dt, hipStream_t st, bool check_only = false) {
    if (dt == VINF_BF16) {
        vinf_status r;
        if (C % 320 == 0)
            r = launch_bf16<5, 4>(x, ctx_pre, ctx_post, weight, bias, gn_a, y, F, S, C, st, nullptr, nullptr, check_only);
        else if (C % 256 == 0)
            r = launch_bf16<4, 4>(x, ctx_pre, ctx_post, weight, bias, gn_a, y, F, S, C, st, nullptr, nullptr, check_only);
        else if (C % 128 == 0)
            r = launch_bf16<2, 4>(x, ctx_pre, ctx_post, weight, bias, gn_a, y, F, S, C, st, nullptr, nullptr, check_only);
        else if (C % 64 == 0)
            r = launch_bf16<2, 2>(x, ctx_pre, ctx_post, weight, bias, gn_a, y, F, S, C, st, nullptr, nullptr, check_only);
        else
            r = launch_bf16<1, 2>(x, ctx_pre, ctx_post, weight, bias, gn_a, y, F, S, C, st, nullptr, nullptr, check_only);
        if (r != VINF_OK) return r;
    } else {
        const int64_t n = (int64_t)F * S * C;
        const int64_t blocks = (n + 255) / 256;
        if (blocks > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "temporal_conv3: grid too large");
        if (check_only) return VINF_OK;
        hipLaunchKernelGGL(conv3_f32, dim3((uint32_t)blocks), dim3(256), 0, st, static_cast<const float*>(x),
                           static_cast<const float*>(ctx_pre), static_cast<const float*>(ctx_post),
                           static_cast<const float*>(weight), bias, gn_a, gn_b, static_cast<float*>(y), F, S, C);
    }
    return VINF_OK;
}

vinf_status launch_conv3(const void* x, const void* ctx_pre, const void* ctx_post, const void* weight,
                         const float* bias, void* y, int F, int S, int C, vinf_dtype dt, hipStream_t st) {
    const vinf_status r = run_conv3(x, ctx_pre, ctx_post, weight, bias, nullptr, nullptr, y, F, S, C, dt, st);
    if (r != VINF_OK) return r;
    return check_launch("temporal_conv3");
}

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

size_t conv3_gn_workspace(int C, vinf_dtype dt) {
    (void)dt;
    return 2 * align256((size_t)C * sizeof(float));
}

vinf_status launch_conv3_gn(const void* x, const void* ctx_pre, const void* ctx_post, const void* weight,
                            const float* bias, const float* mean, const float* rstd, const float* gamma,
                            const float* beta, int groups, void* y, int F, int S, int C, vinf_dtype dt,
                            void* workspace, hipStream_t st) {
    // bf16: the pair table (8*C bytes, C even) at the start of the workspace.
    const int pairs = dt == VINF_BF16 ? 1 : 0;
    float* a = static_cast<float*>(workspace);
    float* b = pairs ? a : reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)C * sizeof(float)));
    // Every size check runs before the coefficient kernel writes the
    // workspace, so a rejected call leaves device memory untouched.
    const vinf_status chk = run_conv3(x, ctx_pre, ctx_post, weight, bias, a, b, y, F, S, C, dt, st, true);
    if (chk != VINF_OK) return chk;
    hipLaunchKernelGGL(conv3_gn_coeffs, dim3((C + 255) / 256), dim3(256), 0, st, mean, rstd, gamma, beta, C,
                       C / groups, pairs, a, b);
    const vinf_status r = run_conv3(x, ctx_pre, ctx_post, weight, bias, a, b, y, F, S, C, dt, st);
    if (r != VINF_OK) return r;
    return check_launch("temporal_conv3_gn");
}

vinf_status launch_qkv_project(const void* x, const void* w, const float* bias, void* q, void* k, void* v, int F,
                               int S, int C, vinf_dtype dt, hipStream_t st) {
    if (dt == VINF_BF16) {
        vinf_status r;
        // C / 32 is even whenever C is a multiple of 64: two slices per barrier.
        if (C % 320 == 0)
            r = launch_bf16<5, 4, 1, 2>(x, nullptr, nullptr, w, bias, nullptr, q, F, S, C, st, k, v);
        else if (C % 256 == 0)
            r = launch_bf16<4, 4, 1, 2>(x, nullptr, nullptr, w, bias, nullptr, q, F, S, C, st, k, v);
        else if (C % 128 == 0)
            r = launch_bf16<2, 4, 1, 2>(x, nullptr, nullptr, w, bias, nullptr, q, F, S, C, st, k, v);
        else if (C % 64 == 0)
            r = launch_bf16<2, 2, 1, 2>(x, nullptr, nullptr, w, bias, nullptr, q, F, S, C, st, k, v);
        else
            r = launch_bf16<1, 2, 1, 1>(x, nullptr, nullptr, w, bias, nullptr, q, F, S, C, st, k, v);
        if (r != VINF_OK) return r;
    } else {
        const int64_t FS = (int64_t)F * S;
        const int64_t blocks = (3 * FS * C + 255) / 256;
        if (blocks > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "qkv_project: grid too large");
        hipLaunchKernelGGL(qkv_project_f32, dim3((uint32_t)blocks), dim3(256), 0, st, static_cast<const float*>(x),
                           static_cast<const float*>(w), bias, static_cast<float*>(q), static_cast<float*>(k),
                           static_cast<float*>(v), FS, C);
    }
    return check_launch("qkv_project");
}

}  // namespace vinf_host

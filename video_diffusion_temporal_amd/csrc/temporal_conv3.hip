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
// bf16 kernel (conv3_bf16): an implicit GEMM with M = F*S output voxels,
// N = C_out, K = 3*C_in, on v_mfma_f32_16x16x32_bf16.
//   * A workgroup tile is 8 frames x 16 locations (128 rows of M) by BN
//     output channels.  For each 32-channel slice of C_in it stages 10 frames
//     x 16 locations of x (the 8 frames plus one halo frame per side) and the
//     three taps' weight rows into LDS; a tap is then a shift of the A operand
//     by one frame (16 LDS rows), so the three taps share one staged tile.
//   * 4 waves as 2 (M) x 2 (N).  Each wave's 64 rows are 4 frames; with the
//     tap shift it reads 6 A fragments and 3*BN/32 B fragments per slice for
//     3*4*BN/32 MFMAs.  The next slice's global loads are issued before the
//     current slice's MFMAs (register prefetch).
//   * LDS rows are 64 bytes with an XOR swizzle of the 16-byte chunks.
//   * Workgroup ids are remapped so that the N tiles of one M tile and the
//     next frame block of the same locations run on the same XCD (shared L2
//     for the re-read x rows and halos).
// fp32 kernel (conv3_f32): one output element per thread, fp32 FMA.
#include "common.h"

namespace vinf {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

constexpr int CV_TF = 8;                  // frames per tile
constexpr int CV_TP = 16;                 // locations per tile
constexpr int CV_AROWS = (CV_TF + 2) * CV_TP;  // 160 staged x rows
constexpr int CV_BK = 32;                 // C_in slice

__device__ __forceinline__ int cv_off(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 3)) << 4); }

template <int NF>
__global__ void __launch_bounds__(256) conv3_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ pre,
                                                  const uint16_t* __restrict__ post,
                                                  const uint16_t* __restrict__ w, const float* __restrict__ bias,
                                                  uint16_t* __restrict__ y, int F, int S, int C, int nfb, int ntn) {
    constexpr int BN = 32 * NF;                   // output channels per workgroup
    constexpr int B_ITEMS = 3 * BN * 4;           // 16-byte chunks of the weight tile
    constexpr int B_IT = (B_ITEMS + 255) / 256;
    constexpr int A_ITEMS = CV_AROWS * 4;         // 640
    constexpr int A_IT = (A_ITEMS + 255) / 256;   // 3
    __shared__ __attribute__((aligned(16))) char sa[CV_AROWS * 64];
    __shared__ __attribute__((aligned(16))) char sb[3 * BN * 64];

    const uint32_t lb = xcd_swizzle(blockIdx.x, gridDim.x);
    const int nt = (int)(lb % (uint32_t)ntn);
    const int mt = (int)(lb / (uint32_t)ntn);
    const int fb = mt % nfb, lbk = mt / nfb;
    const int f0 = fb * CV_TF, s0 = lbk * CV_TP, n0 = nt * BN;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;
    const int64_t rs = (int64_t)S * C;

    // Global source of staged A item i: pointer or null (zeros).
    auto a_src = [&](int i) -> const uint16_t* {
        int r = i >> 2, c = i & 3;
        int f = f0 - 1 + r / CV_TP, s = s0 + r % CV_TP;
        if (s >= S) return nullptr;
        if (f < 0) return pre ? pre + (int64_t)s * C + c * 8 : nullptr;
        if (f >= F) return (f == F && post) ? post + (int64_t)s * C + c * 8 : nullptr;
        return x + f * rs + (int64_t)s * C + c * 8;
    };
    const uint16_t* asrc[A_IT];
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
        int i = tid + it * 256;
        asrc[it] = i < A_ITEMS ? a_src(i) : nullptr;
    }
    const uint16_t* bsrc[B_IT];
#pragma unroll
    for (int it = 0; it < B_IT; ++it) {
        int i = tid + it * 256;
        int r = i >> 2, c = i & 3;          // r = tap*BN + co
        int tap = r / BN, co = r % BN;
        bsrc[it] = i < B_ITEMS ? w + ((int64_t)tap * C + n0 + co) * C + c * 8 : nullptr;
    }

    u32x4_t ra[A_IT], rb[B_IT];
    auto gload = [&](int kc) {
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            ra[it] = u32x4_t{0u, 0u, 0u, 0u};
            if (asrc[it]) ra[it] = *reinterpret_cast<const u32x4_t*>(asrc[it] + kc * CV_BK);
        }
#pragma unroll
        for (int it = 0; it < B_IT; ++it)
            if (bsrc[it]) rb[it] = *reinterpret_cast<const u32x4_t*>(bsrc[it] + kc * CV_BK);
    };
    auto lstore = [&]() {
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            int i = tid + it * 256;
            if (i < A_ITEMS) *reinterpret_cast<u32x4_t*>(sa + cv_off(i >> 2, i & 3)) = ra[it];
        }
#pragma unroll
        for (int it = 0; it < B_IT; ++it) {
            int i = tid + it * 256;
            if (i < B_ITEMS) *reinterpret_cast<u32x4_t*>(sb + cv_off(i >> 2, i & 3)) = rb[it];
        }
    };

    f32x4_t acc[4][NF];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < NF; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = C / CV_BK;
    const int lr = lane & 15, lc = lane >> 4;
    gload(0);
    for (int kc = 0; kc < nk; ++kc) {
        __syncthreads();  // previous slice's fragments are consumed
        lstore();
        __syncthreads();
        if (kc + 1 < nk) gload(kc + 1);
        bf16x8v a[6];
#pragma unroll
        for (int j = 0; j < 6; ++j)
            a[j] = *reinterpret_cast<const bf16x8v*>(sa + cv_off(wm * 64 + j * 16 + lr, lc));
#pragma unroll
        for (int tap = 0; tap < 3; ++tap) {
            bf16x8v b[NF];
#pragma unroll
            for (int ni = 0; ni < NF; ++ni)
                b[ni] = *reinterpret_cast<const bf16x8v*>(sb + cv_off(tap * BN + wn * 16 * NF + ni * 16 + lr, lc));
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < NF; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi + tap], b[ni], acc[mi][ni], 0, 0, 0);
        }
    }

    // Epilogue: fragment (mi, ni) holds frame f0 + 4*wm + mi, locations
    // s0 + 4*(lane/16) + i, channel n0 + wn*16*NF + ni*16 + lane%16.
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        int f = f0 + 4 * wm + mi;
        if (f >= F) continue;
#pragma unroll
        for (int ni = 0; ni < NF; ++ni) {
            int n = n0 + wn * 16 * NF + ni * 16 + lr;
            float bv = bias ? bias[n] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int s = s0 + 4 * lc + i;
                if (s < S) {
                    bf16x2_t r;
                    r[0] = (__bf16)(acc[mi][ni][i] + bv);
                    y[f * rs + (int64_t)s * C + n] = __builtin_bit_cast(uint16_t, r[0]);
                }
            }
        }
    }
}

// float32 I/O: one output element per thread.
__global__ void __launch_bounds__(256) conv3_f32(const float* __restrict__ x, const float* __restrict__ pre,
                                                 const float* __restrict__ post, const float* __restrict__ w,
                                                 const float* __restrict__ bias, float* __restrict__ y, int F, int S,
                                                 int C) {
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
        for (int ci = 0; ci < C; ++ci) acc = fmaf(wr[ci], xr[ci], acc);
    }
    y[idx] = acc;
}

}  // namespace vinf

namespace vinf_host {
using namespace vinf;

template <int NF>
static void launch_bf16(const void* x, const void* pre, const void* post, const void* w, const float* bias, void* y,
                        int F, int S, int C, hipStream_t st, int64_t* blocks_out) {
    const int nfb = (F + CV_TF - 1) / CV_TF, nlb = (S + CV_TP - 1) / CV_TP, ntn = C / (32 * NF);
    const int64_t blocks = (int64_t)nfb * nlb * ntn;
    *blocks_out = blocks;
    if (blocks > 0x7fffffff) return;
    hipLaunchKernelGGL(conv3_bf16<NF>, dim3((uint32_t)blocks), dim3(256), 0, st, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(pre), static_cast<const uint16_t*>(post),
                       static_cast<const uint16_t*>(w), bias, static_cast<uint16_t*>(y), F, S, C, nfb, ntn);
}

vinf_status launch_conv3(const void* x, const void* ctx_pre, const void* ctx_post, const void* weight,
                         const float* bias, void* y, int F, int S, int C, vinf_dtype dt, hipStream_t st) {
    if (dt == VINF_BF16) {
        int64_t blocks = 0;
        if (C % 160 == 0)
            launch_bf16<5>(x, ctx_pre, ctx_post, weight, bias, y, F, S, C, st, &blocks);
        else if (C % 128 == 0)
            launch_bf16<4>(x, ctx_pre, ctx_post, weight, bias, y, F, S, C, st, &blocks);
        else if (C % 64 == 0)
            launch_bf16<2>(x, ctx_pre, ctx_post, weight, bias, y, F, S, C, st, &blocks);
        else
            launch_bf16<1>(x, ctx_pre, ctx_post, weight, bias, y, F, S, C, st, &blocks);
        if (blocks > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "temporal_conv3: grid too large");
    } else {
        const int64_t n = (int64_t)F * S * C;
        const int64_t blocks = (n + 255) / 256;
        if (blocks > 0x7fffffff) return fail(VINF_ERR_UNSUPPORTED, "temporal_conv3: grid too large");
        hipLaunchKernelGGL(conv3_f32, dim3((uint32_t)blocks), dim3(256), 0, st, static_cast<const float*>(x),
                           static_cast<const float*>(ctx_pre), static_cast<const float*>(ctx_post),
                           static_cast<const float*>(weight), bias, static_cast<float*>(y), F, S, C);
    }
    return check_launch("temporal_conv3");
}

}  // namespace vinf_host

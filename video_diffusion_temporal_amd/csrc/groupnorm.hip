// GroupNorm with statistics over the whole video, gfx950.
//
// Method (Video-Infinity write-up, GroupNorm-module paragraph): the group
// means are computed first and aggregated into a global mean; the standard
// deviation is then computed with that global mean and aggregated into a
// global standard deviation; both normalise every frame.
//
// Kernels, all on the caller's stream, no atomics:
//   gn_partial<first>   every block streams a disjoint set of rows of the
//                       [rows = F*H*W][C] tensor with 16-byte loads; each
//                       thread owns one fixed 16-byte channel vector, so its
//                       per-channel fp32 sums never mix channels.  The block
//                       folds its row-slots in LDS in a fixed order and
//                       writes one fp32 partial per channel: partial[B][C].
//   gn_finalize<first>  one block per group sums the group's B*C/G partials
//                       in fp64 in a fixed order -> mean_g.
//   gn_partial<second>  the same sweep accumulating (x - mean_g)^2, walking
//                       the rows from the end, so that its first reads hit
//                       what the first sweep left in the last-level cache.
//   gn_finalize<second> -> rstd_g = 1/sqrt(var_g + eps).
//   gn_apply            y = x * a_c + b_c with a_c = rstd_g*gamma_c and
//                       b_c = beta_c - mean_g*a_c, forward again (its first
//                       rows are the ones the second sweep read last).
// HBM traffic: three reads and one write of the tensor.
#include <math.h>

#include "common.h"

namespace vinf {

constexpr int GN_MAX_BLOCKS = 2048;

struct GnGeom {
    int E;        // elements per 16-byte vector
    int V;        // vectors per row
    int RB;       // rows a block covers per sweep step
    int threads;  // RB * V
    int blocks;   // B
};

static GnGeom gn_geom(int64_t rows, int C, vinf_dtype dt) {
    GnGeom g;
    g.E = dt == VINF_BF16 ? 8 : 4;
    g.V = C / g.E;
    g.RB = g.V <= 256 ? 256 / g.V : 1;
    g.threads = g.RB * g.V;
    int64_t b = (rows + g.RB - 1) / g.RB;
    g.blocks = (int)(b < GN_MAX_BLOCKS ? b : GN_MAX_BLOCKS);
    return g;
}

template <bool BF16>
__device__ __forceinline__ u32x4_t load16(const void* base, int64_t elem) {
    const char* p = static_cast<const char*>(base) + elem * (BF16 ? 2 : 4);
    return *reinterpret_cast<const u32x4_t*>(p);
}

// Unpack one 16-byte vector into E floats.
template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4_t& u, float* f) {
    if constexpr (BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = bf_lo(u[j]);
            f[2 * j + 1] = bf_hi(u[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(u[j]);
    }
}

template <bool BF16, bool SECOND>
__global__ void __launch_bounds__(1024) gn_partial(const void* __restrict__ x, const float* __restrict__ stats,
                                                   float* __restrict__ partial, int64_t rows, int C, int V, int RB,
                                                   int cpg) {
    constexpr int E = BF16 ? 8 : 4;
    extern __shared__ float red[];  // [RB][C]
    const int vi = threadIdx.x % V, rb = threadIdx.x / V;
    const int c0 = vi * E;
    float mu[E], acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        mu[e] = SECOND ? stats[(c0 + e) / cpg] : 0.f;
        acc[e] = 0.f;
    }
    const int64_t stride = (int64_t)gridDim.x * RB;
    int64_t r = (int64_t)blockIdx.x * RB + rb;
    auto row = [&](int64_t i) { return SECOND ? rows - 1 - i : i; };
    auto add = [&](const u32x4_t& u) {
        float f[E];
        unpack<BF16>(u, f);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if constexpr (SECOND) {
                float d = f[e] - mu[e];
                acc[e] = fmaf(d, d, acc[e]);
            } else {
                acc[e] += f[e];
            }
        }
    };
    for (; r + 3 * stride < rows; r += 4 * stride) {
        u32x4_t a = load16<BF16>(x, row(r) * C + c0);
        u32x4_t b = load16<BF16>(x, row(r + stride) * C + c0);
        u32x4_t c = load16<BF16>(x, row(r + 2 * stride) * C + c0);
        u32x4_t d = load16<BF16>(x, row(r + 3 * stride) * C + c0);
        add(a);
        add(b);
        add(c);
        add(d);
    }
    for (; r < rows; r += stride) add(load16<BF16>(x, row(r) * C + c0));

#pragma unroll
    for (int e = 0; e < E; ++e) red[rb * C + c0 + e] = acc[e];
    __syncthreads();
    if (rb == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float s = red[c0 + e];
            for (int i = 1; i < RB; ++i) s += red[i * C + c0 + e];
            partial[(int64_t)blockIdx.x * C + c0 + e] = s;
        }
    }
}

// One block per group: fixed-order fp64 sum of the group's partials.
// stats = [mean_0..mean_{G-1}, rstd_0..rstd_{G-1}] (float).
template <bool SECOND>
__global__ void __launch_bounds__(256) gn_finalize(const float* __restrict__ partial, float* __restrict__ stats,
                                                   float* __restrict__ out, int B, int C, int cpg, int G,
                                                   double inv_n, float eps) {
    __shared__ double red[256];
    const int g = blockIdx.x;
    const int64_t items = (int64_t)B * cpg;
    // item i = (block b = i / cpg, channel g*cpg + i % cpg); thread t owns items
    // t, t+256, ...; eight loads in flight into eight fp64 partial sums.
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int64_t i = threadIdx.x;
    for (; i + 7 * 256 < items; i += 8 * 256) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t it = i + u * 256, b = it / cpg;
            v[u] = partial[b * C + g * cpg + (int)(it - b * cpg)];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += (double)v[u];
    }
    for (int u = 0; i < items; i += 256, ++u) {
        const int64_t b = i / cpg;
        acc[u & 7] += (double)partial[b * C + g * cpg + (int)(i - b * cpg)];
    }
    double s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        double m = red[0] * inv_n;
        float v = SECOND ? (float)(1.0 / sqrt(m + (double)eps)) : (float)m;
        stats[(SECOND ? G : 0) + g] = v;
        if (out) out[g] = v;
    }
}

template <bool BF16>
__global__ void __launch_bounds__(1024) gn_apply(const void* __restrict__ x, void* __restrict__ y,
                                                 const float* __restrict__ stats, const float* __restrict__ gamma,
                                                 const float* __restrict__ beta, int64_t rows, int C, int V, int RB,
                                                 int cpg, int G) {
    constexpr int E = BF16 ? 8 : 4;
    const int vi = threadIdx.x % V, rb = threadIdx.x / V;
    const int c0 = vi * E;
    float a[E], b[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        int g = (c0 + e) / cpg;
        float ga = gamma ? gamma[c0 + e] : 1.f;
        float be = beta ? beta[c0 + e] : 0.f;
        a[e] = stats[G + g] * ga;
        b[e] = be - stats[g] * a[e];
    }
    const int64_t stride = (int64_t)gridDim.x * RB;
    auto emit = [&](int64_t rr, const u32x4_t& u) {
        float f[E];
        unpack<BF16>(u, f);
        u32x4_t o;
        if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = pack_bf16x2(fmaf(f[2 * j], a[2 * j], b[2 * j]), fmaf(f[2 * j + 1], a[2 * j + 1], b[2 * j + 1]));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = __float_as_uint(fmaf(f[j], a[j], b[j]));
        }
        char* p = static_cast<char*>(y) + (rr * C + c0) * (BF16 ? 2 : 4);
        *reinterpret_cast<u32x4_t*>(p) = o;
    };
    int64_t r = (int64_t)blockIdx.x * RB + rb;
    for (; r + 3 * stride < rows; r += 4 * stride) {
        u32x4_t u0 = load16<BF16>(x, r * C + c0);
        u32x4_t u1 = load16<BF16>(x, (r + stride) * C + c0);
        u32x4_t u2 = load16<BF16>(x, (r + 2 * stride) * C + c0);
        u32x4_t u3 = load16<BF16>(x, (r + 3 * stride) * C + c0);
        emit(r, u0);
        emit(r + stride, u1);
        emit(r + 2 * stride, u2);
        emit(r + 3 * stride, u3);
    }
    for (; r < rows; r += stride) emit(r, load16<BF16>(x, r * C + c0));
}

}  // namespace vinf

namespace vinf_host {
using namespace vinf;

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

size_t groupnorm_workspace(int64_t rows, int C, int groups, vinf_dtype dt) {
    GnGeom g = gn_geom(rows, C, dt);
    return align256((size_t)g.blocks * C * sizeof(float)) + align256(2 * (size_t)groups * sizeof(float));
}

template <bool BF16>
static vinf_status run(const void* x, void* y, const float* gamma, const float* beta, float* mean_out,
                       float* rstd_out, int64_t rows, int C, int G, float eps, void* ws, hipStream_t st) {
    GnGeom g = gn_geom(rows, C, BF16 ? VINF_BF16 : VINF_F32);
    float* partial = static_cast<float*>(ws);
    float* stats = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)g.blocks * C * sizeof(float)));
    const int cpg = C / G;
    const double inv_n = 1.0 / ((double)rows * (double)cpg);
    const size_t lds = (size_t)g.RB * C * sizeof(float);
    hipLaunchKernelGGL((gn_partial<BF16, false>), dim3(g.blocks), dim3(g.threads), lds, st, x, stats, partial, rows,
                       C, g.V, g.RB, cpg);
    hipLaunchKernelGGL((gn_finalize<false>), dim3(G), dim3(256), 0, st, partial, stats, mean_out, g.blocks, C, cpg,
                       G, inv_n, eps);
    hipLaunchKernelGGL((gn_partial<BF16, true>), dim3(g.blocks), dim3(g.threads), lds, st, x, stats, partial, rows,
                       C, g.V, g.RB, cpg);
    hipLaunchKernelGGL((gn_finalize<true>), dim3(G), dim3(256), 0, st, partial, stats, rstd_out, g.blocks, C, cpg,
                       G, inv_n, eps);
    hipLaunchKernelGGL((gn_apply<BF16>), dim3(g.blocks), dim3(g.threads), 0, st, x, y, stats, gamma, beta, rows, C,
                       g.V, g.RB, cpg, G);
    return check_launch("groupnorm");
}

vinf_status launch_groupnorm(const void* x, void* y, const float* gamma, const float* beta, float* mean_out,
                             float* rstd_out, int64_t rows, int C, int groups, float eps, vinf_dtype dt,
                             void* workspace, hipStream_t stream) {
    if (dt == VINF_BF16)
        return run<true>(x, y, gamma, beta, mean_out, rstd_out, rows, C, groups, eps, workspace, stream);
    return run<false>(x, y, gamma, beta, mean_out, rstd_out, rows, C, groups, eps, workspace, stream);
}

}  // namespace vinf_host

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
// HBM traffic: three reads and one write of the tensor.  Without y (the
// statistics alone, when the conv applies the normalisation itself) the apply
// is skipped: two reads.
//
// Clip form (the clip-parallelism paragraph: every device holds one clip and
// the statistics are aggregated across devices): the same sweeps over one
// clip write the fp64 group sums instead of a statistic (gn_finalize with
// dsum); the caller adds the clips' sums (one all-reduce per pass) and
// gn_stats_from_sums turns the totals into mean_g / rstd_g for the second
// sweep and the apply.  The statistic expressions are shared, so one clip
// covering the whole video reproduces the whole-video path bit for bit.
#include <math.h>

#include <mutex>

#include "common.h"

namespace vinf {

// Scratch of vinf_groupnorm_global_noalloc: the per-block partial sums and
// the statistics of one call, in a static device array instead of a
// caller-provided workspace.  Every call on a GPU uses that GPU's copy.
static __device__ __align__(256) char scratch[VINF_NOALLOC_SCRATCH_BYTES];

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

// The statistics from fp64 group sums over n voxel-channels.
__device__ __forceinline__ float gn_mean_of(double sum, double n) { return (float)(sum / n); }
__device__ __forceinline__ float gn_rstd_of(double sq_sum, double n, float eps) {
    return (float)(1.0 / sqrt(sq_sum / n + (double)eps));
}

// One block per group: fixed-order fp64 sum of the group's partials.
// stats = [mean_0..mean_{G-1}, rstd_0..rstd_{G-1}] (float).  With stats
// non-null the block writes its statistic there (and to out, if non-null);
// with dsum non-null it writes the raw fp64 sum to dsum[g].
constexpr int GN_FIN_THREADS = 1024;

template <bool SECOND>
__global__ void __launch_bounds__(GN_FIN_THREADS) gn_finalize(const float* __restrict__ partial,
                                                              float* __restrict__ stats, float* __restrict__ out,
                                                              double* __restrict__ dsum, int B, int C, int cpg, int G,
                                                              double n, float eps) {
    constexpr int NT = GN_FIN_THREADS;
    __shared__ double red[NT];
    const int g = blockIdx.x;
    const int items = B * cpg;  // <= GN_MAX_BLOCKS * C
    // item i = (block b = i / cpg, channel g*cpg + i % cpg); thread t owns items
    // t, t+NT, ...; eight loads in flight into eight fp64 partial sums (the
    // group's items are a few per thread, so the sweep is a few load rounds).
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int i = threadIdx.x;
    for (; i + 7 * NT < items; i += 8 * NT) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int it = i + u * NT, b = it / cpg;
            v[u] = partial[(int64_t)b * C + g * cpg + (it - b * cpg)];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += (double)v[u];
    }
    for (int u = 0; i < items; i += NT, ++u) {
        const int b = i / cpg;
        acc[u & 7] += (double)partial[(int64_t)b * C + g * cpg + (i - b * cpg)];
    }
    double s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = NT / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (dsum) dsum[g] = red[0];
        if (stats) {
            const float v = SECOND ? gn_rstd_of(red[0], n, eps) : gn_mean_of(red[0], n);
            stats[(SECOND ? G : 0) + g] = v;
            if (out) out[g] = v;
        }
    }
}

// stats[g] = mean_g from sum[g]; with sq_sum non-null also stats[G+g] = rstd_g.
__global__ void __launch_bounds__(256) gn_stats_from_sums(const double* __restrict__ sum,
                                                          const double* __restrict__ sq_sum, float* __restrict__ stats,
                                                          float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                          int G, double n, float eps) {
    for (int g = blockIdx.x * blockDim.x + threadIdx.x; g < G; g += gridDim.x * blockDim.x) {
        const float m = gn_mean_of(sum[g], n);
        stats[g] = m;
        if (mean_out) mean_out[g] = m;
        if (sq_sum) {
            const float r = gn_rstd_of(sq_sum[g], n, eps);
            stats[G + g] = r;
            if (rstd_out) rstd_out[g] = r;
        }
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

struct GnBufs {
    GnGeom g;
    float* partial;  // [B][C]
    float* stats;    // [2G]: mean_g, rstd_g
};

static GnBufs gn_bufs(int64_t rows, int C, vinf_dtype dt, void* ws) {
    GnBufs b;
    b.g = gn_geom(rows, C, dt);
    b.partial = static_cast<float*>(ws);
    b.stats = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)b.g.blocks * C * sizeof(float)));
    return b;
}

template <bool BF16, bool SECOND>
static void sweep(const void* x, const GnBufs& b, int64_t rows, int C, int cpg, hipStream_t st) {
    const size_t lds = (size_t)b.g.RB * C * sizeof(float);
    hipLaunchKernelGGL((gn_partial<BF16, SECOND>), dim3(b.g.blocks), dim3(b.g.threads), lds, st, x, b.stats,
                       b.partial, rows, C, b.g.V, b.g.RB, cpg);
}

template <bool BF16>
static void apply(const void* x, void* y, const float* gamma, const float* beta, const GnBufs& b, int64_t rows, int C,
                  int cpg, int G, hipStream_t st) {
    hipLaunchKernelGGL((gn_apply<BF16>), dim3(b.g.blocks), dim3(b.g.threads), 0, st, x, y, b.stats, gamma, beta,
                       rows, C, b.g.V, b.g.RB, cpg, G);
}

template <bool BF16>
static vinf_status run(const void* x, void* y, const float* gamma, const float* beta, float* mean_out,
                       float* rstd_out, int64_t rows, int C, int G, float eps, void* ws, hipStream_t st) {
    const GnBufs b = gn_bufs(rows, C, BF16 ? VINF_BF16 : VINF_F32, ws);
    const int cpg = C / G;
    const double n = (double)rows * (double)cpg;
    sweep<BF16, false>(x, b, rows, C, cpg, st);
    hipLaunchKernelGGL((gn_finalize<false>), dim3(G), dim3(GN_FIN_THREADS), 0, st, b.partial, b.stats, mean_out, nullptr,
                       b.g.blocks, C, cpg, G, n, eps);
    sweep<BF16, true>(x, b, rows, C, cpg, st);
    hipLaunchKernelGGL((gn_finalize<true>), dim3(G), dim3(GN_FIN_THREADS), 0, st, b.partial, b.stats, rstd_out, nullptr,
                       b.g.blocks, C, cpg, G, n, eps);
    if (y) apply<BF16>(x, y, gamma, beta, b, rows, C, cpg, G, st);
    return check_launch("groupnorm");
}

template <bool BF16>
static vinf_status run_clip_sums(const void* x, const double* mean_sums, double* sums, int64_t rows, int C, int G,
                                 double n_total, void* ws, hipStream_t st) {
    const GnBufs b = gn_bufs(rows, C, BF16 ? VINF_BF16 : VINF_F32, ws);
    const int cpg = C / G;
    if (mean_sums) {
        hipLaunchKernelGGL(gn_stats_from_sums, dim3((G + 255) / 256), dim3(256), 0, st, mean_sums, nullptr, b.stats,
                           nullptr, nullptr, G, n_total, 0.f);
        sweep<BF16, true>(x, b, rows, C, cpg, st);
        hipLaunchKernelGGL((gn_finalize<true>), dim3(G), dim3(GN_FIN_THREADS), 0, st, b.partial, nullptr, nullptr, sums,
                           b.g.blocks, C, cpg, G, n_total, 0.f);
    } else {
        sweep<BF16, false>(x, b, rows, C, cpg, st);
        hipLaunchKernelGGL((gn_finalize<false>), dim3(G), dim3(GN_FIN_THREADS), 0, st, b.partial, nullptr, nullptr, sums,
                           b.g.blocks, C, cpg, G, n_total, 0.f);
    }
    return check_launch("groupnorm_clip_sums");
}

template <bool BF16>
static vinf_status run_clip_apply(const void* x, void* y, const float* gamma, const float* beta, const double* sums,
                                  const double* sq_sums, float* mean_out, float* rstd_out, int64_t rows, int C, int G,
                                  double n_total, float eps, void* ws, hipStream_t st) {
    const GnBufs b = gn_bufs(rows, C, BF16 ? VINF_BF16 : VINF_F32, ws);
    hipLaunchKernelGGL(gn_stats_from_sums, dim3((G + 255) / 256), dim3(256), 0, st, sums, sq_sums, b.stats, mean_out,
                       rstd_out, G, n_total, eps);
    if (x) apply<BF16>(x, y, gamma, beta, b, rows, C, C / G, G, st);
    return check_launch("groupnorm_clip_apply");
}

vinf_status launch_groupnorm(const void* x, void* y, const float* gamma, const float* beta, float* mean_out,
                             float* rstd_out, int64_t rows, int C, int groups, float eps, vinf_dtype dt,
                             void* workspace, hipStream_t stream) {
    if (dt == VINF_BF16)
        return run<true>(x, y, gamma, beta, mean_out, rstd_out, rows, C, groups, eps, workspace, stream);
    return run<false>(x, y, gamma, beta, mean_out, rstd_out, rows, C, groups, eps, workspace, stream);
}

// The device address of the scratch array on the current device, looked up
// once per device (the array's name in host code is not a device address).
static vinf_status scratch_address(void** out) {
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static void* addr[MAX_DEVICES] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return fail(VINF_ERR_HIP, "groupnorm_noalloc: no current device (or more than %d)", MAX_DEVICES);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(VINF_ERR_HIP, "groupnorm_noalloc: hipGetSymbolAddress failed on device %d: %s", dev,
                        hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return VINF_OK;
}

vinf_status launch_groupnorm_noalloc(const void* x, void* y, const float* gamma, const float* beta, float* mean_out,
                                     float* rstd_out, int64_t rows, int C, int groups, float eps, vinf_dtype dt,
                                     hipStream_t stream) {
    const size_t need = groupnorm_workspace(rows, C, groups, dt);
    if (need > VINF_NOALLOC_SCRATCH_BYTES)
        return fail(VINF_ERR_UNSUPPORTED,
                    "vinf_groupnorm_global_noalloc: C=%d needs %zu bytes of scratch, more than the %zu the library holds",
                    C, need, (size_t)VINF_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    const vinf_status r = scratch_address(&ws);
    if (r != VINF_OK) return r;
    return launch_groupnorm(x, y, gamma, beta, mean_out, rstd_out, rows, C, groups, eps, dt, ws, stream);
}

vinf_status launch_groupnorm_clip_sums(const void* x, const double* mean_sums, double* sums, int64_t rows, int C,
                                       int groups, double n_total, vinf_dtype dt, void* workspace,
                                       hipStream_t stream) {
    if (dt == VINF_BF16)
        return run_clip_sums<true>(x, mean_sums, sums, rows, C, groups, n_total, workspace, stream);
    return run_clip_sums<false>(x, mean_sums, sums, rows, C, groups, n_total, workspace, stream);
}

vinf_status launch_groupnorm_clip_apply(const void* x, void* y, const float* gamma, const float* beta,
                                        const double* sums, const double* sq_sums, float* mean_out, float* rstd_out,
                                        int64_t rows, int C, int groups, double n_total, float eps, vinf_dtype dt,
                                        void* workspace, hipStream_t stream) {
    if (dt == VINF_BF16)
        return run_clip_apply<true>(x, y, gamma, beta, sums, sq_sums, mean_out, rstd_out, rows, C, groups, n_total,
                                    eps, workspace, stream);
    return run_clip_apply<false>(x, y, gamma, beta, sums, sq_sums, mean_out, rstd_out, rows, C, groups, n_total, eps,
                                 workspace, stream);
}

}  // namespace vinf_host

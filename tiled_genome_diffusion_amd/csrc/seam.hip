// Standalone seam kernels: overlap-consistency projection and the per-seam
// RMS discrepancy with a fixed-order summary reduction.  The fused variants
// live in the chain step kernel; these serve projections every K > 1 steps,
// post-projection checks and states produced elsewhere.
#include "common.hpp"
#include "launch.hpp"

namespace pc {
namespace {

__device__ __forceinline__ void pair_indices(int p, int O, int &lidx, int &ridx) {
    int pp, qq;
    block_pair_row_col(p, O, pp, qq);
    lidx = packed_index(kBeads - O + pp, kBeads - O + qq);
    ridx = packed_index(pp, qq);
}

// One lane per (chain, seam, column, pair).
__global__ __launch_bounds__(256) void k_seam_project(float *__restrict__ state, int64_t total, int32_t n_cols,
                                                      ChainArgs ch, int64_t block0) {
    const int64_t it = (block0 + blockIdx.x) * blockDim.x + threadIdx.x;
    if (it >= total) return;
    const int NP = ch.n_pairs, L = ch.chain_len;
    const int p = static_cast<int>(it % NP);
    const int64_t sc = it / NP;                 // ((c (L-1) + j) n_cols + col)
    const int col = static_cast<int>(sc % n_cols);
    const int64_t cj = sc / n_cols;
    const int64_t c = cj / (L - 1);
    const int64_t j = cj - c * (L - 1);
    int li, ri;
    pair_indices(p, ch.overlap, li, ri);
    const size_t map_l = static_cast<size_t>((c * L + j) * n_cols + col);
    const size_t map_r = map_l + n_cols;
    const float m = (state[map_l * kPacked + li] + state[map_r * kPacked + ri]) * 0.5f;
    state[map_l * kPacked + li] = m;
    state[map_r * kPacked + ri] = m;
}

// One wavefront per (chain, seam, column): lane l sums the squared
// differences of pairs l, l + 64, ... in that order, and a DPP tree over the
// lanes (fixed order, so the result is deterministic) forms the sum over the
// seam's pairs.
constexpr int kDiscThreads = 256;
constexpr int kDiscWaves = kDiscThreads / 64;

__global__ __launch_bounds__(kDiscThreads) void k_seam_disc(const float *__restrict__ state, int64_t total,
                                                            int32_t n_cols, ChainArgs ch, float *__restrict__ rms,
                                                            int64_t block0) {
    const int64_t sc = (block0 + blockIdx.x) * kDiscWaves + (threadIdx.x >> 6);
    if (sc >= total) return;  // uniform over the wavefront
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int L = ch.chain_len, NP = ch.n_pairs;
    const int col = static_cast<int>(sc % n_cols);
    const int64_t cj = sc / n_cols;
    const int64_t c = cj / (L - 1);
    const int64_t j = cj - c * (L - 1);
    const float *xl = state + static_cast<size_t>((c * L + j) * n_cols + col) * kPacked;
    const float *xr = xl + static_cast<size_t>(n_cols) * kPacked;
    float acc = 0.f;
    for (int p = lane; p < NP; p += 64) {
        int li, ri;
        pair_indices(p, ch.overlap, li, ri);
        const float d = xl[li] - xr[ri];
        acc = fmaf(d, d, acc);
    }
    const float sum = wave_sum(acc);
    if (lane == 0) rms[sc] = sqrtf(sum / static_cast<float>(NP));
}

// Paper-form seam discrepancy: one 1024-lane workgroup per (chain, seam,
// weight g).  Lane (j, p), j < J = 1024 / NP, sums pair p's left and right
// copies over the trajectories s = j, j + J, ... in index order (float64);
// lane p then adds its J partial sums in order, and a fixed-order tree over
// the pairs forms the mean of |mean left - mean right|.
constexpr int kMeanAbsThreads = 1024;

__global__ __launch_bounds__(kMeanAbsThreads) void k_seam_mean_abs(const float *__restrict__ state, int32_t G,
                                                                  int32_t S, ChainArgs ch, float *__restrict__ out,
                                                                  int64_t block0) {
    __shared__ double s_l[kMeanAbsThreads], s_r[kMeanAbsThreads];
    const int NP = ch.n_pairs, L = ch.chain_len;
    const int J = kMeanAbsThreads / NP;
    const int64_t blk = block0 + blockIdx.x;            // (c (L - 1) + seam) G + g
    const int cj = static_cast<int>(blk / G);           // c (L - 1) + seam
    const int g = static_cast<int>(blk - static_cast<int64_t>(cj) * G);
    const int c = cj / (L - 1);
    const int seam = cj - c * (L - 1);
    const int n_cols = G * S;
    const int t = static_cast<int>(threadIdx.x);
    const int j = t / NP, p = t - j * NP;
    double sl = 0.0, sr = 0.0;
    if (j < J) {
        int li, ri;
        pair_indices(p, ch.overlap, li, ri);
        const float *xl = state + (static_cast<size_t>(c * L + seam) * n_cols + static_cast<size_t>(g) * S) * kPacked + li;
        const float *xr = xl + static_cast<size_t>(n_cols) * kPacked - li + ri;
        int s = j;
        for (; s + 3 * J < S; s += 4 * J) {  // four trajectories in flight, summed in index order
            const float a0 = xl[static_cast<size_t>(s) * kPacked], a1 = xl[static_cast<size_t>(s + J) * kPacked];
            const float a2 = xl[static_cast<size_t>(s + 2 * J) * kPacked];
            const float a3 = xl[static_cast<size_t>(s + 3 * J) * kPacked];
            const float b0 = xr[static_cast<size_t>(s) * kPacked], b1 = xr[static_cast<size_t>(s + J) * kPacked];
            const float b2 = xr[static_cast<size_t>(s + 2 * J) * kPacked];
            const float b3 = xr[static_cast<size_t>(s + 3 * J) * kPacked];
            sl += a0; sl += a1; sl += a2; sl += a3;
            sr += b0; sr += b1; sr += b2; sr += b3;
        }
        for (; s < S; s += J) {
            sl += xl[static_cast<size_t>(s) * kPacked];
            sr += xr[static_cast<size_t>(s) * kPacked];
        }
    }
    s_l[t] = sl;
    s_r[t] = sr;
    __syncthreads();
    double v = 0.0;
    if (t < NP) {
        double tl = 0.0, tr = 0.0;
        for (int jj = 0; jj < J; ++jj) {
            tl += s_l[jj * NP + t];
            tr += s_r[jj * NP + t];
        }
        v = fabs(tl - tr) / S;
    }
    __syncthreads();
    s_l[t] = v;
    __syncthreads();
    for (int h = kMeanAbsThreads / 2; h > 0; h >>= 1) {
        if (t < h) s_l[t] += s_l[t + h];
        __syncthreads();
    }
    if (t == 0) out[blk] = static_cast<float>(s_l[0] / NP);
}

// Mean and max of n values by one workgroup: each lane folds a strided slice
// in index order (eight loads in flight), then a fixed tree over the lanes.
// Deterministic.
constexpr int kMeanMaxThreads = 1024;

__global__ __launch_bounds__(kMeanMaxThreads) void k_mean_max(const float *__restrict__ v, int64_t n,
                                                              float *__restrict__ out) {
    __shared__ double s_sum[kMeanMaxThreads];
    __shared__ float s_max[kMeanMaxThreads];
    constexpr int T = kMeanMaxThreads;
    double acc = 0.0;
    float mx = 0.f;
    int64_t i = threadIdx.x;
    for (; i + 7 * T < n; i += 8 * T) {
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = v[i + k * T];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            acc += x[k];
            mx = fmaxf(mx, x[k]);
        }
    }
    for (; i < n; i += T) {
        acc += v[i];
        mx = fmaxf(mx, v[i]);
    }
    s_sum[threadIdx.x] = acc;
    s_max[threadIdx.x] = mx;
    __syncthreads();
    for (int h = T / 2; h > 0; h >>= 1) {
        if (static_cast<int>(threadIdx.x) < h) {
            s_sum[threadIdx.x] += s_sum[threadIdx.x + h];
            s_max[threadIdx.x] = fmaxf(s_max[threadIdx.x], s_max[threadIdx.x + h]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[0] = n > 0 ? static_cast<float>(s_sum[0] / static_cast<double>(n)) : 0.f;
        out[1] = s_max[0];
    }
}

}  // namespace

hipError_t launch_seam_project(float *state, int32_t n_chains, int32_t n_cols, ChainArgs ch, hipStream_t stream) {
    const int64_t total = static_cast<int64_t>(n_chains) * (ch.chain_len - 1) * n_cols * ch.n_pairs;
    return launch_slices((total + 255) / 256, 256, [&](int64_t first, uint32_t count) {
        hipLaunchKernelGGL(k_seam_project, dim3(count), dim3(256), 0, stream, state, total, n_cols, ch, first);
    });
}

hipError_t launch_seam_mean_abs(const float *state, int32_t n_chains, int32_t G, int32_t S, ChainArgs ch, float *out,
                                hipStream_t stream) {
    const int64_t blocks = static_cast<int64_t>(n_chains) * (ch.chain_len - 1) * G;
    return launch_slices(blocks, kMeanAbsThreads, [&](int64_t first, uint32_t count) {
        hipLaunchKernelGGL(k_seam_mean_abs, dim3(count), dim3(kMeanAbsThreads), 0, stream, state, G, S, ch, out,
                           first);
    });
}

hipError_t launch_seam_discrepancy(const float *state, int32_t n_chains, int32_t n_cols, ChainArgs ch, float *rms,
                                   float *summary, hipStream_t stream) {
    const int64_t total = static_cast<int64_t>(n_chains) * (ch.chain_len - 1) * n_cols;
    const hipError_t e = launch_slices((total + kDiscWaves - 1) / kDiscWaves, kDiscThreads,
                                       [&](int64_t first, uint32_t count) {
        hipLaunchKernelGGL(k_seam_disc, dim3(count), dim3(kDiscThreads), 0, stream, state, total, n_cols, ch, rms,
                           first);
    });
    if (e != hipSuccess || !summary) return e;
    hipLaunchKernelGGL(k_mean_max, dim3(1), dim3(kMeanMaxThreads), 0, stream, rms, total, summary);
    return hipGetLastError();
}

}  // namespace pc

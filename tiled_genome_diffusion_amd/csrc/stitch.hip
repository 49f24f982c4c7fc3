// Rigid stitching of adjacent tiles' point clouds into one chain per joint
// sample (chain c, weight g, trajectory s): one 64-lane workgroup per joint
// sample, lane i owning bead i of the current tile, walking the chain's
// tiles in order.
//
// Tile k+1 is aligned onto the aligned tile k by the orthogonal map R and
// translation that best superpose its first O beads on tile k's last O beads:
// with centred shared beads x (tile k+1) and y (tile k), H = x^T y and R is the
// orthogonal polar factor of H (= U V^T for H = U S V^T; reflections allowed,
// since distance maps carry no chirality), found by Higham's scaled Newton
// iteration X <- (g X + X^{-T} / g) / 2.  The seam's residual is the RMS
// distance over the shared beads after alignment; a shared bead takes the
// mean of its two aligned positions.  Centroids, H and the residual are DPP
// wavefront sums over the O shared lanes.
#include "common.hpp"
#include "launch.hpp"

namespace pc {
namespace {

__device__ __forceinline__ float det3(const float (&m)[3][3]) {
    return m[0][0] * (m[1][1] * m[2][2] - m[1][2] * m[2][1]) - m[0][1] * (m[1][0] * m[2][2] - m[1][2] * m[2][0]) +
           m[0][2] * (m[1][0] * m[2][1] - m[1][1] * m[2][0]);
}

// Orthogonal polar factor of a non-singular 3x3 (wave-uniform values).
__device__ __forceinline__ void polar3(float (&x)[3][3]) {
    for (int it = 0; it < 12; ++it) {
        const float d = det3(x);
        if (d == 0.f) return;
        // inverse-transpose = cofactor matrix / det
        float it_[3][3];
        it_[0][0] = (x[1][1] * x[2][2] - x[1][2] * x[2][1]) / d;
        it_[0][1] = (x[1][2] * x[2][0] - x[1][0] * x[2][2]) / d;
        it_[0][2] = (x[1][0] * x[2][1] - x[1][1] * x[2][0]) / d;
        it_[1][0] = (x[0][2] * x[2][1] - x[0][1] * x[2][2]) / d;
        it_[1][1] = (x[0][0] * x[2][2] - x[0][2] * x[2][0]) / d;
        it_[1][2] = (x[0][1] * x[2][0] - x[0][0] * x[2][1]) / d;
        it_[2][0] = (x[0][1] * x[1][2] - x[0][2] * x[1][1]) / d;
        it_[2][1] = (x[0][2] * x[1][0] - x[0][0] * x[1][2]) / d;
        it_[2][2] = (x[0][0] * x[1][1] - x[0][1] * x[1][0]) / d;
        float nx = 0.f, ni = 0.f;
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                nx += x[a][b] * x[a][b];
                ni += it_[a][b] * it_[a][b];
            }
        const float g = it < 8 ? sqrtf(sqrtf(ni / nx)) : 1.f;  // scaled steps, then plain Newton
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b) x[a][b] = 0.5f * (g * x[a][b] + it_[a][b] / g);
    }
}

__global__ __launch_bounds__(64) void k_stitch(const float *__restrict__ coords, int32_t G, int32_t S,
                                               ChainArgs ch, float *__restrict__ chain, float *__restrict__ resid) {
    const int i = threadIdx.x;
    const int n_cols = G * S;
    const int c = static_cast<int>(blockIdx.x) / n_cols;
    const int gs = static_cast<int>(blockIdx.x) - c * n_cols;
    const int L = ch.chain_len, O = ch.overlap, stride = kBeads - O;
    const int n_beads = (L - 1) * stride + kBeads;
    float *out = chain + (static_cast<size_t>(c) * n_cols + gs) * n_beads * 3;
    const bool shared = i < O;
    float prev[3] = {0.f, 0.f, 0.f};
    for (int k = 0; k < L; ++k) {
        const size_t map = (static_cast<size_t>(c) * L + k) * n_cols + gs;
        const float *src = coords + (map * kBeads + i) * 3;
        float x[3] = {src[0], src[1], src[2]};
        float cur[3] = {x[0], x[1], x[2]};
        float yp[3] = {0.f, 0.f, 0.f};  // tile k's aligned partner of bead i (shared lanes)
        if (k > 0) {
            const int partner = shared ? kBeads - O + i : i;
#pragma unroll
            for (int a = 0; a < 3; ++a) yp[a] = __shfl(prev[a], partner);
            float xm[3], ym[3];
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                xm[a] = wave_sum(shared ? x[a] : 0.f) / O;
                ym[a] = wave_sum(shared ? yp[a] : 0.f) / O;
            }
            float h[3][3];
#pragma unroll
            for (int a = 0; a < 3; ++a)
#pragma unroll
                for (int b = 0; b < 3; ++b) h[a][b] = wave_sum(shared ? (x[a] - xm[a]) * (yp[b] - ym[b]) : 0.f);
            polar3(h);
#pragma unroll
            for (int b = 0; b < 3; ++b)
                cur[b] = (x[0] - xm[0]) * h[0][b] + (x[1] - xm[1]) * h[1][b] + (x[2] - xm[2]) * h[2][b] + ym[b];
            float d2 = 0.f;
#pragma unroll
            for (int a = 0; a < 3; ++a) d2 += (cur[a] - yp[a]) * (cur[a] - yp[a]);
            const float r2 = wave_sum(shared ? d2 : 0.f) / O;
            if (i == 0) resid[(static_cast<size_t>(c) * (L - 1) + k - 1) * n_cols + gs] = sqrtf(r2);
        }
        // Shared beads are written as the mean of both copies by the later tile.
        const bool later = k > 0 && shared;
        const bool deferred = i >= stride && k < L - 1;
        float *dst = out + (static_cast<size_t>(k) * stride + i) * 3;
        if (later) {
#pragma unroll
            for (int a = 0; a < 3; ++a) dst[a] = 0.5f * (cur[a] + yp[a]);
        } else if (!deferred) {
#pragma unroll
            for (int a = 0; a < 3; ++a) dst[a] = cur[a];
        }
#pragma unroll
        for (int a = 0; a < 3; ++a) prev[a] = cur[a];
    }
}

}  // namespace

hipError_t launch_stitch(const float *coords, int32_t n_chains, int32_t G, int32_t S, ChainArgs ch, float *chain,
                         float *resid, hipStream_t stream) {
    const int64_t blocks = static_cast<int64_t>(n_chains) * G * S;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_stitch, dim3(static_cast<uint32_t>(blocks)), dim3(64), 0, stream, coords, G, S, ch, chain,
                       resid);
    return hipGetLastError();
}

}  // namespace pc

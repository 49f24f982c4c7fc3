// Rigid stitching of adjacent tiles' point clouds into one chain per joint
// sample (chain c, weight g, trajectory s).
//
// Tile k is aligned onto the aligned tile k-1 by the orthogonal map and
// translation that best superpose its first O beads on tile k-1's last O
// beads.  The best fit onto a rigidly moved target is the moved best fit, so
// with F_k the fit of raw tile k onto raw tile k-1 (row vectors:
// F_k(x) = x R_k + t_k) the aligned frame of tile k is T_k = T_{k-1} o F_k,
// T_0 = identity: M_k = R_k M_{k-1}, u_k = t_k M_{k-1} + u_{k-1}.  Hence one
// 1024-lane workgroup per joint sample works in three phases:
//   1. each of its 16 wavefronts fits seams k = 1..L-1 in turn (lane i < O
//      holds shared bead i of both tiles): centroids, H = x^T y of the centred
//      beads, R_k = the orthogonal polar factor of H (= U V^T for
//      H = U S V^T; reflections allowed, since distance maps carry no
//      chirality) by Higham's scaled Newton iteration, and the seam's
//      residual, the RMS distance over the shared beads after
//      the fit, which no rigid motion of both tiles changes;
//   2. one lane composes the L transforms in order (LDS);
//   3. the wavefronts move their tiles' beads into the chain frame; a shared
//      bead takes the mean of its two aligned positions (written by the later
//      tile).
#include "common.hpp"
#include "launch.hpp"

namespace pc {
namespace {

constexpr int kStitchThreads = 1024;
constexpr int kStitchWaves = kStitchThreads / 64;

__device__ __forceinline__ float det3(const float (&m)[3][3]) {
    return m[0][0] * (m[1][1] * m[2][2] - m[1][2] * m[2][1]) - m[0][1] * (m[1][0] * m[2][2] - m[1][2] * m[2][0]) +
           m[0][2] * (m[1][0] * m[2][1] - m[1][1] * m[2][0]);
}

// Orthogonal polar factor of a non-singular 3x3 (wave-uniform values) by
// Higham's scaled Newton iteration X <- (g X + X^{-T} / g) / 2, X^{-T} the
// cofactor matrix over det X, g = (|X^{-1}|_F / |X|_F)^(1/2) for the first
// steps and 1 after.  The iteration corrects its own rounding, so the
// hardware reciprocal and square root serve; it stops once a step moves X by
// less than float32 resolution (quadratic convergence: 5 to 8 steps).
__device__ __forceinline__ void polar3(float (&x)[3][3]) {
    for (int it = 0; it < 12; ++it) {
        const float d = det3(x);
        if (d == 0.f) return;
        const float rd = __builtin_amdgcn_rcpf(d);
        float it_[3][3];
        it_[0][0] = (x[1][1] * x[2][2] - x[1][2] * x[2][1]) * rd;
        it_[0][1] = (x[1][2] * x[2][0] - x[1][0] * x[2][2]) * rd;
        it_[0][2] = (x[1][0] * x[2][1] - x[1][1] * x[2][0]) * rd;
        it_[1][0] = (x[0][2] * x[2][1] - x[0][1] * x[2][2]) * rd;
        it_[1][1] = (x[0][0] * x[2][2] - x[0][2] * x[2][0]) * rd;
        it_[1][2] = (x[0][1] * x[2][0] - x[0][0] * x[2][1]) * rd;
        it_[2][0] = (x[0][1] * x[1][2] - x[0][2] * x[1][1]) * rd;
        it_[2][1] = (x[0][2] * x[1][0] - x[0][0] * x[1][2]) * rd;
        it_[2][2] = (x[0][0] * x[1][1] - x[0][1] * x[1][0]) * rd;
        float nx = 0.f, ni = 0.f;
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                nx = fmaf(x[a][b], x[a][b], nx);
                ni = fmaf(it_[a][b], it_[a][b], ni);
            }
        const float g = it < 6 ? __builtin_amdgcn_sqrtf(__builtin_amdgcn_sqrtf(ni * __builtin_amdgcn_rcpf(nx))) : 1.f;
        const float hg = 0.5f * g, hr = 0.5f * __builtin_amdgcn_rcpf(g);
        float moved = 0.f;
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                const float v = fmaf(hg, x[a][b], hr * it_[a][b]);
                moved = fmaf(v - x[a][b], v - x[a][b], moved);
                x[a][b] = v;
            }
        if (it >= 6 && moved <= 1e-13f * nx) return;  // converged to float32 resolution
    }
}

// Rigid transform x -> x M + u of a row vector; M row-major at t[0..8], u at t[9..11].
__device__ __forceinline__ void apply(const float *t, const float (&x)[3], float (&y)[3]) {
#pragma unroll
    for (int b = 0; b < 3; ++b) y[b] = fmaf(x[0], t[b], fmaf(x[1], t[3 + b], fmaf(x[2], t[6 + b], t[9 + b])));
}

__global__ __launch_bounds__(kStitchThreads) void k_stitch(const float *__restrict__ coords, int32_t G, int32_t S,
                                                           ChainArgs ch, float *__restrict__ chain,
                                                           float *__restrict__ resid) {
    extern __shared__ float s_t[];  // [L][12]: F_k after phase 1, T_k after phase 2
    const int wave = static_cast<int>(threadIdx.x) >> 6, lane = static_cast<int>(threadIdx.x) & 63;
    const int n_cols = G * S;
    const int c = static_cast<int>(blockIdx.x) / n_cols;
    const int gs = static_cast<int>(blockIdx.x) - c * n_cols;
    const int L = ch.chain_len, O = ch.overlap, stride = kBeads - O;
    const int n_beads = (L - 1) * stride + kBeads;
    auto bead = [&](int k, int i) {  // raw coordinates of bead i of tile k
        const float *p = coords + ((static_cast<size_t>(c * L + k) * n_cols + gs) * kBeads + i) * 3;
        return p;
    };
    const bool shared = lane < O;

    // 1. pairwise fits of raw tile k onto raw tile k-1
    for (int k = 1 + wave; k < L; k += kStitchWaves) {
        float x[3] = {0.f, 0.f, 0.f}, y[3] = {0.f, 0.f, 0.f};
        if (shared) {
            const float *px = bead(k, lane), *py = bead(k - 1, stride + lane);
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                x[a] = px[a];
                y[a] = py[a];
            }
        }
        float xm[3], ym[3];
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            xm[a] = wave_sum(x[a]) / O;
            ym[a] = wave_sum(y[a]) / O;
        }
        float h[3][3];
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b) h[a][b] = wave_sum(shared ? (x[a] - xm[a]) * (y[b] - ym[b]) : 0.f);
        polar3(h);
        float fx[3];
#pragma unroll
        for (int b = 0; b < 3; ++b)
            fx[b] = (x[0] - xm[0]) * h[0][b] + (x[1] - xm[1]) * h[1][b] + (x[2] - xm[2]) * h[2][b] + ym[b];
        float d2 = 0.f;
#pragma unroll
        for (int a = 0; a < 3; ++a) d2 += (fx[a] - y[a]) * (fx[a] - y[a]);
        const float r2 = wave_sum(shared ? d2 : 0.f) / O;
        if (lane == 0) {
            resid[(static_cast<size_t>(c) * (L - 1) + k - 1) * n_cols + gs] = sqrtf(r2);
            float *t = s_t + 12 * k;
#pragma unroll
            for (int a = 0; a < 3; ++a)
#pragma unroll
                for (int b = 0; b < 3; ++b) t[3 * a + b] = h[a][b];
            // t_k = ym - xm R
#pragma unroll
            for (int b = 0; b < 3; ++b) t[9 + b] = ym[b] - (xm[0] * h[0][b] + xm[1] * h[1][b] + xm[2] * h[2][b]);
        }
    }
    __syncthreads();

    // 2. compose: T_0 = identity, M_k = R_k M_{k-1}, u_k = t_k M_{k-1} + u_{k-1}
    if (threadIdx.x == 0) {
        float m[9] = {1.f, 0.f, 0.f, 0.f, 1.f, 0.f, 0.f, 0.f, 1.f}, u[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 9; ++e) s_t[e] = m[e];
        s_t[9] = s_t[10] = s_t[11] = 0.f;
        for (int k = 1; k < L; ++k) {
            float *t = s_t + 12 * k;
            float nm[9], nu[3];
#pragma unroll
            for (int a = 0; a < 3; ++a)
#pragma unroll
                for (int b = 0; b < 3; ++b)
                    nm[3 * a + b] = fmaf(t[3 * a], m[b], fmaf(t[3 * a + 1], m[3 + b], t[3 * a + 2] * m[6 + b]));
#pragma unroll
            for (int b = 0; b < 3; ++b)
                nu[b] = fmaf(t[9], m[b], fmaf(t[10], m[3 + b], fmaf(t[11], m[6 + b], u[b])));
#pragma unroll
            for (int e = 0; e < 9; ++e) t[e] = m[e] = nm[e];
#pragma unroll
            for (int b = 0; b < 3; ++b) t[9 + b] = u[b] = nu[b];
        }
    }
    __syncthreads();

    // 3. move every tile into the chain frame
    float *out = chain + (static_cast<size_t>(c) * n_cols + gs) * n_beads * 3;
    for (int k = wave; k < L; k += kStitchWaves) {
        const float *p = bead(k, lane);
        const float x[3] = {p[0], p[1], p[2]};
        float cur[3];
        apply(s_t + 12 * k, x, cur);
        float *dst = out + (static_cast<size_t>(k) * stride + lane) * 3;
        if (k > 0 && shared) {  // mean with tile k-1's aligned copy of the same bead
            const float *q = bead(k - 1, stride + lane);
            const float y[3] = {q[0], q[1], q[2]};
            float prev[3];
            apply(s_t + 12 * (k - 1), y, prev);
#pragma unroll
            for (int a = 0; a < 3; ++a) dst[a] = 0.5f * (cur[a] + prev[a]);
        } else if (!(lane >= stride && k < L - 1)) {  // beads shared with tile k+1 are written by it
#pragma unroll
            for (int a = 0; a < 3; ++a) dst[a] = cur[a];
        }
    }
}

}  // namespace

hipError_t launch_stitch(const float *coords, int32_t n_chains, int32_t G, int32_t S, ChainArgs ch, float *chain,
                         float *resid, hipStream_t stream) {
    const int64_t blocks = static_cast<int64_t>(n_chains) * G * S;
    if (blocks == 0) return hipSuccess;
    const size_t lds = static_cast<size_t>(ch.chain_len) * 12 * sizeof(float);
    hipLaunchKernelGGL(k_stitch, dim3(static_cast<uint32_t>(blocks)), dim3(kStitchThreads), lds, stream, coords, G, S,
                       ch, chain, resid);
    return hipGetLastError();
}

}  // namespace pc

// Rigid stitching of adjacent tiles' point clouds into one chain per joint
// sample (chain c, weight g, trajectory s).
//
// Tile k is aligned onto the aligned tile k-1 by the orthogonal map and
// translation that best superpose its first O beads on tile k-1's last O
// beads.  The best fit onto a rigidly moved target is the moved best fit, so
// with F_k the fit of raw tile k onto raw tile k-1 (row vectors:
// F_k(x) = x R_k + t_k) the aligned frame of tile k is
// T_k = F_1 o F_2 o ... o F_k, an inclusive scan under composition.  One
// 256-lane workgroup per joint sample works in three phases:
//   1. the tiles are taken in chunks of 64, one lane per tile: lane k fits
//      seam k on its own (centroids and H = x^T y of the centred shared
//      beads in one shifted pass, R_k = the orthogonal polar factor of H by
//      Higham's scaled Newton iteration, reflections allowed since distance
//      maps carry no chirality, then the seam's residual, the RMS distance
//      over the shared beads after the fit, which no rigid motion of both
//      tiles changes), and a wavefront scan composes the chunk's fits;
//   2. the chunks' scans are joined by carrying each chunk's total into the
//      next (LDS, at most 16 chunks);
//   3. the wavefronts move their tiles' beads into the chain frame, one lane
//      per bead; a shared bead takes the mean of its two aligned positions
//      (written by the later tile).
// PROPER restricts every fit to rotations (det +1), Kabsch's fit with the
// determinant correction: where the polar factor Q of H is a reflection, the
// best rotation is Q (I - 2 v v^T), v the unit eigenvector of the symmetric
// factor P = Q^T H for its smallest eigenvalue (with H = U S V^T, Q = U V^T,
// P = V S V^T, and the fit U diag(1, 1, -1) V^T = Q - 2 (Q v) v^T).
#include "common.hpp"
#include "launch.hpp"

namespace pc {
namespace {

constexpr int kStitchThreads = 256;
constexpr int kStitchWaves = kStitchThreads / 64;
constexpr int kStitchMaxChunks = 16;  // chains of up to 1024 tiles

__device__ __forceinline__ float det3(const float (&m)[3][3]) {
    return m[0][0] * (m[1][1] * m[2][2] - m[1][2] * m[2][1]) - m[0][1] * (m[1][0] * m[2][2] - m[1][2] * m[2][0]) +
           m[0][2] * (m[1][0] * m[2][1] - m[1][1] * m[2][0]);
}

// Orthogonal polar factor of a non-singular 3x3 (one per lane) by
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

// Unit eigenvector of a symmetric 3x3 for its smallest eigenvalue: the
// eigenvalue from the trigonometric solution of the characteristic cubic
// (Smith, CACM 4(4), 1961), the vector as the longest cross product of two
// rows of P - lambda I (which spans the eigenvalue's null space).
__device__ __forceinline__ void smallest_eigvec3(const float (&p)[3][3], float (&v)[3]) {
    const float q = (p[0][0] + p[1][1] + p[2][2]) * (1.f / 3.f);
    const float off = fmaf(p[0][1], p[0][1], fmaf(p[0][2], p[0][2], p[1][2] * p[1][2]));
    const float d0 = p[0][0] - q, d1 = p[1][1] - q, d2 = p[2][2] - q;
    const float s = sqrtf(fmaf(d0, d0, fmaf(d1, d1, fmaf(d2, d2, 2.f * off))) * (1.f / 6.f));
    float lam = q;
    if (s > 0.f) {
        const float is = 1.f / s;
        const float b[3][3] = {{d0 * is, p[0][1] * is, p[0][2] * is},
                               {p[1][0] * is, d1 * is, p[1][2] * is},
                               {p[2][0] * is, p[2][1] * is, d2 * is}};
        const float r = fminf(1.f, fmaxf(-1.f, 0.5f * det3(b)));
        lam = fmaf(2.f * s, cosf(acosf(r) * (1.f / 3.f) + 2.09439510239319549f), q);  // + 2 pi / 3
    }
    const float m[3][3] = {{p[0][0] - lam, p[0][1], p[0][2]},
                           {p[1][0], p[1][1] - lam, p[1][2]},
                           {p[2][0], p[2][1], p[2][2] - lam}};
    float best = -1.f;
    v[0] = 0.f;
    v[1] = 0.f;
    v[2] = 1.f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b2 = a + 1; b2 < 3; ++b2) {
            const float c[3] = {m[a][1] * m[b2][2] - m[a][2] * m[b2][1], m[a][2] * m[b2][0] - m[a][0] * m[b2][2],
                                m[a][0] * m[b2][1] - m[a][1] * m[b2][0]};
            const float n2 = fmaf(c[0], c[0], fmaf(c[1], c[1], c[2] * c[2]));
            if (n2 > best) {
                best = n2;
                v[0] = c[0];
                v[1] = c[1];
                v[2] = c[2];
            }
        }
    // Rank one or zero (the smallest eigenvalue is repeated): every vector orthogonal to the
    // rows is an eigenvector; take one orthogonal to the longest row (any vector if all vanish).
    float w[3] = {m[0][0], m[0][1], m[0][2]}, wn = fmaf(w[0], w[0], fmaf(w[1], w[1], w[2] * w[2]));
#pragma unroll
    for (int a = 1; a < 3; ++a) {
        const float n = fmaf(m[a][0], m[a][0], fmaf(m[a][1], m[a][1], m[a][2] * m[a][2]));
        if (n > wn) {
            wn = n;
            w[0] = m[a][0];
            w[1] = m[a][1];
            w[2] = m[a][2];
        }
    }
    if (!(best > 1e-8f * wn * wn) && wn > 0.f) {
        // w x e_j for the axis e_j least aligned with w
        const int j = fabsf(w[0]) <= fabsf(w[1]) ? (fabsf(w[0]) <= fabsf(w[2]) ? 0 : 2)
                                                 : (fabsf(w[1]) <= fabsf(w[2]) ? 1 : 2);
        v[0] = j == 0 ? 0.f : (j == 1 ? -w[2] : w[1]);
        v[1] = j == 0 ? w[2] : (j == 1 ? 0.f : -w[0]);
        v[2] = j == 0 ? -w[1] : (j == 1 ? w[0] : 0.f);
        best = fmaf(v[0], v[0], fmaf(v[1], v[1], v[2] * v[2]));
    }
    if (best > 0.f) {
        const float in = 1.f / sqrtf(best);
        v[0] *= in;
        v[1] *= in;
        v[2] *= in;
    }
}

// q <- the best rotation for H where the polar factor q of H is a reflection.
__device__ __forceinline__ void make_proper(float (&q)[3][3], const float (&h)[3][3]) {
    if (!(det3(q) < 0.f)) return;
    float pm[3][3];
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) pm[a][b] = fmaf(q[0][a], h[0][b], fmaf(q[1][a], h[1][b], q[2][a] * h[2][b]));
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = a + 1; b < 3; ++b) pm[a][b] = pm[b][a] = 0.5f * (pm[a][b] + pm[b][a]);
    float v[3];
    smallest_eigvec3(pm, v);
    float qv[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) qv[a] = fmaf(q[a][0], v[0], fmaf(q[a][1], v[1], q[a][2] * v[2]));
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) q[a][b] = fmaf(-2.f * qv[a], v[b], q[a][b]);
}

// Rigid transform x -> x M + u of a row vector; M row-major at t[0..8], u at t[9..11].
__device__ __forceinline__ void apply(const float *t, const float (&x)[3], float (&y)[3]) {
#pragma unroll
    for (int b = 0; b < 3; ++b) y[b] = fmaf(x[0], t[b], fmaf(x[1], t[3 + b], fmaf(x[2], t[6 + b], t[9 + b])));
}

// out = a o b (b first, then a): x (M_b M_a) + (u_b M_a + u_a).  out may alias b.
__device__ __forceinline__ void compose(const float (&a)[12], float (&b)[12]) {
    float r[12];
#pragma unroll
    for (int i = 0; i < 4; ++i)  // rows 0..2 of M_b, then u_b (row 3, plus u_a)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            r[3 * i + j] = fmaf(b[3 * i], a[j], fmaf(b[3 * i + 1], a[3 + j], fmaf(b[3 * i + 2], a[6 + j],
                                                                             i == 3 ? a[9 + j] : 0.f)));
#pragma unroll
    for (int e = 0; e < 12; ++e) b[e] = r[e];
}

__device__ __forceinline__ void identity(float (&t)[12]) {
#pragma unroll
    for (int e = 0; e < 12; ++e) t[e] = (e == 0 || e == 4 || e == 8) ? 1.f : 0.f;
}

// Fit of O beads x (tile k's first) onto y (tile k-1's last): t = (R, shift) with
// y ~ x R + shift; returns the mean squared distance after the fit.  The sums
// are shifted by each block's first bead, so centring loses nothing to
// cancellation.
template <bool PROPER>
__device__ float fit(const float *x, const float *y, int O, float (&t)[12]) {
    float x0[3], y0[3], sx[3] = {0.f, 0.f, 0.f}, sy[3] = {0.f, 0.f, 0.f}, h[3][3] = {};
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        x0[a] = x[a];
        y0[a] = y[a];
    }
    for (int i = 1; i < O; ++i) {
        float dx[3], dy[3];
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            dx[a] = x[3 * i + a] - x0[a];
            dy[a] = y[3 * i + a] - y0[a];
            sx[a] += dx[a];
            sy[a] += dy[a];
        }
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 3; ++b) h[a][b] = fmaf(dx[a], dy[b], h[a][b]);
    }
    const float inv = 1.f / static_cast<float>(O);
    float xm[3], ym[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        xm[a] = sx[a] * inv;  // centroid offsets from bead 0
        ym[a] = sy[a] * inv;
    }
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) h[a][b] = fmaf(-static_cast<float>(O) * xm[a], ym[b], h[a][b]);
    float hc[3][3];
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) hc[a][b] = h[a][b];
    polar3(h);
    if (PROPER) make_proper(h, hc);
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        xm[a] += x0[a];
        ym[a] += y0[a];
    }
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) t[3 * a + b] = h[a][b];
#pragma unroll
    for (int b = 0; b < 3; ++b) t[9 + b] = ym[b] - (xm[0] * h[0][b] + xm[1] * h[1][b] + xm[2] * h[2][b]);
    float r2 = 0.f;
    for (int i = 0; i < O; ++i) {
        const float p[3] = {x[3 * i], x[3 * i + 1], x[3 * i + 2]};
        float q[3];
        apply(t, p, q);
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            const float d = q[a] - y[3 * i + a];
            r2 = fmaf(d, d, r2);
        }
    }
    return r2 * inv;
}

template <bool PROPER>
__global__ __launch_bounds__(kStitchThreads) void k_stitch(const float *__restrict__ coords, int32_t G, int32_t S,
                                                           ChainArgs ch, float *__restrict__ chain,
                                                           float *__restrict__ resid, int64_t block0) {
    extern __shared__ float s_t[];  // [L][12]: chunk-local scans, then T_k; [16][12]: chunk totals, then carries
    const int wave = static_cast<int>(threadIdx.x) >> 6, lane = static_cast<int>(threadIdx.x) & 63;
    const int n_cols = G * S;
    const int64_t blk = block0 + blockIdx.x;  // joint sample c n_cols + gs
    const int c = static_cast<int>(blk / n_cols);
    const int gs = static_cast<int>(blk - static_cast<int64_t>(c) * n_cols);
    const int L = ch.chain_len, O = ch.overlap, stride = kBeads - O;
    const int n_beads = (L - 1) * stride + kBeads;
    const int n_chunks = (L + 63) >> 6;
    float *s_tot = s_t + 12 * L;
    auto tile = [&](int k) {  // raw coordinates of tile k, [64][3]
        return coords + (static_cast<size_t>(c * L + k) * n_cols + gs) * kBeads * 3;
    };

    // 1. per-lane fits, scanned within each 64-tile chunk
    for (int j = wave; j < n_chunks; j += kStitchWaves) {
        const int k = 64 * j + lane;
        float t[12];
        identity(t);
        if (k >= 1 && k < L) {
            const float r2 = fit<PROPER>(tile(k), tile(k - 1) + stride * 3, O, t);
            resid[(static_cast<size_t>(c) * (L - 1) + k - 1) * n_cols + gs] = sqrtf(r2);
        }
        // inclusive scan: t_k <- t_{k-d} o t_k
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            float o[12];
#pragma unroll
            for (int e = 0; e < 12; ++e) o[e] = __shfl_up(t[e], d, 64);
            if (lane >= d) compose(o, t);
        }
        if (k < L) {
#pragma unroll
            for (int e = 0; e < 12; ++e) s_t[12 * k + e] = t[e];
        }
        if (lane == 63) {
#pragma unroll
            for (int e = 0; e < 12; ++e) s_tot[12 * j + e] = t[e];
        }
    }
    __syncthreads();

    // 2. carries: C_0 = identity, C_{j+1} = C_j o total_j (stored over the totals)
    if (threadIdx.x == 0 && n_chunks > 1) {
        float cur[12];
        identity(cur);
        for (int j = 0; j < n_chunks; ++j) {
            float nxt[12];
#pragma unroll
            for (int e = 0; e < 12; ++e) nxt[e] = s_tot[12 * j + e];
            compose(cur, nxt);
#pragma unroll
            for (int e = 0; e < 12; ++e) {
                s_tot[12 * j + e] = cur[e];
                cur[e] = nxt[e];
            }
        }
    }
    __syncthreads();
    if (n_chunks > 1) {
        for (int k = 64 + static_cast<int>(threadIdx.x); k < L; k += kStitchThreads) {
            float cj[12], t[12];
#pragma unroll
            for (int e = 0; e < 12; ++e) {
                cj[e] = s_tot[12 * (k >> 6) + e];
                t[e] = s_t[12 * k + e];
            }
            compose(cj, t);
#pragma unroll
            for (int e = 0; e < 12; ++e) s_t[12 * k + e] = t[e];
        }
        __syncthreads();
    }

    // 3. move every tile into the chain frame
    float *out = chain + (static_cast<size_t>(c) * n_cols + gs) * n_beads * 3;
    const bool shared = lane < O;
    for (int k = wave; k < L; k += kStitchWaves) {
        const float *p = tile(k) + lane * 3;
        const float x[3] = {p[0], p[1], p[2]};
        float cur[3];
        apply(s_t + 12 * k, x, cur);
        float *dst = out + (static_cast<size_t>(k) * stride + lane) * 3;
        if (k > 0 && shared) {  // mean with tile k-1's aligned copy of the same bead
            const float *q = tile(k - 1) + (stride + lane) * 3;
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
                         float *resid, bool proper, hipStream_t stream) {
    if (ch.chain_len > 64 * kStitchMaxChunks) return hipErrorInvalidValue;
    const int64_t blocks = static_cast<int64_t>(n_chains) * G * S;
    const size_t lds = static_cast<size_t>(ch.chain_len + kStitchMaxChunks) * 12 * sizeof(float);
    return launch_slices(blocks, kStitchThreads, [&](int64_t first, uint32_t count) {
        if (proper)
            hipLaunchKernelGGL(k_stitch<true>, dim3(count), dim3(kStitchThreads), lds, stream, coords, G, S, ch, chain,
                               resid, first);
        else
            hipLaunchKernelGGL(k_stitch<false>, dim3(count), dim3(kStitchThreads), lds, stream, coords, G, S, ch,
                               chain, resid, first);
    });
}

}  // namespace pc
